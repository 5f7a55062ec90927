// Prompt processing as dense GEMMs on the matrix cores (MFMA), for the
// positions before the last prompt token: the work of a prompt of P tokens is
// a [P x d] x [d x N] product per projection, which is what the matrix cores
// are for (the per-token decode path stays on the dot2 vector ALU).
//
// The prompt is processed in chunks of up to kPfChunk positions, layer by
// layer, with one launch per operation on the engine's stream:
//   X = E[tokens]                                   (fp32 residual, [M][d])
//   per layer:  Xn = RMSNorm(X) * g_attn            (activation, [M][d])
//               QKV = Xn Wq^T | Xn Wk^T | Xn Wv^T   (fp32, [M][qd + 2 kvd])
//               rotary embedding of q (in place, fp32) and k; k, v appended
//               to the KV cache
//               A = causal attention of q over the cache rows 0 .. p0+m
//               X += A Wo^T
//               Xn = RMSNorm(X) * g_ffn
//               H = silu(Xn Wg^T) * (Xn Wu^T)       (activation, [M][F])
//               X += H Wd^T
// The last prompt position then runs through the persistent decode kernel as
// one forced step, which appends its KV row and yields the LM-head logits and
// the first token (kie_prefill in kie_runtime.hip).
//
// Activations: fp16 models store them as fp16, the matrix cores' input.  bf16
// models store them as fp32 and the GEMMs split each value into three bf16
// terms (b0 = bf16(x), b1 = bf16(x - b0), b2 = bf16(x - b0 - b1)), one product
// per term against the exact bf16 weights: fp32-accurate activations, as the
// decode path's bf16 GEMVs take them.  Attention splits the scaled queries
// and the softmax probabilities into two bf16 terms likewise.
//
// Matrix-core layout (v_mfma_f32_32x32x16_{f16,bf16}, checked on the device):
// lane l holds A[m = l%32][k = 8*(l/32) + 0..7] and B[k = 8*(l/32) + 0..7][n =
// l%32]; accumulator element 4i+j is C[m = 8i + 4*(l/32) + j][n = l%32].
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <cstdio>
#include <cstdlib>
#include <type_traits>

#include "kie.h"
#include "kie_params.hpp"
#include "kie_prefill.hpp"

namespace kie {
namespace {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef __bf16 b8_t __attribute__((ext_vector_type(8)));
typedef float f16x_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float h2f(uint16_t u) { return (float)__builtin_bit_cast(_Float16, u); }
__device__ __forceinline__ uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }
__device__ __forceinline__ float bf2f(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }  // nearest even

// 16-bit storage format of the engine dtype
template <int DT>
__device__ __forceinline__ float to_f(uint16_t u) {
  return DT == KIE_BF16 ? bf2f(u) : h2f(u);
}
template <int DT>
__device__ __forceinline__ uint16_t from_f(float f) {
  return DT == KIE_BF16 ? f2bf(f) : f2h(f);
}

// Activation element between the prompt-path kernels: fp16 (fp16 models) or
// fp32 (bf16 models, split into bf16 terms where a GEMM stages it).
template <int DT>
using act_t = typename std::conditional<DT == KIE_BF16, float, uint16_t>::type;
template <int DT>
constexpr int kTerms = DT == KIE_BF16 ? 3 : 1;  // A-operand terms per GEMM product
template <int DT>
__device__ __forceinline__ act_t<DT> to_act(float v) {
  if constexpr (DT == KIE_BF16)
    return v;
  else
    return f2h(v);
}

// One 32x32x16 matrix-core product in the engine dtype; operands are 8 16-bit
// values per lane.
template <int DT>
__device__ __forceinline__ f16x_t mma(uint4 a, uint4 b, f16x_t c) {
  if constexpr (DT == KIE_BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(b8_t, a), __builtin_bit_cast(b8_t, b), c, 0,
                                                    0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8_t, a), __builtin_bit_cast(h8_t, b), c, 0,
                                                   0, 0);
}

// x -> bf16 terms: term t of the split b0 = bf16(x), b1 = bf16(x - b0), ...
// packed two per word (element 2e in the low half).
template <int T>
__device__ __forceinline__ void split_pair(float x0, float x1, uint32_t (&w)[T]) {
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const uint16_t b0 = f2bf(x0), b1 = f2bf(x1);
    w[t] = (uint32_t)b0 | ((uint32_t)b1 << 16);
    x0 -= bf2f(b0);
    x1 -= bf2f(b1);
  }
}

// ---- embedding and RMSNorm -------------------------------------------------

template <int DT>
__global__ __launch_bounds__(256) void pf_embed(const uint16_t* E, const int* tok, int M, int d, float* X) {
  const int m = blockIdx.x;
  if (m >= M) return;
  const uint16_t* row = E + (size_t)tok[m] * d;
  for (int i = threadIdx.x; i < d; i += 256) X[(size_t)m * d + i] = to_f<DT>(row[i]);
}

// Xn[n .. n+3] = v * r * g[n .. n+3] as activations (one 8- or 16-byte store).
template <int DT>
__device__ __forceinline__ void norm_store4(act_t<DT>* xn, const uint16_t* g, float4 v, float r) {
  const uint2 gw = *reinterpret_cast<const uint2*>(g);
  const float g0 = to_f<DT>((uint16_t)gw.x), g1 = to_f<DT>((uint16_t)(gw.x >> 16));
  const float g2 = to_f<DT>((uint16_t)gw.y), g3 = to_f<DT>((uint16_t)(gw.y >> 16));
  if constexpr (DT == KIE_BF16) {
    *reinterpret_cast<float4*>(xn) = make_float4(v.x * r * g0, v.y * r * g1, v.z * r * g2, v.w * r * g3);
  } else {
    *reinterpret_cast<uint2*>(xn) = make_uint2((uint32_t)f2h(v.x * r * g0) | ((uint32_t)f2h(v.y * r * g1) << 16),
                                               (uint32_t)f2h(v.z * r * g2) | ((uint32_t)f2h(v.w * r * g3) << 16));
  }
}

// One work-group per row: the row (d <= 4096, a multiple of 128) in float4
// pieces, 4 consecutive columns per thread and pass, kept in registers between
// the sum of squares and the scaled store.
template <int DT>
__global__ __launch_bounds__(256) void pf_rmsnorm(const float* X, const uint16_t* g, float eps, int M, int d,
                                                  act_t<DT>* Xn) {
  __shared__ float part[4];
  const int m = blockIdx.x;
  if (m >= M) return;
  float4 v[4];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = 4 * (int)threadIdx.x + 1024 * j;
    if (n >= d) continue;
    v[j] = *reinterpret_cast<const float4*>(X + (size_t)m * d + n);
    ss += v[j].x * v[j].x + v[j].y * v[j].y + v[j].z * v[j].z + v[j].w * v[j].w;
  }
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float r = 1.0f / sqrtf((part[0] + part[1] + part[2] + part[3]) / (float)d + eps);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = 4 * (int)threadIdx.x + 1024 * j;
    if (n < d) norm_store4<DT>(Xn + (size_t)m * d + n, g + n, v[j], r);
  }
}

// ---- GEMM: C[M][N] = A[M][K] W[N][K]^T on the matrix cores --------------------
//
// Work-group (4 waves) tile 128 x 128, k-tiles of 64 (fp16) or 32 (bf16)
// staged in LDS (row-major, rows padded to 144 or 80 bytes so that the
// 16-byte operand reads of 16 lanes hit distinct banks), double-buffered with
// one barrier per k-tile; the next
// k-tile's global loads are in flight during the current one's products.
// Wave (wm, wn) computes rows 64wm .. and columns 64wn .. as 2 x 2
// accumulators of 32 x 32.  Both operands are k-contiguous in memory and in
// LDS, so every lane reads its 8 consecutive k values with one 16-byte load.
// bf16: A arrives in fp32 and is split into kTerms bf16 planes while staged;
// each product runs once per plane, the smallest first.
//   EPI_STORE / EPI_ADD: W is up to three matrices stacked along N (the
//   column tile picks one; segment widths are multiples of 128).
//   EPI_SWIGLU: a work-group tile covers 64 output columns; its B rows are 64
//   rows of the gate matrix then the same 64 rows of the up matrix, and wave
//   (wm, wn) takes gate columns 32wn .. and the matching up columns, so gate
//   and up of one output land in the same lane: H = silu(gate) * up.
// Rows of A beyond M re-read row M-1 and are not stored.  K % 64 == 0.
// 72 KB of LDS per work-group (fp16: two per CU), 80 KB (bf16, three A term
// planes: two per CU).
enum : int { EPI_STORE = 0, EPI_ADD = 1, EPI_SWIGLU = 2, EPI_PART = 3 };
constexpr int kTM = 128, kTN = 128;
template <int DT>
constexpr int kBK = DT == KIE_BF16 ? 32 : 64;  // k-tile width (measured best per dtype)
template <int DT>
constexpr int kLS = kBK<DT> + 8;  // LDS row stride in halves (144 or 80 bytes)
template <int DT>
constexpr int kTile = kTM * kLS<DT>;  // halves per operand tile
template <int DT>
constexpr int kPPR = kBK<DT> / 8;  // 8-element pieces per tile row
template <int DT>
constexpr int kRPP = 256 / kPPR<DT>;  // tile rows staged per pass
template <int DT>
constexpr int kPasses = kTM / kRPP<DT>;  // passes per operand tile (4 or 2)
constexpr int kBKMax = 64;                // every supported reduction width is a multiple of this

struct GemmB {
  const uint16_t* w[3];  // stacked matrices ([rows][K] each); EPI_SWIGLU: gate, up
  int end[3];            // cumulative row counts
};

// Write one staged A piece (8 elements: v0, and v1 for fp32) to LDS: fp16 as
// is; fp32 as kTerms bf16 planes of kTile halves each.
template <int DT>
__device__ __forceinline__ void stage_a(uint4 v0, uint4 v1, uint16_t* dst) {
  if constexpr (DT == KIE_BF16) {
    const float x[8] = {__uint_as_float(v0.x), __uint_as_float(v0.y), __uint_as_float(v0.z), __uint_as_float(v0.w),
                        __uint_as_float(v1.x), __uint_as_float(v1.y), __uint_as_float(v1.z), __uint_as_float(v1.w)};
    uint32_t w[4][kTerms<DT>];
#pragma unroll
    for (int e = 0; e < 4; ++e) split_pair<kTerms<DT>>(x[2 * e], x[2 * e + 1], w[e]);
#pragma unroll
    for (int t = 0; t < kTerms<DT>; ++t)
      *reinterpret_cast<uint4*>(dst + t * kTile<DT>) = make_uint4(w[0][t], w[1][t], w[2][t], w[3][t]);
  } else {
    *reinterpret_cast<uint4*>(dst) = v0;
  }
}

template <int EPI, int DT>
__global__ __launch_bounds__(256, 2) void pf_gemm(const act_t<DT>* A, int M, int K, GemmB wb,
                                                                        float* C, int ldc, act_t<DT>* H, int ldh) {
  constexpr int NT = kTerms<DT>;
  constexpr int BK = kBK<DT>, LS = kLS<DT>, TILE = kTile<DT>, PPR = kPPR<DT>, RPP = kRPP<DT>, PASSES = kPasses<DT>;
  constexpr int kBuf = (NT + 1) * TILE;  // halves per buffer: NT A planes, then B
  __shared__ __align__(16) uint16_t lds[2][kBuf];
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63, r = l & 31, hf = l >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * kTM;
  // B rows of this tile: 128 consecutive rows of one stacked matrix, or 64 gate + 64 up rows
  const uint16_t* b_lo;
  const uint16_t* b_hi;
  int n0;
  if constexpr (EPI == EPI_SWIGLU) {
    n0 = blockIdx.x * 64;
    b_lo = wb.w[0] + (size_t)n0 * K;
    b_hi = wb.w[1] + (size_t)n0 * K;
  } else {
    n0 = blockIdx.x * kTN;
    const bool s0 = n0 < wb.end[0], s1 = n0 < wb.end[1];  // selects, not an indexed argument (no scratch copy)
    const uint16_t* wsel = s0 ? wb.w[0] : s1 ? wb.w[1] : wb.w[2];
    b_lo = wsel + (size_t)(n0 - (s0 ? 0 : s1 ? wb.end[0] : wb.end[1])) * K;
    b_hi = b_lo + (size_t)64 * K;
  }
  // staging: thread t moves 8-element piece t%8 of rows t/8 + 32i (i = 0..3) of both tiles
  const int pc = tid % PPR, pr = tid / PPR;
  const act_t<DT>* ag[4];
  const uint16_t* bg[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = pr + RPP * (i % PASSES);
    ag[i] = A + (size_t)min(m0 + row, M - 1) * K + 8 * pc;
    bg[i] = (row < 64 ? b_lo + (size_t)row * K : b_hi + (size_t)(row - 64) * K) + 8 * pc;
  }
  // operand rows read by this lane: A rows 64wm + 32i + r; B rows per column block j
  const int arow0 = 64 * wm + r;
  const int brow0 = EPI == EPI_SWIGLU ? 32 * wn + r : 64 * wn + r;
  const int bstep = EPI == EPI_SWIGLU ? 64 : 32;  // B row offset of column block 1 (up rows for SwiGLU)
  const int soff = pr * LS + 8 * pc;              // this thread's staging offset (row pr, piece pc)
  f16x_t acc[2][2] = {};
  // split-K (EPI_PART): slice z of gridDim.z takes k-tiles [kt0, kt0 + nk) and
  // writes its partial product to C + z * M * ldc; otherwise one slice
  const int nk_all = K / BK;
  const int kt0 = (int)((long)nk_all * blockIdx.z / gridDim.z);
  const int nk = (int)((long)nk_all * (blockIdx.z + 1) / gridDim.z) - kt0;
  if constexpr (EPI == EPI_PART) C += (size_t)blockIdx.z * M * ldc;
  constexpr bool F32A = DT == KIE_BF16;  // fp32 A pieces: two 16-byte vectors each
  uint4 a00, a01, a10, a11, a20, a21, a30, a31, rb0, rb1, rb2, rb3;
  a01 = a11 = a21 = a31 = make_uint4(0, 0, 0, 0);
#define KIE_PF_LDA(i, k0, v) reinterpret_cast<const uint4*>(ag[i] + (k0))[v]
#define KIE_PF_FETCH(k0)                                    \
  do {                                                      \
    a00 = KIE_PF_LDA(0, k0, 0);                             \
    a10 = KIE_PF_LDA(1, k0, 0);                             \
    if constexpr (F32A) {                                   \
      a01 = KIE_PF_LDA(0, k0, 1);                           \
      a11 = KIE_PF_LDA(1, k0, 1);                           \
    }                                                       \
    rb0 = *reinterpret_cast<const uint4*>(bg[0] + (k0));    \
    rb1 = *reinterpret_cast<const uint4*>(bg[1] + (k0));    \
    if constexpr (PASSES > 2) {                            \
      a20 = KIE_PF_LDA(2, k0, 0);                           \
      a30 = KIE_PF_LDA(3, k0, 0);                           \
      if constexpr (F32A) {                                 \
        a21 = KIE_PF_LDA(2, k0, 1);                         \
        a31 = KIE_PF_LDA(3, k0, 1);                         \
      }                                                     \
      rb2 = *reinterpret_cast<const uint4*>(bg[2] + (k0));  \
      rb3 = *reinterpret_cast<const uint4*>(bg[3] + (k0));  \
    }                                                       \
  } while (0)
#define KIE_PF_STAGE(buf)                                   \
  do {                                                      \
    uint16_t* sa = &lds[buf][soff];                         \
    stage_a<DT>(a00, a01, sa);                              \
    stage_a<DT>(a10, a11, sa + RPP * LS);                 \
    if constexpr (PASSES > 2) {                            \
      stage_a<DT>(a20, a21, sa + 2 * RPP * LS);           \
      stage_a<DT>(a30, a31, sa + 3 * RPP * LS);           \
    }                                                       \
    uint16_t* sb = sa + NT * TILE;                         \
    *reinterpret_cast<uint4*>(sb) = rb0;                    \
    *reinterpret_cast<uint4*>(sb + RPP * LS) = rb1;       \
    if constexpr (PASSES > 2) {                            \
      *reinterpret_cast<uint4*>(sb + 2 * RPP * LS) = rb2; \
      *reinterpret_cast<uint4*>(sb + 3 * RPP * LS) = rb3; \
    }                                                       \
  } while (0)
  KIE_PF_FETCH(kt0 * BK);
  KIE_PF_STAGE(0);
  __syncthreads();
  for (int t = 0; t < nk; ++t) {
    if (t + 1 < nk) KIE_PF_FETCH((kt0 + t + 1) * BK);
    const uint16_t* la = lds[t & 1];
    const uint16_t* lb = la + NT * TILE;
    // every operand of the k-tile is read before the first product, so the
    // LDS latency is paid once per tile
    constexpr int KS = BK / 16;
    uint4 ob[KS][2], oa[KS][NT][2];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int ko = 16 * kk + 8 * hf;
      ob[kk][0] = *reinterpret_cast<const uint4*>(lb + brow0 * LS + ko);
      ob[kk][1] = *reinterpret_cast<const uint4*>(lb + (brow0 + bstep) * LS + ko);
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        const uint16_t* lt = la + tt * TILE;
        oa[kk][tt][0] = *reinterpret_cast<const uint4*>(lt + arow0 * LS + ko);
        oa[kk][tt][1] = *reinterpret_cast<const uint4*>(lt + (arow0 + 32) * LS + ko);
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the products
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
#pragma unroll
      for (int tt = NT - 1; tt >= 0; --tt) {
        acc[0][0] = mma<DT>(oa[kk][tt][0], ob[kk][0], acc[0][0]);
        acc[0][1] = mma<DT>(oa[kk][tt][0], ob[kk][1], acc[0][1]);
        acc[1][0] = mma<DT>(oa[kk][tt][1], ob[kk][0], acc[1][0]);
        acc[1][1] = mma<DT>(oa[kk][tt][1], ob[kk][1], acc[1][1]);
      }
    if (t + 1 < nk) KIE_PF_STAGE((t + 1) & 1);
    __syncthreads();
  }
#undef KIE_PF_LDA
#undef KIE_PF_FETCH
#undef KIE_PF_STAGE
  // accumulator element 4ii + jj of acc[i][j]: row 64wm + 32i + 8ii + 4hf + jj, column block j, column r
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int m = m0 + 64 * wm + 32 * i + 8 * ii + 4 * hf + jj;
        if (m >= M) continue;
        const int e = 4 * ii + jj;
        if constexpr (EPI == EPI_SWIGLU) {
          const float gt = acc[i][0][e], up = acc[i][1][e];
          H[(size_t)m * ldh + n0 + 32 * wn + r] = to_act<DT>(gt / (1.0f + expf(-gt)) * up);
        } else {
          float* cp = C + (size_t)m * ldc + n0 + 64 * wn + r;
          if constexpr (EPI == EPI_ADD) {
            cp[0] += acc[i][0][e];
            cp[32] += acc[i][1][e];
          } else {  // EPI_STORE, EPI_PART
            cp[0] = acc[i][0][e];
            cp[32] = acc[i][1][e];
          }
        }
      }
}

// ---- GEMMs for long prompts (fp16) -------------------------------------------
//
// The three GEMM forms on 256 x 256 work-group tiles, 8 waves (512 threads, one
// work-group per CU: 144 KB of LDS).  Wave (wm, wn), wm < 2, wn < 4, computes
// rows 128wm .. 128wm+127 of the tile against two 32-row blocks of its B rows:
// 4 x 2 accumulators of 32 x 32, so each 16-byte LDS operand read feeds 1.33
// matrix-core products (the 128 x 128 tile's 64 x 64 wave blocks: 1).
//   EPI_STORE / EPI_ADD: 256 consecutive rows of one stacked matrix (segment
//   widths multiples of 256); wave wn takes B rows 64wn .. 64wn+63.
//   EPI_SWIGLU: 128 gate rows, then the same 128 up rows, for 128 output
//   columns; wave wn takes gate rows 32wn .. and the matching up rows, so gate
//   and up of one output land in the same lane.
// k-tiles of 64, rows padded to 144 bytes, double-buffered, one barrier per
// k-tile; the next k-tile's LDS writes are spread over the current one's
// products, a quarter after each 16-deep k step, and each quarter's registers
// are then refilled from the k-tile after that, so a global load has a whole
// k-tile of products to land.  Rows of A beyond M
// re-read row M-1 and are not stored.  Used when the grid fills the chip
// (big_tiles_pay); the 128 x 128 kernel covers the rest.
typedef uint32_t v4u_t __attribute__((ext_vector_type(4)));  // staging registers the compiler keeps in VGPRs
constexpr int kBigT = 256;                                     // tile rows of A and of B

template <int EPI>
__global__ __launch_bounds__(512, 1) void pf_gemm_big(const uint16_t* A, int M, int K, GemmB wb, float* C, int ldc,
                                                     uint16_t* H, int ldh) {
  constexpr int BK = 64, LS = 72, NT = 512, RPP = NT / 8, PA = kBigT / RPP, PB = kBigT / RPP, BI = 4;
  static_assert(PA == BK / 16 && PB == BK / 16, "one staging piece of A and of B per k step");
  constexpr bool SWI = EPI == EPI_SWIGLU;
  __shared__ __align__(16) uint16_t lds[2][2 * kBigT * LS];
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63, r = l & 31, hf = l >> 5;
  const int wm = wave >> 2, wn = wave & 3;
  const int m0 = blockIdx.y * kBigT, n0 = blockIdx.x * (SWI ? kBigT / 2 : kBigT);
  const int pc = tid & 7, pr = tid >> 3;  // staging: piece pc of rows pr + 64i
  const uint16_t* ag[PA];
  const uint16_t* bg[PB];
#pragma unroll
  for (int i = 0; i < PA; ++i) ag[i] = A + (size_t)min(m0 + pr + RPP * i, M - 1) * K + 8 * pc;
  if constexpr (SWI) {
#pragma unroll
    for (int i = 0; i < PB; ++i)  // B rows 0..127 gate, 128..255 up
      bg[i] = (i < PB / 2 ? wb.w[0] : wb.w[1]) + (size_t)(n0 + pr + RPP * (i % (PB / 2))) * K + 8 * pc;
  } else {
    const bool s0 = n0 < wb.end[0], s1 = n0 < wb.end[1];  // selects, not an indexed argument
    const uint16_t* wsel = s0 ? wb.w[0] : s1 ? wb.w[1] : wb.w[2];
    const uint16_t* b0 = wsel + (size_t)(n0 - (s0 ? 0 : s1 ? wb.end[0] : wb.end[1])) * K;
#pragma unroll
    for (int i = 0; i < PB; ++i) bg[i] = b0 + (size_t)(pr + RPP * i) * K + 8 * pc;
  }
  const int soff = pr * LS + 8 * pc;
  const int arow = 128 * wm + r;
  const int brow0 = SWI ? 32 * wn + r : 64 * wn + r, bstep = SWI ? 128 : 32;  // B rows of blocks 0 and 1
  f16x_t acc[BI][2];
#pragma unroll
  for (int i = 0; i < BI; ++i) acc[i][0] = acc[i][1] = f16x_t{};
  v4u_t sa[PA], sb[PB];
  const int nk = K / BK;
  auto fetch = [&](int k0, int i) {  // staging piece i of A and of B from global memory
    sa[i] = *reinterpret_cast<const v4u_t*>(ag[i] + k0);
    sb[i] = *reinterpret_cast<const v4u_t*>(bg[i] + k0);
  };
  auto stage = [&](uint16_t* d, int i) {  // staging piece i of A and of B into LDS
    *reinterpret_cast<v4u_t*>(&d[soff + RPP * i * LS]) = sa[i];
    *reinterpret_cast<v4u_t*>(&d[kBigT * LS + soff + RPP * i * LS]) = sb[i];
  };
  // The refills and LDS writes run on every k-tile, the k offset clamped to the
  // last tile (repeated loads of it, written to the buffer no later tile
  // reads): without branches around them the compiler waits for each piece's
  // own loads, not for all loads in flight.
#pragma unroll
  for (int i = 0; i < PA; ++i) fetch(0, i);
#pragma unroll
  for (int i = 0; i < PA; ++i) stage(lds[0], i);
#pragma unroll
  for (int i = 0; i < PA; ++i) {  // in piece order, as the loop issues them
    fetch(min(1, nk - 1) * BK, i);
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();
  for (int t = 0; t < nk; ++t) {
    const uint16_t* la = lds[t & 1];
    const uint16_t* lb = la + kBigT * LS;
    // per 16-deep k step: read its operands, run its 8 products, then write one
    // quarter of the next k-tile into the other buffer (last read before the
    // previous barrier), so the LDS writes spread over the tile's products,
    // and refill the freed registers with the same quarter of the k-tile after
    // that: every global load has a whole k-tile of products to land in
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int ko = 16 * kk + 8 * hf;
      v4u_t oa[BI], ob[2];
#pragma unroll
      for (int i = 0; i < BI; ++i) oa[i] = *reinterpret_cast<const v4u_t*>(la + (arow + 32 * i) * LS + ko);
      ob[0] = *reinterpret_cast<const v4u_t*>(lb + brow0 * LS + ko);
      ob[1] = *reinterpret_cast<const v4u_t*>(lb + (brow0 + bstep) * LS + ko);
      __builtin_amdgcn_sched_barrier(0);  // keep the step's reads ahead of its products
#pragma unroll
      for (int i = 0; i < BI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8_t, oa[i]),
                                                             __builtin_bit_cast(h8_t, ob[j]), acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      stage(lds[(t + 1) & 1], kk);
      fetch(min(t + 2, nk - 1) * BK, kk);
    }
    __syncthreads();
  }
  // accumulator element 4ii + jj of acc[i][j]: row 128wm + 32i + 8ii + 4hf + jj; column: SwiGLU 32wn + r
  // (gate j = 0, up j = 1), otherwise 64wn + 32j + r
#pragma unroll
  for (int i = 0; i < BI; ++i)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int m = m0 + 128 * wm + 32 * i + 8 * ii + 4 * hf + jj;
        if (m >= M) continue;
        const int e = 4 * ii + jj;
        if constexpr (SWI) {
          const float gt = acc[i][0][e], up = acc[i][1][e];
          H[(size_t)m * ldh + n0 + 32 * wn + r] = f2h(gt / (1.0f + expf(-gt)) * up);
        } else {
          float* cp = C + (size_t)m * ldc + n0 + 64 * wn + r;
          if constexpr (EPI == EPI_ADD) {
            cp[0] += acc[i][0][e];
            cp[32] += acc[i][1][e];
          } else {
            cp[0] = acc[i][0][e];
            cp[32] = acc[i][1][e];
          }
        }
      }
}

// Whether the 256 x 256 kernel pays for an output of M rows and `cols` tile
// columns: one full round of work-groups (one per CU of the 256) for the store
// and add forms, two for gate/up + SwiGLU (measured: 128 x 128 tiles win on
// smaller grids).
__host__ __device__ constexpr bool big_tiles_pay(int M, int cols, bool swiglu) {
  return cols * ((M + kBigT - 1) / kBigT) >= (swiglu ? 512 : 256);
}

// Split-K reduction: C[m][n] (+)= sum over z = 0 .. S-1 of P[z][m][n], the
// slices added in order (deterministic).  Four columns per thread; N % 4 == 0.
template <bool ADD>
__global__ __launch_bounds__(256) void pf_splitk(const float* P, int S, int M, int N, float* C, int ldc) {
  const int q = blockIdx.x * 256 + threadIdx.x, nq = N >> 2;
  if (q >= M * nq) return;
  const int m = q / nq, n = (q % nq) * 4;
  float4 a = *reinterpret_cast<const float4*>(P + (size_t)m * N + n);
  for (int z = 1; z < S; ++z) {
    const float4 b = *reinterpret_cast<const float4*>(P + ((size_t)z * M + m) * N + n);
    a.x += b.x;
    a.y += b.y;
    a.z += b.z;
    a.w += b.w;
  }
  float4* c = reinterpret_cast<float4*>(C + (size_t)m * ldc + n);
  if (ADD) {
    const float4 o = *c;
    a.x += o.x;
    a.y += o.y;
    a.z += o.z;
    a.w += o.w;
  }
  *c = a;
}

// Split-K reduction into the residual, fused with the RMSNorm that consumes
// it: one work-group per row m; X[m] += sum over z = 0 .. S-1 of P[z][m]
// (slices added in order, then the residual, as pf_splitk), then Xn[m] =
// RMSNorm(X[m]) * g.  Each thread keeps its 4-column groups of the row (at
// most 16 values: d <= 4096) in registers between the two steps.
template <int DT>
__global__ __launch_bounds__(256) void pf_splitk_norm(const float* P, int S, int M, int d, float* X,
                                                      const uint16_t* g, float eps, act_t<DT>* Xn) {
  __shared__ float part[4];
  const int m = blockIdx.x;
  if (m >= M) return;
  float4 v[4];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = 4 * (int)threadIdx.x + 1024 * j;
    if (n >= d) continue;
    float4 a = *reinterpret_cast<const float4*>(P + (size_t)m * d + n);
    for (int z = 1; z < S; ++z) {
      const float4 b = *reinterpret_cast<const float4*>(P + ((size_t)z * M + m) * d + n);
      a.x += b.x;
      a.y += b.y;
      a.z += b.z;
      a.w += b.w;
    }
    float4* xp = reinterpret_cast<float4*>(X + (size_t)m * d + n);
    const float4 o = *xp;
    a.x += o.x;
    a.y += o.y;
    a.z += o.z;
    a.w += o.w;
    *xp = a;
    v[j] = a;
    ss += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w;
  }
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float r = 1.0f / sqrtf((part[0] + part[1] + part[2] + part[3]) / (float)d + eps);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = 4 * (int)threadIdx.x + 1024 * j;
    if (n < d) norm_store4<DT>(Xn + (size_t)m * d + n, g + n, v[j], r);
  }
}

// ---- rotary embedding, KV append ------------------------------------------
//
// Thread (m, i) for rotary pairs i .. i+3 (i a multiple of 4, < hd/2) of every
// head: q rotated in place (fp32, as the decode path keeps it); k rotated and
// v copied into the cache rows at position p0 + m.  16-byte loads of the
// fp32 rows and of the (cos, sin) table, 8-byte stores into the cache.
template <int DT>
__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
  return make_uint2((uint32_t)from_f<DT>(a) | ((uint32_t)from_f<DT>(b) << 16),
                    (uint32_t)from_f<DT>(c) | ((uint32_t)from_f<DT>(d) << 16));
}

template <int DT>
__global__ __launch_bounds__(256) void pf_rope_kv(float* QKV, int M, int hq, int hkv, int hd, const float* rope,
                                                  int p0, int max_seq, uint16_t* kc, uint16_t* vc) {
  const int half = hd >> 1, qd = hq * hd, kvd = hkv * hd, ld = qd + 2 * kvd;
  const int per_row = ((hq + hkv) * half + hkv * half) / 4;  // groups of 4 q, k and v pairs
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= M * per_row) return;
  const int m = idx / per_row, r = 4 * (idx % per_row), pos = p0 + m;
  float* row = QKV + (size_t)m * ld;
  if (r < (hq + hkv) * half) {
    const int h = r / half, i = r % half;
    const float4 cs0 = *reinterpret_cast<const float4*>(rope + ((size_t)pos * half + i) * 2);
    const float4 cs1 = *reinterpret_cast<const float4*>(rope + ((size_t)pos * half + i) * 2 + 4);
    float* src = row + (size_t)h * hd;  // q heads, then k heads (contiguous)
    const float4 a = *reinterpret_cast<const float4*>(src + i), b = *reinterpret_cast<const float4*>(src + i + half);
    const float4 ra = make_float4(a.x * cs0.x - b.x * cs0.y, a.y * cs0.z - b.y * cs0.w, a.z * cs1.x - b.z * cs1.y,
                                  a.w * cs1.z - b.w * cs1.w);
    const float4 rb = make_float4(a.x * cs0.y + b.x * cs0.x, a.y * cs0.w + b.y * cs0.z, a.z * cs1.y + b.z * cs1.x,
                                  a.w * cs1.w + b.w * cs1.z);
    if (h < hq) {
      *reinterpret_cast<float4*>(src + i) = ra;
      *reinterpret_cast<float4*>(src + i + half) = rb;
    } else {
      uint16_t* dst = kc + ((size_t)(h - hq) * max_seq + pos) * hd;
      *reinterpret_cast<uint2*>(dst + i) = pack4<DT>(ra.x, ra.y, ra.z, ra.w);
      *reinterpret_cast<uint2*>(dst + i + half) = pack4<DT>(rb.x, rb.y, rb.z, rb.w);
    }
  } else {
    const int rr = r - (hq + hkv) * half, g = rr / half, i = rr % half;
    const float* src = row + qd + kvd + (size_t)g * hd;
    uint16_t* dst = vc + ((size_t)g * max_seq + pos) * hd;
    const float4 a = *reinterpret_cast<const float4*>(src + i), b = *reinterpret_cast<const float4*>(src + i + half);
    *reinterpret_cast<uint2*>(dst + i) = pack4<DT>(a.x, a.y, a.z, a.w);
    *reinterpret_cast<uint2*>(dst + i + half) = pack4<DT>(b.x, b.y, b.z, b.w);
  }
}

// ---- causal attention on the matrix cores ------------------------------------
//
// Flash attention over the cache rows 0 .. p0+m of query m.  A work-group (4
// waves) takes one block of query rows and one KV head g with up to four of
// its query heads: HW = min(G, 4) heads and 4/HW sub-blocks of 32 rows, wave w
// on head hb + w%HW and sub-block w/HW.  Per tile of 32 cache rows the
// work-group stages K row-major and V transposed ([dimension][row]) in LDS,
// double-buffered with one barrier per tile, the next tile's loads in flight
// during the current tile's products.  Each wave then
//   - forms S^T = K Q^T (32 rows x 32 queries) on the matrix cores, so that
//     lane l owns query l%32 and 16 of the 32 rows (8i + 4(l/32) + j);
//   - takes the online softmax in base 2 (scores pre-scaled by log2(e)/sqrt(hd)),
//     the running maximum shared with lane l^32, the running sum per lane;
//   - accumulates O^T += V^T P^T: P's fp16 values are already in the B-operand
//     layout, with operand row 8(l/32) + s holding cache row
//     16c + 8(s/4) + 4(l/32) + s%4 for product c = 0, 1 of the tile, and V^T is
//     read from LDS in that same row order.
// Rows past the work-group's last key re-read that key (finite values, masked).
// On large grids a work-group takes two query blocks in turn, the longest and
// the shortest key range of a pair, so causal work is even across
// work-groups; smaller grids keep one block per work-group (pairing would
// leave compute units idle).
template <int HD, int DT>
__global__ __launch_bounds__(256, 2) void pf_attn(const float* QKV, int M, int hq, int hkv, int p0, int max_seq,
                                               const uint16_t* kc, const uint16_t* vc, act_t<DT>* Aout, int pair) {
  constexpr int KS = HD + 8;  // K tile row stride (halves): 16-byte aligned rows, 4-bank skew
  constexpr int VS = 36;      // V^T tile row stride (halves): 8-byte reads of 32 rows hit distinct banks
  constexpr int KT = 32 * KS, VT = HD * VS, NO = HD / 32, NK = HD / 16;
  constexpr int CPR = HD / 8;  // 16-byte pieces per cache row
  __shared__ __align__(16) uint16_t lds[2 * (KT + VT)];
  const int G = hq / hkv, HW = G < 4 ? G : 4, QB = 4 / HW, sets = G / HW;
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63, r = l & 31, hf = l >> 5;
  const int rows = 32 * QB, nqb = (M + rows - 1) / rows;
  // work-group b takes query block nqb-1-b (the longest key range first);
  // with `pair`, then block b (the shortest): every work-group streams about
  // the same number of key tiles, so one round of work-groups ends together
  for (int pass = 0; pass < 2; ++pass) {
    const int qb = pass == 0 ? nqb - 1 - (int)blockIdx.x : (int)blockIdx.x;
    if (pass == 1 && (!pair || qb >= nqb - 1 - (int)blockIdx.x)) break;  // an odd count's middle block runs once
    const int g = (int)blockIdx.y / sets, h = g * G + ((int)blockIdx.y % sets) * HW + wave % HW;
    const int mq0 = qb * rows + (wave / HW) * 32;
    const int nkeys = p0 + min((qb + 1) * rows, M), nt = (nkeys + 31) / 32;
    const int qd = hq * HD, ldq = qd + 2 * hkv * HD;

    // this lane's query, scaled for base-2 exponentials, as B operands (bf16:
    // QT terms of the split, each a product of its own)
    constexpr int QT = DT == KIE_BF16 ? 2 : 1;
    const float scale = 1.4426950408889634f / sqrtf((float)HD);
    uint4 qf[QT][NK];
    {
      const float* qp = QKV + (size_t)min(mq0 + r, M - 1) * ldq + (size_t)h * HD + 8 * hf;
  #pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const float4 a = *reinterpret_cast<const float4*>(qp + 16 * kk);
        const float4 b = *reinterpret_cast<const float4*>(qp + 16 * kk + 4);
        const float x[8] = {a.x * scale, a.y * scale, a.z * scale, a.w * scale,
                            b.x * scale, b.y * scale, b.z * scale, b.w * scale};
        if constexpr (DT == KIE_BF16) {
          uint32_t w[4][QT];
  #pragma unroll
          for (int e = 0; e < 4; ++e) split_pair<QT>(x[2 * e], x[2 * e + 1], w[e]);
  #pragma unroll
          for (int t = 0; t < QT; ++t) qf[t][kk] = make_uint4(w[0][t], w[1][t], w[2][t], w[3][t]);
        } else {
          qf[0][kk] = __builtin_bit_cast(uint4, h8_t{(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3],
                                                     (_Float16)x[4], (_Float16)x[5], (_Float16)x[6], (_Float16)x[7]});
        }
      }
    }

    // tile staging.  K: thread t moves 16-byte piece t%CPR of cache rows
    // 2(t/CPR), +1 (a wave's row-major writes cover consecutive banks).  V:
    // thread t moves piece t/16 of rows 2(t%16), +1, so that the 16 lanes of a
    // piece write the transposed words of 16 consecutive row pairs, 64 lanes
    // spanning all banks.
    const int tid = threadIdx.x, pe = tid % CPR, pr = tid / CPR, vpe = tid >> 4, vpr = tid & 15;
    const bool loader = tid < 16 * CPR;
    const uint16_t* kb = kc + (size_t)g * max_seq * HD + 8 * pe;
    const uint16_t* vb = vc + (size_t)g * max_seq * HD + 8 * vpe;
    uint4 k0r, k1r, v0r, v1r;
    auto fetch = [&](int t) {
      const int j0 = min(32 * t + 2 * pr, nkeys - 1), j1 = min(32 * t + 2 * pr + 1, nkeys - 1);
      k0r = *reinterpret_cast<const uint4*>(kb + (size_t)j0 * HD);
      k1r = *reinterpret_cast<const uint4*>(kb + (size_t)j1 * HD);
      const int i0 = min(32 * t + 2 * vpr, nkeys - 1), i1 = min(32 * t + 2 * vpr + 1, nkeys - 1);
      v0r = *reinterpret_cast<const uint4*>(vb + (size_t)i0 * HD);
      v1r = *reinterpret_cast<const uint4*>(vb + (size_t)i1 * HD);
    };
    auto stage = [&](int buf) {
      uint16_t* kt = lds + buf * (KT + VT);
      uint16_t* vt = kt + KT;
      *reinterpret_cast<uint4*>(kt + (2 * pr) * KS + 8 * pe) = k0r;
      *reinterpret_cast<uint4*>(kt + (2 * pr + 1) * KS + 8 * pe) = k1r;
      const uint32_t a[4] = {v0r.x, v0r.y, v0r.z, v0r.w}, b[4] = {v1r.x, v1r.y, v1r.z, v1r.w};
  #pragma unroll
      for (int u = 0; u < 4; ++u) {  // dimensions 8vpe+2u and 8vpe+2u+1, rows 2vpr (low half) and 2vpr+1
        *reinterpret_cast<uint32_t*>(vt + (8 * vpe + 2 * u) * VS + 2 * vpr) = (a[u] & 0xFFFFu) | (b[u] << 16);
        *reinterpret_cast<uint32_t*>(vt + (8 * vpe + 2 * u + 1) * VS + 2 * vpr) =
            (a[u] >> 16) | (b[u] & 0xFFFF0000u);
      }
    };

    f16x_t o[NO] = {};
    float mrun = -INFINITY, lrun = 0.f;
    const int qpos = p0 + mq0 + r;
    if (loader) {
      fetch(0);
      stage(0);
    }
    __syncthreads();
    for (int t = 0; t < nt; ++t) {
      if (loader && t + 1 < nt) fetch(t + 1);
      const uint16_t* kt = lds + (t & 1) * (KT + VT);
      const uint16_t* vt = kt + KT;
      f16x_t s = {};
  #pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const uint4 ka = *reinterpret_cast<const uint4*>(kt + r * KS + 16 * kk + 8 * hf);
  #pragma unroll
        for (int t = QT - 1; t >= 0; --t) s = mma<DT>(ka, qf[t][kk], s);
      }
      const int k0 = 32 * t;
      if (k0 + 31 > p0 + mq0) {  // the tile reaches past this wave's first query: causal mask
  #pragma unroll
        for (int e = 0; e < 16; ++e)
          if (k0 + 8 * (e >> 2) + 4 * hf + (e & 3) > qpos) s[e] = -INFINITY;
      }
      float tm = s[0];
  #pragma unroll
      for (int e = 1; e < 16; ++e) tm = fmaxf(tm, s[e]);
      tm = fmaxf(tm, __shfl_xor(tm, 32));
      // Lazy rescaling: the reference maximum mrun moves only when a score
      // exceeds it by more than 8 (base 2), so probabilities stay below 2^8 and
      // most tiles skip rescaling the accumulators (the first tile always moves
      // it: cache row 0 is in every query's range, so tm is finite).
      const bool grow = tm > mrun + 8.f;
      if (__any(grow)) {
        const float mn = grow ? tm : mrun;
        const float al = __builtin_amdgcn_exp2f(mrun - mn);
        lrun *= al;
  #pragma unroll
        for (int ot = 0; ot < NO; ++ot) o[ot] *= al;
        mrun = mn;
      }
      const float mn = mrun;
      float ps = 0.f;
      float pv[16];
  #pragma unroll
      for (int e = 0; e < 16; ++e) {
        pv[e] = __builtin_amdgcn_exp2f(s[e] - mn);
        ps += pv[e];
      }
      uint4 pb[QT][2];  // probabilities as B operands (bf16: QT terms)
  #pragma unroll
      for (int c = 0; c < 2; ++c) {
        if constexpr (DT == KIE_BF16) {
          uint32_t w[4][QT];
  #pragma unroll
          for (int e = 0; e < 4; ++e) split_pair<QT>(pv[8 * c + 2 * e], pv[8 * c + 2 * e + 1], w[e]);
  #pragma unroll
          for (int t = 0; t < QT; ++t) pb[t][c] = make_uint4(w[0][t], w[1][t], w[2][t], w[3][t]);
        } else {
          const float* q = pv + 8 * c;
          pb[0][c] = __builtin_bit_cast(uint4, h8_t{(_Float16)q[0], (_Float16)q[1], (_Float16)q[2], (_Float16)q[3],
                                                    (_Float16)q[4], (_Float16)q[5], (_Float16)q[6], (_Float16)q[7]});
        }
      }
      lrun += ps;
  #pragma unroll
      for (int c = 0; c < 2; ++c)
  #pragma unroll
        for (int ot = 0; ot < NO; ++ot) {
          const uint16_t* vp = vt + (32 * ot + r) * VS + 16 * c + 4 * hf;
          const uint2 lo = *reinterpret_cast<const uint2*>(vp), hi = *reinterpret_cast<const uint2*>(vp + 8);
          const uint4 a = make_uint4(lo.x, lo.y, hi.x, hi.y);
  #pragma unroll
          for (int t = QT - 1; t >= 0; --t) o[ot] = mma<DT>(a, pb[t][c], o[ot]);
        }
      if (loader && t + 1 < nt) stage((t + 1) & 1);
      __syncthreads();
    }
    const float inv = 1.0f / (lrun + __shfl_xor(lrun, 32));
    const int m = mq0 + r;
    if (m < M) {
      act_t<DT>* op = Aout + (size_t)m * qd + (size_t)h * HD + 4 * hf;
  #pragma unroll
      for (int ot = 0; ot < NO; ++ot)
  #pragma unroll
        for (int i = 0; i < 4; ++i) {  // dimensions 32ot + 8i + 4(l/32) + 0..3
          const f16x_t& v = o[ot];
          if constexpr (DT == KIE_BF16) {
            *reinterpret_cast<float4*>(op + 32 * ot + 8 * i) =
                make_float4(v[4 * i] * inv, v[4 * i + 1] * inv, v[4 * i + 2] * inv, v[4 * i + 3] * inv);
          } else {
            *reinterpret_cast<uint2*>(op + 32 * ot + 8 * i) =
                make_uint2((uint32_t)f2h(v[4 * i] * inv) | ((uint32_t)f2h(v[4 * i + 1] * inv) << 16),
                           (uint32_t)f2h(v[4 * i + 2] * inv) | ((uint32_t)f2h(v[4 * i + 3] * inv) << 16));
          }
        }
    }
  }
}

}  // namespace

bool prefill_supported(const kie_config& c) {
  const int qd = c.n_heads * c.head_dim, kvd = c.n_kv_heads * c.head_dim;
  return (c.dtype == KIE_F16 || c.dtype == KIE_BF16) && (c.head_dim == 64 || c.head_dim == 128) &&
         c.d_model % kTN == 0 && qd % kTN == 0 && kvd % kTN == 0 && c.d_ffn % kTN == 0 && c.d_model % kBKMax == 0 &&
         qd % kBKMax == 0 && c.d_ffn % kBKMax == 0;
}

size_t prefill_act_bytes(const kie_config& c) { return c.dtype == KIE_BF16 ? 4 : 2; }

size_t prefill_part_floats(const kie_config& c, int chunk) {
  const size_t n = (size_t)c.n_heads * c.head_dim + 2ull * c.n_kv_heads * c.head_dim;
  const size_t widest = n > (size_t)c.d_model ? n : (size_t)c.d_model;
  const size_t need = 4ull * chunk * widest, cap = 1024ull * kTM * kTN;
  return need < cap ? need : cap;
}

namespace {

// Split-K slices of C[M][N] (+)= A[M][K] W^T: with fewer than 512 output
// tiles (two work-groups per CU) the k-loop is split into S <= 4 slices whose
// partial products pf_splitk adds in order; S * tiles < 1024 bounds the
// partial buffer at 1024 tiles of 128 x 128.
template <int DT>
int splitk_slices(int M, int N, int K) {
  const int tiles = (N / kTN) * ((M + kTM - 1) / kTM), nk = K / kBK<DT>;
  int S = tiles >= 512 ? 1 : (512 + tiles - 1) / tiles;
  S = S > 4 ? 4 : S;
  return S > nk ? nk : S;
}

// C (+)= A W^T for EPI_STORE / EPI_ADD, split over k when splitk_slices says
// so (partials in P: S * M * N floats).
template <int DT>
void launch_gemm(bool add, const act_t<DT>* A, int M, int K, const GemmB& b, int N, float* C, int ldc, float* P,
                 hipStream_t st) {
  if constexpr (DT == KIE_F16) {
    if (N % kBigT == 0 && b.end[0] % kBigT == 0 && b.end[1] % kBigT == 0 && big_tiles_pay(M, N / kBigT, false)) {
      const dim3 g(N / kBigT, (M + kBigT - 1) / kBigT);
      if (add)
        pf_gemm_big<EPI_ADD><<<g, dim3(512), 0, st>>>(A, M, K, b, C, ldc, nullptr, 0);
      else
        pf_gemm_big<EPI_STORE><<<g, dim3(512), 0, st>>>(A, M, K, b, C, ldc, nullptr, 0);
      return;
    }
  }
  const dim3 blk(256);
  const int mt = (M + kTM - 1) / kTM, S = splitk_slices<DT>(M, N, K);
  if (S == 1) {
    if (add)
      pf_gemm<EPI_ADD, DT><<<dim3(N / kTN, mt), blk, 0, st>>>(A, M, K, b, C, ldc, nullptr, 0);
    else
      pf_gemm<EPI_STORE, DT><<<dim3(N / kTN, mt), blk, 0, st>>>(A, M, K, b, C, ldc, nullptr, 0);
    return;
  }
  pf_gemm<EPI_PART, DT><<<dim3(N / kTN, mt, S), blk, 0, st>>>(A, M, K, b, P, N, nullptr, 0);
  const int q = (M * N / 4 + 255) / 256;
  if (add)
    pf_splitk<true><<<q, blk, 0, st>>>(P, S, M, N, C, ldc);
  else
    pf_splitk<false><<<q, blk, 0, st>>>(P, S, M, N, C, ldc);
}

// X += A W^T (the residual add), then, if g is not null, Xn = RMSNorm(X) * g:
// with split-K the reduction and the norm run as one pass over the rows.
template <int DT>
void launch_add_norm(const act_t<DT>* A, int M, int K, const GemmB& b, int d, float* X, float* P, const uint16_t* g,
                     float eps, act_t<DT>* Xn, hipStream_t st) {
  const int S = splitk_slices<DT>(M, d, K);
  const bool big = DT == KIE_F16 && d % kBigT == 0 && b.end[0] % kBigT == 0 && b.end[1] % kBigT == 0 &&
                   big_tiles_pay(M, d / kBigT, false);
  if (S == 1 || big || !g || d > 4096) {
    launch_gemm<DT>(true, A, M, K, b, d, X, d, P, st);
    if (g) pf_rmsnorm<DT><<<M, dim3(256), 0, st>>>(X, g, eps, M, d, Xn);
    return;
  }
  pf_gemm<EPI_PART, DT><<<dim3(d / kTN, (M + kTM - 1) / kTM, S), dim3(256), 0, st>>>(A, M, K, b, P, d, nullptr, 0);
  pf_splitk_norm<DT><<<M, dim3(256), 0, st>>>(P, S, M, d, X, g, eps, Xn);
}

// H = silu(A Wg^T) * (A Wu^T), [M][F] activations.
template <int DT>
void launch_swiglu(const act_t<DT>* A, int M, int K, const uint16_t* wg, const uint16_t* wu, int F, act_t<DT>* H,
                   hipStream_t st) {
  if constexpr (DT == KIE_F16) {
    if (F % (kBigT / 2) == 0 && big_tiles_pay(M, F / (kBigT / 2), true)) {
      pf_gemm_big<EPI_SWIGLU><<<dim3(F / (kBigT / 2), (M + kBigT - 1) / kBigT), dim3(512), 0, st>>>(
          A, M, K, GemmB{{wg, wu}, {F, F, F}}, nullptr, 0, H, F);
      return;
    }
  }
  const int mt = (M + kTM - 1) / kTM;
  pf_gemm<EPI_SWIGLU, DT><<<dim3(F / 64, mt), dim3(256), 0, st>>>(A, M, K, GemmB{{wg, wu}, {F, F, F}}, nullptr, 0,
                                                                  H, F);
}

// Causal flash attention of query rows p0 .. p0+M-1 over cache rows 0 .. p0+m.
template <int DT>
void attn_launch(const float* qkv, int M, int hq, int hkv, int hd, int p0, int max_seq, const uint16_t* kc,
                 const uint16_t* vc, void* out, hipStream_t st) {
  const int G = hq / hkv, hw = G < 4 ? G : 4, rows = 32 * (4 / hw), nqb = (M + rows - 1) / rows;
  const int ny = hkv * (G / hw);
  // pairs of query blocks while the paired grid still gives every compute
  // unit two work-groups (measured: 8192 rows from position 0 gain, 4096-row
  // chunks and short prompts lose)
  const int pair = ((nqb + 1) / 2) * ny >= 512 ? 1 : 0;
  const dim3 ag(pair ? (nqb + 1) / 2 : nqb, ny);
  act_t<DT>* o = static_cast<act_t<DT>*>(out);
  if (hd == 128)
    pf_attn<128, DT><<<ag, dim3(256), 0, st>>>(qkv, M, hq, hkv, p0, max_seq, kc, vc, o, pair);
  else
    pf_attn<64, DT><<<ag, dim3(256), 0, st>>>(qkv, M, hq, hkv, p0, max_seq, kc, vc, o, pair);
}

template <int DT>
hipError_t run_chunk(const PrefillCtx& x, const int* tok_dev, int p0, int M) {
  const kie_config& c = x.cfg;
  const int d = c.d_model, qd = c.n_heads * c.head_dim, kvd = c.n_kv_heads * c.head_dim, F = c.d_ffn;
  const int ldq = qd + 2 * kvd;
  const dim3 blk(256);
  hipStream_t st = x.stream;
  act_t<DT>* Xn = static_cast<act_t<DT>*>(x.Xn);
  act_t<DT>* Aa = static_cast<act_t<DT>*>(x.A);
  act_t<DT>* Hh = static_cast<act_t<DT>*>(x.H);
  auto gemm = [&](bool add, const act_t<DT>* A, int K, const GemmB& b, int N, float* C, int ldc) {
    launch_gemm<DT>(add, A, M, K, b, N, C, ldc, x.P, st);
  };
  pf_embed<DT><<<M, blk, 0, st>>>(x.tok_emb, tok_dev, M, d, x.X);
  pf_rmsnorm<DT><<<M, blk, 0, st>>>(x.X, x.wtab[W_ATTN_NORM], c.rms_eps, M, d, Xn);
  for (int l = 0; l < c.n_layers; ++l) {
    const uint16_t* const* w = x.wtab + (size_t)l * W_PER_LAYER;
    const size_t plane = (size_t)l * c.n_kv_heads * c.max_seq * c.head_dim;
    // Xn holds RMSNorm(X) * g_attn of this layer (the previous layer's last step made it)
    const GemmB bqkv{{w[W_Q], w[W_K], w[W_V]}, {qd, qd + kvd, ldq}};
    gemm(false, Xn, d, bqkv, ldq, x.QKV, ldq);
    const int pairs = (c.n_heads + 2 * c.n_kv_heads) * (c.head_dim / 2);
    pf_rope_kv<DT><<<(M * (pairs / 4) + 255) / 256, blk, 0, st>>>(x.QKV, M, c.n_heads, c.n_kv_heads, c.head_dim, x.rope,
                                                            p0, c.max_seq, x.kc + plane, x.vc + plane);
    attn_launch<DT>(x.QKV, M, c.n_heads, c.n_kv_heads, c.head_dim, p0, c.max_seq, x.kc + plane, x.vc + plane, Aa,
                    st);
    launch_add_norm<DT>(Aa, M, qd, GemmB{{w[W_O]}, {d, d, d}}, d, x.X, x.P, w[W_FFN_NORM], c.rms_eps, Xn, st);
    launch_swiglu<DT>(Xn, M, d, w[W_GATE], w[W_UP], F, Hh, st);
    const uint16_t* g_next = l + 1 < c.n_layers ? x.wtab[(size_t)(l + 1) * W_PER_LAYER + W_ATTN_NORM] : nullptr;
    launch_add_norm<DT>(Hh, M, F, GemmB{{w[W_DOWN]}, {d, d, d}}, d, x.X, x.P, g_next, c.rms_eps, Xn, st);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t prefill_chunk(const PrefillCtx& x, const int* tok_dev, int p0, int M) {
  return x.cfg.dtype == KIE_BF16 ? run_chunk<KIE_BF16>(x, tok_dev, p0, M) : run_chunk<KIE_F16>(x, tok_dev, p0, M);
}

namespace {

template <int DT>
void probe_launch(int op, const void* A, int M, int K, const uint16_t* w, const uint16_t* w2, int N, void* out,
                  float* P, hipStream_t st) {
  const act_t<DT>* a = static_cast<const act_t<DT>*>(A);
  if (op == KIE_GEMM_SWIGLU)
    launch_swiglu<DT>(a, M, K, w, w2, N, static_cast<act_t<DT>*>(out), st);
  else
    launch_gemm<DT>(op == KIE_GEMM_ADD, a, M, K, GemmB{{w}, {N, N, N}}, N, static_cast<float*>(out), N, P, st);
}

}  // namespace
}  // namespace kie

extern "C" kie_status kie_attn_probe(int32_t dtype, const float* qkv_dev, int32_t M, int32_t n_heads,
                                     int32_t n_kv_heads, int32_t head_dim, int32_t p0, int32_t max_seq,
                                     const void* k_cache_dev, const void* v_cache_dev, void* out_dev, int32_t reps,
                                     void* hip_stream, float* kernel_ms) {
  using namespace kie;
  if (dtype != KIE_F16 && dtype != KIE_BF16) return KIE_ERR_ARG;
  if (!qkv_dev || !k_cache_dev || !v_cache_dev || !out_dev || reps < 1) return KIE_ERR_ARG;
  if (head_dim != 64 && head_dim != 128) return KIE_ERR_ARG;
  if (n_kv_heads < 1 || n_heads < n_kv_heads || n_heads % n_kv_heads || n_heads > 256) return KIE_ERR_ARG;
  const int G = n_heads / n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return KIE_ERR_ARG;
  if (M < 1 || M > 65536 || p0 < 0 || max_seq < 1 || (int64_t)p0 + M > max_seq) return KIE_ERR_ARG;
  const uintptr_t al = reinterpret_cast<uintptr_t>(qkv_dev) | reinterpret_cast<uintptr_t>(k_cache_dev) |
                       reinterpret_cast<uintptr_t>(v_cache_dev) | reinterpret_cast<uintptr_t>(out_dev);
  if (al & 15) return KIE_ERR_ARG;
  hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
  const uint16_t* kc = static_cast<const uint16_t*>(k_cache_dev);
  const uint16_t* vc = static_cast<const uint16_t*>(v_cache_dev);
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return KIE_ERR_HIP;
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return KIE_ERR_HIP;
  }
  hipError_t he = hipEventRecord(e0, st);
  for (int r = 0; r < reps && he == hipSuccess; ++r) {
    if (dtype == KIE_BF16)
      attn_launch<KIE_BF16>(qkv_dev, M, n_heads, n_kv_heads, head_dim, p0, max_seq, kc, vc, out_dev, st);
    else
      attn_launch<KIE_F16>(qkv_dev, M, n_heads, n_kv_heads, head_dim, p0, max_seq, kc, vc, out_dev, st);
    he = hipGetLastError();
  }
  if (he == hipSuccess) he = hipEventRecord(e1, st);
  if (he == hipSuccess) he = hipStreamSynchronize(st);
  float ms = 0.f;
  if (he == hipSuccess) he = hipEventElapsedTime(&ms, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (he != hipSuccess) {
    if (getenv("KIE_VERBOSE")) fprintf(stderr, "kie: attention probe failed: %s\n", hipGetErrorString(he));
    return KIE_ERR_HIP;
  }
  if (kernel_ms) *kernel_ms = ms / reps;
  return KIE_OK;
}

extern "C" kie_status kie_gemm_probe(int32_t op, int32_t dtype, const void* A_dev, int32_t M, int32_t K,
                                     const void* W_dev, const void* W2_dev, int32_t N, void* out_dev, void* part_dev,
                                     size_t part_bytes, int32_t reps, void* hip_stream, int32_t* slices,
                                     float* kernel_ms) {
  using namespace kie;
  if (op != KIE_GEMM_STORE && op != KIE_GEMM_ADD && op != KIE_GEMM_SWIGLU) return KIE_ERR_ARG;
  if (dtype != KIE_F16 && dtype != KIE_BF16) return KIE_ERR_ARG;
  if (!A_dev || !W_dev || !out_dev || (op == KIE_GEMM_SWIGLU && !W2_dev) || reps < 1) return KIE_ERR_ARG;
  if (M < 1 || M > 65536 || K < kBKMax || K % kBKMax || K > 65536 || N < 64 || N > 65536 ||
      (int64_t)M * N > INT32_MAX)
    return KIE_ERR_ARG;
  if (N % (op == KIE_GEMM_SWIGLU ? 64 : kTN)) return KIE_ERR_ARG;
  const uintptr_t al = reinterpret_cast<uintptr_t>(A_dev) | reinterpret_cast<uintptr_t>(W_dev) |
                       reinterpret_cast<uintptr_t>(W2_dev) | reinterpret_cast<uintptr_t>(out_dev) |
                       reinterpret_cast<uintptr_t>(part_dev);
  if (al & 15) return KIE_ERR_ARG;
  const int S = op == KIE_GEMM_SWIGLU ? 1 : dtype == KIE_BF16 ? splitk_slices<KIE_BF16>(M, N, K)
                                                              : splitk_slices<KIE_F16>(M, N, K);
  if (S > 1 && (!part_dev || part_bytes < (size_t)S * M * N * sizeof(float))) return KIE_ERR_CAPACITY;
  hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
  const uint16_t* w = static_cast<const uint16_t*>(W_dev);
  const uint16_t* w2 = static_cast<const uint16_t*>(W2_dev);
  float* P = static_cast<float*>(part_dev);
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return KIE_ERR_HIP;
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return KIE_ERR_HIP;
  }
  hipError_t he = hipEventRecord(e0, st);
  for (int r = 0; r < reps && he == hipSuccess; ++r) {
    if (dtype == KIE_BF16)
      probe_launch<KIE_BF16>(op, A_dev, M, K, w, w2, N, out_dev, P, st);
    else
      probe_launch<KIE_F16>(op, A_dev, M, K, w, w2, N, out_dev, P, st);
    he = hipGetLastError();
  }
  if (he == hipSuccess) he = hipEventRecord(e1, st);
  if (he == hipSuccess) he = hipStreamSynchronize(st);
  float ms = 0.f;
  if (he == hipSuccess) he = hipEventElapsedTime(&ms, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (he != hipSuccess) {
    if (getenv("KIE_VERBOSE")) fprintf(stderr, "kie: gemm probe failed: %s\n", hipGetErrorString(he));
    return KIE_ERR_HIP;
  }
  if (slices) *slices = S;
  if (kernel_ms) *kernel_ms = ms / reps;
  return KIE_OK;
}
