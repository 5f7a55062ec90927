// The persistent decode monokernel for gfx950 (MI355X), its GEMV engine and
// the isolated GEMV probe kernel.
//
// One work-group per compute unit stays resident for the whole call and loops
// over decode steps; inside a step it walks the layers stage by stage.  The
// design follows the Kog pages (revietech.ru, "Kog vyzhimayet maksimum iz GPU:
// 3000 tokenov/s", sections "Chto takoye monokernel" and "Arkhitektura i
// osobennosti"): one resident program for the whole decode loop including
// LM-head sampling and the EOS test; hand-offs between work-groups through
// NaN-initialised buffers that consumers poll; batch-1 projections on the dot2
// vector ALU instructions.  The tiling below is written for CDNA4 (wave64,
// 256 CUs in 8 XCDs, non-coherent per-XCD L2), not taken from the pages.
//
// Stage order of one decode step (t = token, p = position):
//   embed:    x = E[t] (each work-group, into LDS)
//   per layer l:
//     QKV     n = RMSNorm(x)*g; rows of [Wq;Wk;Wv] . n published unrotated
//     ATTN    split-KV units (KV head, chunk): rotary on q (and on the new k,
//             which the unit holding position p appends to the KV cache),
//             partial (m, l, o) per query head
//     MERGE   units (head, 8 dims): combine the chunk partials -> attention out
//     WO      x_mid = x + Wo a           (rows split over work-groups)
//     GATEUP  h = silu(Wg n) * (Wu n), n = RMSNorm(x_mid)*g
//     DOWN    x_next = x_mid + Wd h
//   LM head:  logits rows, per-work-group (max, index) partial
//   argmax:   every work-group reduces all partials -> same next token; EOS test
//
// Code-generation note.  All stages are inlined into one kernel.  Each stage
// re-derives the thread index and the parameter pointer through an empty asm
// statement (opaque_*), so the compiler cannot hoist per-stage address
// arithmetic out of the layer loop and keep it live across all stages.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kie_device.hpp"

#define KIE_INLINE __attribute__((always_inline))

namespace kie {

__device__ __forceinline__ int opaque_v(int v) {
  asm volatile("" : "+v"(v));
  return v;
}
template <class T>
__device__ __forceinline__ T* opaque_s(T* p) {
  asm volatile("" : "+s"(p));
  return p;
}

// ---------------------------------------------------------------------------
// LDS view
// ---------------------------------------------------------------------------
struct Lds {
  float* xres;     // fp32 residual stream copy [d]
  uint16_t* xn;    // 16-bit activation fed to dot2 [Kmax]
  float* red;      // GEMV per-wave partial sums [kRedCap]
  float* yv;       // GEMV finished rows [kYCap]
  float* scr;      // attention scratch (aliases red/yv)
  float* misc;     // 64 floats: block reductions
  int* imisc;      // 64 ints
};

__device__ __forceinline__ Lds lds_view(char* smem, const Params& P) {
  Lds s;
  s.xres = reinterpret_cast<float*>(smem + P.lds_xres);
  s.xn = reinterpret_cast<uint16_t*>(smem + P.lds_xn);
  s.red = reinterpret_cast<float*>(smem + P.lds_scr);
  s.yv = s.red + kRedCap;
  s.scr = s.red;
  s.misc = reinterpret_cast<float*>(smem + P.lds_misc);
  s.imisc = reinterpret_cast<int*>(s.misc + 64);
  return s;
}

// Per-stage context: everything re-derived at stage entry (see note above).
struct Sc {
  const Params& P;
  Lds s;
  Watch w;
  int t, wg, nb;
};

__device__ __forceinline__ Sc stage_ctx(const Params* Pp, char* smem) {
  const Params& P = *opaque_s(Pp);
  return Sc{P, lds_view(smem, P), Watch{P.timeout, P.ctl + CTL_STATUS}, opaque_v((int)threadIdx.x),
            (int)blockIdx.x, (int)gridDim.x};
}

// Work-group-wide "any thread failed" with a barrier.
__device__ __forceinline__ bool any_failed(bool failed) { return __syncthreads_or(failed ? 1 : 0) != 0; }

// Deterministic block sum (fixed order); every thread receives the total.
__device__ __forceinline__ float block_sum(float v, float* misc, int t) {
  v = sum64_tail(v);
  if ((t & 63) == 63) misc[t >> 6] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) s += misc[w];
  __syncthreads();
  return s;
}

// ---------------------------------------------------------------------------
// Input preparation
// ---------------------------------------------------------------------------
// Poll n fp32 words (n even) of an exchange buffer into LDS as fp32.
__device__ __forceinline__ bool poll_f32(const uint32_t* src, int n, float* dst, const Watch& w, int t) {
  bool ok = true;
  for (int i = t; i < (n >> 1); i += kThreads) {
    uint64_t v = 0;
    if (ok && poll64(src + 2 * i, v, w, Ready32x2{})) {
      dst[2 * i] = lo_f(v);
      dst[2 * i + 1] = hi_f(v);
    } else {
      ok = false;
    }
  }
  return !any_failed(!ok);
}
// Poll n fp32 words into LDS as 16-bit activations.
template <int DT>
__device__ __forceinline__ bool poll_to16(const uint32_t* src, int n, uint16_t* dst, const Watch& w, int t) {
  bool ok = true;
  for (int i = t; i < (n >> 1); i += kThreads) {
    uint64_t v = 0;
    if (ok && poll64(src + 2 * i, v, w, Ready32x2{})) {
      reinterpret_cast<uint32_t*>(dst)[i] = pack16<DT>(lo_f(v), hi_f(v));
    } else {
      ok = false;
    }
  }
  return !any_failed(!ok);
}
// xn = RMSNorm(x) * g, rounded to 16 bits.  Ends with a barrier.
template <int DT>
__device__ __forceinline__ void rmsnorm_to16(const float* x, const uint16_t* g, int n, float eps, uint16_t* xn,
                                             float* misc, int t) {
  float ss = 0.f;
  for (int i = t; i < n; i += kThreads) ss += x[i] * x[i];
  ss = block_sum(ss, misc, t);
  const float r = 1.0f / sqrtf(ss / (float)n + eps);
  for (int i = t; i < n; i += kThreads) xn[i] = to_16<DT>(x[i] * r * to_f32<DT>(g[i]));
  __syncthreads();
}

// ---------------------------------------------------------------------------
// GEMV engine.
//
// A work-group owns `nrows` rows of K columns (row pointers from rowptr(r)).
// The rows are read as 16-byte vectors (8 elements): lanes_per_row = min(K/8,
// 512) consecutive threads read consecutive vectors of one row, so every wave
// load is 1 KB of contiguous memory; rows_per_pass = 512 / lanes_per_row rows
// are read per pass, and rows longer than 512 vectors give each thread VPT
// vectors per row.  Each thread keeps kDepth vectors in flight in a register
// ring; the first kDepth loads are issued BEFORE the input is polled, so the
// weight stream runs while the hand-off completes.  Partial dot products
// (v_dot2c, fp32) are reduced across the lanes of a row on DPP and across
// waves through LDS in a fixed order (deterministic).
// ---------------------------------------------------------------------------
struct Gv {
  int nrows, vpr, lpr, rp, passes, J, sub, kl, nwr;
};

template <int VPT>
__device__ __forceinline__ Gv gv_plan(int nrows, int K, int t) {
  Gv g;
  g.nrows = nrows;
  g.vpr = K >> 3;
  g.lpr = g.vpr < kThreads ? g.vpr : kThreads;
  g.rp = kThreads / g.lpr;
  g.passes = (nrows + g.rp - 1) / g.rp;
  g.J = g.passes * VPT;
  g.sub = t / g.lpr;
  g.kl = t % g.lpr;
  g.nwr = g.lpr >= 64 ? g.lpr / 64 : 1;
  return g;
}

template <int VPT, class RowPtr>
__device__ __forceinline__ const uint16_t* gv_addr(const Gv& g, RowPtr& rowptr, int j) {
  const int p = j / VPT, i = j % VPT;
  const int row = p * g.rp + g.sub;
  const int kv = g.kl + i * g.lpr;
  // out-of-range vectors re-read row 0 (a cache hit) and are discarded
  const bool ok = row < g.nrows && kv < g.vpr;
  return rowptr(ok ? row : 0) + (size_t)(ok ? kv : 0) * 8;
}

// Reduce one row-partial over the lanes of its row and park it in LDS.
// WIDE: a row spans >= 64 lanes (K >= 512); else 32 lanes (K = 256).
template <bool WIDE>
__device__ __forceinline__ void gv_park(float acc, int p, const Gv& g, float* red, int t) {
  const int row = p * g.rp + g.sub;
  if constexpr (WIDE) {
    acc = sum64_tail(acc);
    if ((t & 63) == 63 && row < g.nrows) red[row * g.nwr + (g.kl >> 6)] = acc;
  } else {  // two rows per wave
    acc = sum32_tail(acc);
    if ((t & 31) == 31 && row < g.nrows) red[row] = acc;
  }
}

// Runs prep() (poll + normalisation; must end with a barrier and leave the
// 16-bit input in xs) between the ring prologue and the main loop.  On return
// yv[r] holds row r's dot product for r < nrows (after a barrier).
//
// The vector count per thread is padded to a multiple of kDepth so that the
// unrolled ring has no data-dependent branches: every slot is consumed and
// refilled unconditionally (padding vectors read row 0 again and are
// discarded), which lets the compiler wait for exactly the oldest load
// (vmcnt(kDepth-1)) instead of draining the queue.
template <int DT, int VPT, bool WIDE, class RowPtr, class Prep>
__device__ __forceinline__ bool gemv(int nrows, int K, RowPtr rowptr, Prep prep, const uint16_t* xs, float* red,
                                     float* yv, int t) {
  const Gv g = gv_plan<VPT>(nrows, K, t);
  const int Jp = (g.J + kDepth - 1) / kDepth * kDepth;
  uint4 ring[kDepth];
  if (Jp > 0) {
#pragma unroll
    for (int i = 0; i < kDepth; ++i) ring[i] = ldw(gv_addr<VPT>(g, rowptr, i));
  }
  if (!prep()) return false;
  if (Jp > 0) {
    uint4 xr[VPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int kv = g.kl + i * g.lpr;
      xr[i] = kv < g.vpr ? *reinterpret_cast<const uint4*>(xs + kv * 8) : make_uint4(0, 0, 0, 0);
    }
    float acc = 0.f;
    int j0 = 0;
    for (; j0 + kDepth < Jp; j0 += kDepth) {
#pragma unroll
      for (int i = 0; i < kDepth; ++i) {
        acc = dot8<DT>(ring[i], xr[i % VPT], acc);
        ring[i] = ldw(gv_addr<VPT>(g, rowptr, j0 + i + kDepth));
        if (i % VPT == VPT - 1) {
          gv_park<WIDE>(acc, (j0 + i) / VPT, g, red, t);
          acc = 0.f;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kDepth; ++i) {  // last block: drain
      acc = dot8<DT>(ring[i], xr[i % VPT], acc);
      if (i % VPT == VPT - 1) {
        gv_park<WIDE>(acc, (j0 + i) / VPT, g, red, t);
        acc = 0.f;
      }
    }
  }
  __syncthreads();
  for (int r = t; r < nrows; r += kThreads) {
    float y = 0.f;
    for (int w = 0; w < g.nwr; ++w) y += red[r * g.nwr + w];
    yv[r] = y;
  }
  __syncthreads();
  return true;
}

template <int DT, class RowPtr, class Prep>
__device__ __forceinline__ bool gemv_any(int nrows, int K, RowPtr rowptr, Prep prep, const uint16_t* xs, float* red,
                                         float* yv, int t) {
  const int vpr = K >> 3;
  if (vpr < 64) return gemv<DT, 1, false>(nrows, K, rowptr, prep, xs, red, yv, t);
  if (vpr <= kThreads) return gemv<DT, 1, true>(nrows, K, rowptr, prep, xs, red, yv, t);
  if (vpr <= 2 * kThreads) return gemv<DT, 2, true>(nrows, K, rowptr, prep, xs, red, yv, t);
  return gemv<DT, 4, true>(nrows, K, rowptr, prep, xs, red, yv, t);
}

__device__ __forceinline__ int split_lo(int n, int parts, int i) { return (int)(((long long)n * i) / parts); }

__device__ __forceinline__ const uint16_t* lw_ptr(const Params& P, int l, int k) {
  return P.lw[l * W_PER_LAYER + k];
}

// ---------------------------------------------------------------------------
// Stages
// ---------------------------------------------------------------------------

// QKV projection: rows [r0, r1) of the stacked [Wq; Wk; Wv] (contiguous row
// segments of the three matrices), published unrotated in fp32.  Input x_l:
// LDS xres (layer 0: the embedding) or polled from the previous layer's xout.
template <int DT>
__device__ KIE_INLINE bool st_qkv(const Params* Pp, char* smem, int l, uint32_t* X) {
  const Sc c = stage_ctx(Pp, smem);
  const Params& P = c.P;
  const int hd = P.hd, d = P.d;
  const int nq = P.hq * hd, nk = P.hkv * hd;
  const int N = nq + 2 * nk;
  const int r0 = split_lo(N, c.nb, c.wg), r1 = split_lo(N, c.nb, c.wg + 1);
  const uint16_t* wq = lw_ptr(P, l, W_Q);
  const uint16_t* wk = lw_ptr(P, l, W_K);
  const uint16_t* wv = lw_ptr(P, l, W_V);
  auto rowptr = [&](int r) -> const uint16_t* {
    const int row = r0 + r;
    return row < nq ? wq + (size_t)row * d
         : row < nq + nk ? wk + (size_t)(row - nq) * d : wv + (size_t)(row - nq - nk) * d;
  };
  auto prep = [&]() -> bool {
    if (l > 0 && !poll_f32(X + P.xl.xout + (size_t)(l - 1) * d, d, c.s.xres, c.w, c.t)) return false;
    rmsnorm_to16<DT>(c.s.xres, lw_ptr(P, l, W_ATTN_NORM), d, P.eps, c.s.xn, c.s.misc, c.t);
    return true;
  };
  if (!gemv_any<DT>(r1 - r0, d, rowptr, prep, c.s.xn, c.s.red, c.s.yv, c.t)) return false;
  uint32_t* dst = X + P.xl.qkv + (size_t)l * N;
  for (int r = c.t; r < r1 - r0; r += kThreads) xst32(dst + r0 + r, __float_as_uint(c.s.yv[r]));
  return true;
}

__device__ __forceinline__ void attn_chunking(const Params& P, int n, int& CL, int& nch) {
  CL = (n + P.cmax - 1) / P.cmax;
  if (CL < kClMin) CL = kClMin;
  nch = (n + CL - 1) / CL;
}

// Rotary embedding in place on LDS vectors: nvec vectors of hd floats, pair
// (i, i + hd/2) turned by the angle of `pos` (table built on the host in
// double precision).  Ends with a barrier.
__device__ __forceinline__ void rope_lds(float* v, int nvec, int hd, const float* rope, int pos, int t) {
  const int half = hd >> 1;
  for (int k = t; k < nvec * half; k += kThreads) {
    const int h = k / half, i = k % half;
    const float cs = rope[((size_t)pos * half + i) * 2], sn = rope[((size_t)pos * half + i) * 2 + 1];
    const float a = v[h * hd + i], b = v[h * hd + i + half];
    v[h * hd + i] = a * cs - b * sn;
    v[h * hd + i + half] = a * sn + b * cs;
  }
  __syncthreads();
}

// Split-KV attention (flash-decoding): unit (KV head g, chunk c) computes, for
// the G query heads that read head g, the partial softmax statistics over the
// chunk's positions: m = max score, l = sum exp(s - m), o = sum exp(s - m) v.
// Rotary embedding of q and of the new k is fused here; the unit whose chunk
// holds the current position also appends (rotated k, v) to the KV cache.
template <int DT, int G>
__device__ KIE_INLINE bool st_attn(const Params* Pp, char* smem, int l, int pos, uint32_t* X) {
  const Sc c = stage_ctx(Pp, smem);
  const Params& P = c.P;
  const int t = c.t;
  const int hd = P.hd, hkv = P.hkv, hq = P.hq;
  const int N = (hq + 2 * hkv) * hd;
  const int n = pos + 1;
  int CL, nch;
  attn_chunking(P, n, CL, nch);
  const int units = hkv * nch;
  const int LPP = hd >> 3;                // lanes per position row
  const int PP = kThreads / LPP;          // positions per pass
  const int pp = t / LPP, e8 = (t % LPP) * 8;
  const float scale = 1.0f / sqrtf((float)hd);
  float* qs = c.s.scr;                    // [G][hd]
  float* kn = qs + G * hd;                // [hd] new key (fp32, rotated); must follow qs
  float* vn = kn + hd;                    // [hd] new value
  uint16_t* kv16 = reinterpret_cast<uint16_t*>(vn + hd);  // [2][hd] new row as stored
  float* ored = vn + 2 * hd;              // [kWaves][G][hd]
  float* ml = ored + kWaves * G * hd;     // [G][2] (padded to 16 floats)
  float* sc = ml + 16;                    // [G][cl_cap]
  constexpr int APF = 8;                  // passes prefetched into registers
  const uint32_t* src = X + P.xl.qkv + (size_t)l * N;
  const int wave = t >> 6, lane = t & 63;
  for (int u = c.wg; u < units; u += c.nb) {
    const int g = u % hkv, ch = u / hkv;
    const int j0 = ch * CL, j1 = min(n, j0 + CL), len = j1 - j0;
    const bool has_new = pos >= j0 && pos < j1;
    const int npass = (len + PP - 1) / PP;
    const size_t plane = ((size_t)l * hkv + g) * P.max_seq * hd;
    uint16_t* kb = P.kc + plane;
    uint16_t* vb = P.vc + plane;
    // cached rows (written by earlier steps) are independent of this step:
    // start streaming them before waiting for q
    uint4 kr[APF], vr[APF];
#pragma unroll
    for (int a = 0; a < APF; ++a) {
      const int j = j0 + a * PP + pp;
      if (a < npass && j < j1 && j != pos) {
        kr[a] = ldw(kb + (size_t)j * hd + e8);
        vr[a] = ldw(vb + (size_t)j * hd + e8);
      }
    }
    bool ok = true;
    // queries of the G heads sharing KV head g (+ the new k, v of head g)
    const int nq2 = (G * hd) >> 1;
    const int nw2 = nq2 + (has_new ? hd : 0);
    for (int i = t; i < nw2; i += kThreads) {
      const uint32_t* sp;
      float* dp;
      if (i < nq2) {
        sp = src + (size_t)g * G * hd + 2 * i;
        dp = qs + 2 * i;
      } else if (i < nq2 + (hd >> 1)) {
        const int k = i - nq2;
        sp = src + (size_t)hq * hd + (size_t)g * hd + 2 * k;
        dp = kn + 2 * k;
      } else {
        const int k = i - nq2 - (hd >> 1);
        sp = src + (size_t)(hq + hkv) * hd + (size_t)g * hd + 2 * k;
        dp = vn + 2 * k;
      }
      uint64_t v = 0;
      if (ok && poll64(sp, v, c.w, Ready32x2{})) {
        dp[0] = lo_f(v);
        dp[1] = hi_f(v);
      } else {
        ok = false;
      }
    }
    if (any_failed(!ok)) return false;
    rope_lds(qs, has_new ? G + 1 : G, hd, P.rope, pos, t);  // kn follows qs: rotated too
    if (has_new) {
      // append the new row to the cache (read by later steps) and keep the
      // stored 16-bit values for this step's own use
      uint32_t* kd = reinterpret_cast<uint32_t*>(kb + (size_t)pos * hd);
      uint32_t* vd = reinterpret_cast<uint32_t*>(vb + (size_t)pos * hd);
      for (int i = t; i < hd; i += kThreads) {  // i < hd/2: key pairs, else value pairs
        const bool isk = i < (hd >> 1);
        const int k = isk ? i : i - (hd >> 1);
        const float* f = isk ? kn : vn;
        const uint32_t wv = pack16<DT>(f[2 * k], f[2 * k + 1]);
        xst32((isk ? kd : vd) + k, wv);
        reinterpret_cast<uint32_t*>(kv16)[(isk ? 0 : (hd >> 1)) + k] = wv;
      }
      __syncthreads();
#pragma unroll
      for (int a = 0; a < APF; ++a) {
        const int j = j0 + a * PP + pp;
        if (a < npass && j == pos) {
          kr[a] = *reinterpret_cast<const uint4*>(kv16 + e8);
          vr[a] = *reinterpret_cast<const uint4*>(kv16 + hd + e8);
        }
      }
    }
    // scores
    for (int a = 0; a < npass; ++a) {
      const int j = j0 + a * PP + pp;
      const bool valid = j < j1;
      uint4 kv4 = make_uint4(0, 0, 0, 0);
      if (a < APF) {
#pragma unroll
        for (int b = 0; b < APF; ++b)
          if (b == a) kv4 = kr[b];
      } else if (valid) {
        kv4 = j == pos ? *reinterpret_cast<const uint4*>(kv16 + e8) : ldw(kb + (size_t)j * hd + e8);
      }
      float kf[8];
      unpack8<DT>(kv4, kf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float* qh = qs + h * hd + e8;
        float sdot = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) sdot += qh[e] * kf[e];
        sdot = (LPP == 16) ? sum16(sdot) : sum8(sdot);
        if ((t % LPP) == 0 && valid) sc[h * P.cl_cap + (j - j0)] = sdot * scale;
      }
    }
    __syncthreads();
    // softmax statistics: wave h handles head h
    for (int h = wave; h < G; h += kWaves) {
      float* sh = sc + h * P.cl_cap;
      float m = -INFINITY;
      for (int j = lane; j < len; j += 64) m = fmaxf(m, sh[j]);
      m = wave_max(m);
      float sum = 0.f;
      for (int j = lane; j < len; j += 64) {
        const float pj = expf(sh[j] - m);
        sh[j] = pj;
        sum += pj;
      }
      sum = wave_sum(sum);
      if (lane == 0) {
        ml[2 * h] = m;
        ml[2 * h + 1] = sum;
      }
    }
    __syncthreads();
    // o = sum_j p_j v_j
    float o[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
    for (int a = 0; a < npass; ++a) {
      const int j = j0 + a * PP + pp;
      if (j >= j1) continue;
      uint4 vv4 = make_uint4(0, 0, 0, 0);
      if (a < APF) {
#pragma unroll
        for (int b = 0; b < APF; ++b)
          if (b == a) vv4 = vr[b];
      } else {
        vv4 = j == pos ? *reinterpret_cast<const uint4*>(kv16 + hd + e8) : ldw(vb + (size_t)j * hd + e8);
      }
      float vf[8];
      unpack8<DT>(vv4, vf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float pj = sc[h * P.cl_cap + (j - j0)];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] += pj * vf[e];
      }
    }
    // reduce over the position groups of the wave (lanes with equal t % LPP)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v = o[h][e];
        for (int msk = LPP; msk < 64; msk <<= 1) v += __shfl_xor(v, msk);
        o[h][e] = v;
      }
    if (lane < LPP) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) ored[(wave * G + h) * hd + e8 + e] = o[h][e];
    }
    __syncthreads();
    uint32_t* att = X + P.xl.att;
    for (int idx = t; idx < G * hd; idx += kThreads) {
      const int h = idx / hd, e = idx % hd;
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) acc += ored[(w * G + h) * hd + e];
      uint32_t* rowp = att + (((size_t)l * hq + (size_t)g * G + h) * P.cmax + ch) * P.astride;
      xst32(rowp + 4 + e, __float_as_uint(acc));
      if (e == 0) xst64(rowp, pack2f(ml[2 * h], ml[2 * h + 1]));
    }
    __syncthreads();
  }
  return true;
}

// Merge of the split-KV partials.  Unit (head h, dims 8s..8s+7) runs on one
// wave; lanes walk the chunks with an online rescaling, then the wave combines.
template <int DT>
__device__ KIE_INLINE bool st_merge(const Params* Pp, char* smem, int l, int pos, uint32_t* X) {
  const Sc c = stage_ctx(Pp, smem);
  const Params& P = c.P;
  const int hd = P.hd, hq = P.hq;
  int CL, nch;
  attn_chunking(P, pos + 1, CL, nch);
  const int spl = hd >> 3;
  const int units = hq * spl;
  const int wave = c.t >> 6, lane = c.t & 63;
  bool ok = true;
  for (int u = c.wg + wave * c.nb; u < units; u += c.nb * kWaves) {
    const int h = u / spl, sl = u % spl;
    float m = -INFINITY, ls = 0.f, o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;
    for (int ch = lane; ch < nch && ok; ch += 64) {
      const uint32_t* rowp = X + P.xl.att + (((size_t)l * hq + h) * P.cmax + ch) * P.astride;
      uint64_t mlv = 0, o01 = 0, o23 = 0, o45 = 0, o67 = 0;
      const uint32_t* op = rowp + 4 + sl * 8;
      ok = poll64(rowp, mlv, c.w, Ready32x2{}) && poll64(op, o01, c.w, Ready32x2{}) &&
           poll64(op + 2, o23, c.w, Ready32x2{}) && poll64(op + 4, o45, c.w, Ready32x2{}) &&
           poll64(op + 6, o67, c.w, Ready32x2{});
      if (!ok) break;
      const float mc = lo_f(mlv), lc = hi_f(mlv);
      const float mn = fmaxf(m, mc);
      const float a = expf(m - mn), b = expf(mc - mn);
      ls = ls * a + lc * b;
      const float oc[8] = {lo_f(o01), hi_f(o01), lo_f(o23), hi_f(o23), lo_f(o45), hi_f(o45), lo_f(o67), hi_f(o67)};
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = o[e] * a + oc[e] * b;
      m = mn;
    }
    const float M = wave_max(m);
    const float f = (m == -INFINITY) ? 0.f : expf(m - M);
    ls = sum64_tail(ls * f);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = sum64_tail(o[e] * f);
    if (lane == 63 && ok) {
      const float inv = 1.0f / ls;
      uint32_t* dst = X + P.xl.a + (size_t)l * hq * hd + (size_t)h * hd + sl * 8;
      xst64(dst, pack2f(o[0] * inv, o[1] * inv));
      xst64(dst + 2, pack2f(o[2] * inv, o[3] * inv));
      xst64(dst + 4, pack2f(o[4] * inv, o[5] * inv));
      xst64(dst + 6, pack2f(o[6] * inv, o[7] * inv));
    }
  }
  return !any_failed(!ok);
}

// x_mid = x_l + Wo a  (rows split over work-groups)
template <int DT>
__device__ KIE_INLINE bool st_wo(const Params* Pp, char* smem, int l, uint32_t* X) {
  const Sc c = stage_ctx(Pp, smem);
  const Params& P = c.P;
  const int d = P.d, K = P.hq * P.hd;
  const int r0 = split_lo(d, c.nb, c.wg), r1 = split_lo(d, c.nb, c.wg + 1);
  const uint16_t* W = lw_ptr(P, l, W_O);
  auto rowptr = [&](int r) -> const uint16_t* { return W + (size_t)(r0 + r) * K; };
  auto prep = [&]() -> bool { return poll_to16<DT>(X + P.xl.a + (size_t)l * K, K, c.s.xn, c.w, c.t); };
  if (!gemv_any<DT>(r1 - r0, K, rowptr, prep, c.s.xn, c.s.red, c.s.yv, c.t)) return false;
  uint32_t* dst = X + P.xl.xmid + (size_t)l * d;
  for (int r = c.t; r < r1 - r0; r += kThreads)
    xst32(dst + r0 + r, __float_as_uint(c.s.xres[r0 + r] + c.s.yv[r]));
  return true;
}

// h = silu(Wg n) * (Wu n), n = RMSNorm(x_mid) * g_ffn
template <int DT>
__device__ KIE_INLINE bool st_gateup(const Params* Pp, char* smem, int l, uint32_t* X) {
  const Sc c = stage_ctx(Pp, smem);
  const Params& P = c.P;
  const int d = P.d, F = P.F;
  const int f0 = split_lo(F, c.nb, c.wg), f1 = split_lo(F, c.nb, c.wg + 1);
  const int nf = f1 - f0;
  const uint16_t* Wg = lw_ptr(P, l, W_GATE);
  const uint16_t* Wu = lw_ptr(P, l, W_UP);
  auto rowptr = [&](int r) -> const uint16_t* {
    return r < nf ? Wg + (size_t)(f0 + r) * d : Wu + (size_t)(f0 + r - nf) * d;
  };
  auto prep = [&]() -> bool {
    if (!poll_f32(X + P.xl.xmid + (size_t)l * d, d, c.s.xres, c.w, c.t)) return false;
    rmsnorm_to16<DT>(c.s.xres, lw_ptr(P, l, W_FFN_NORM), d, P.eps, c.s.xn, c.s.misc, c.t);
    return true;
  };
  if (!gemv_any<DT>(2 * nf, d, rowptr, prep, c.s.xn, c.s.red, c.s.yv, c.t)) return false;
  uint32_t* dst = X + P.xl.h + (size_t)l * F;
  for (int f = c.t; f < nf; f += kThreads) {
    const float gt = c.s.yv[f], up = c.s.yv[nf + f];
    xst32(dst + f0 + f, __float_as_uint(gt / (1.0f + expf(-gt)) * up));
  }
  return true;
}

// x_next = x_mid + Wd h
template <int DT>
__device__ KIE_INLINE bool st_down(const Params* Pp, char* smem, int l, uint32_t* X) {
  const Sc c = stage_ctx(Pp, smem);
  const Params& P = c.P;
  const int d = P.d, F = P.F;
  const int r0 = split_lo(d, c.nb, c.wg), r1 = split_lo(d, c.nb, c.wg + 1);
  const uint16_t* W = lw_ptr(P, l, W_DOWN);
  auto rowptr = [&](int r) -> const uint16_t* { return W + (size_t)(r0 + r) * F; };
  auto prep = [&]() -> bool { return poll_to16<DT>(X + P.xl.h + (size_t)l * F, F, c.s.xn, c.w, c.t); };
  if (!gemv_any<DT>(r1 - r0, F, rowptr, prep, c.s.xn, c.s.red, c.s.yv, c.t)) return false;
  uint32_t* dst = X + P.xl.xout + (size_t)l * d;
  for (int r = c.t; r < r1 - r0; r += kThreads)
    xst32(dst + r0 + r, __float_as_uint(c.s.xres[r0 + r] + c.s.yv[r]));
  return true;
}

// (value, index) order for greedy argmax: larger value wins, lower index on ties.
__device__ __forceinline__ bool arg_better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  for (int msk = 1; msk < 64; msk <<= 1) {
    const float ov = __shfl_xor(v, msk);
    const int oi = __shfl_xor(i, msk);
    if (arg_better(ov, oi, v, i)) {
      v = ov;
      i = oi;
    }
  }
}
// Block argmax in a fixed order; every thread receives the result.
__device__ __forceinline__ void block_argmax(float& v, int& i, const Lds& s, int t) {
  wave_argmax(v, i);
  if ((t & 63) == 0) {
    s.misc[t >> 6] = v;
    s.imisc[t >> 6] = i;
  }
  __syncthreads();
  float bv = s.misc[0];
  int bi = s.imisc[0];
  for (int w = 1; w < kWaves; ++w)
    if (arg_better(s.misc[w], s.imisc[w], bv, bi)) {
      bv = s.misc[w];
      bi = s.imisc[w];
    }
  __syncthreads();
  v = bv;
  i = bi;
}

// LM head on this work-group's vocabulary rows; logits optionally written.
template <int DT>
__device__ KIE_INLINE bool st_lmhead(const Params* Pp, char* smem, uint32_t* X, float* logits, float& best_v,
                                     int& best_i) {
  const Sc c = stage_ctx(Pp, smem);
  const Params& P = c.P;
  const int d = P.d, V = P.V;
  const int v0 = split_lo(V, c.nb, c.wg), v1 = split_lo(V, c.nb, c.wg + 1);
  const int vpr = d >> 3;
  const int nwr = vpr >= 64 ? (vpr < kThreads ? vpr : kThreads) / 64 : 1;
  int cap = kRedCap / nwr;
  if (cap > kYCap) cap = kYCap;
  float bv = -INFINITY;
  int bi = 0x7FFFFFFF;
  for (int b0 = v0; b0 < v1 || b0 == v0; b0 += cap) {
    const int rows = min(cap, v1 - b0);
    auto rowptr = [&](int r) -> const uint16_t* { return P.lm_head + (size_t)(b0 + r) * d; };
    auto prep = [&]() -> bool {
      if (b0 != v0) return true;
      if (!poll_f32(X + P.xl.xout + (size_t)(P.L - 1) * d, d, c.s.xres, c.w, c.t)) return false;
      rmsnorm_to16<DT>(c.s.xres, P.final_norm, d, P.eps, c.s.xn, c.s.misc, c.t);
      return true;
    };
    if (!gemv_any<DT>(rows, d, rowptr, prep, c.s.xn, c.s.red, c.s.yv, c.t)) return false;
    for (int r = c.t; r < rows; r += kThreads) {
      const float y = c.s.yv[r];
      if (logits) logits[b0 + r] = y;
      if (arg_better(y, b0 + r, bv, bi)) {
        bv = y;
        bi = b0 + r;
      }
    }
    __syncthreads();
    if (rows <= 0) break;
  }
  block_argmax(bv, bi, c.s, c.t);
  best_v = bv;
  best_i = bi;
  return true;
}

// Reset this work-group's share of exchange set `Xr` to the NaN pattern.
// Set Xr was last used two steps ago; every work-group finished reading it
// before publishing its partial of the previous step, which this work-group
// has already consumed.
__device__ KIE_INLINE void reset_set(const Params* Pp, char* smem, uint32_t* Xr, int nch_prev) {
  const Sc c = stage_ctx(Pp, smem);
  const Params& P = c.P;
  const uint64_t sent2 = ~0ull;
  const uint64_t dense2 = P.xl.dense >> 1;  // in 8-byte units
  {
    const uint64_t a = dense2 * c.wg / c.nb, b = dense2 * (c.wg + 1) / c.nb;
    for (uint64_t k = a + c.t; k < b; k += kThreads) xst64(Xr + 2 * k, sent2);
  }
  if (nch_prev > 0) {
    const uint64_t per = (uint64_t)nch_prev * P.astride / 2;  // 8-byte units per (layer, head)
    const uint64_t blocks = (uint64_t)P.L * P.hq;
    const uint64_t tot = per * blocks;
    const uint64_t a = tot * c.wg / c.nb, b = tot * (c.wg + 1) / c.nb;
    uint32_t* att = Xr + P.xl.att;
    for (uint64_t k = a + c.t; k < b; k += kThreads) {
      const uint64_t blk = k / per, off = k % per;
      xst64(att + blk * (uint64_t)P.cmax * P.astride + 2 * off, sent2);
    }
  }
}

// Gather the per-work-group (max, index) partials -> the greedy token.  Every
// work-group reduces the same values in the same order, so all agree.
__device__ KIE_INLINE bool gather_token(const Params* Pp, char* smem, uint32_t* X, int& tok) {
  const Sc c = stage_ctx(Pp, smem);
  const Params& P = c.P;
  float gv = -INFINITY;
  int gi = 0x7FFFFFFF;
  bool ok = true;
  for (int w = c.t; w < c.nb; w += kThreads) {
    uint64_t v = 0;
    if (ok && poll64(X + P.xl.arg + 2 * w, v, c.w, Ready32x2{})) {
      const float vv = lo_f(v);
      const int vi = __float_as_int(hi_f(v));
      if (arg_better(vv, vi, gv, gi)) {
        gv = vv;
        gi = vi;
      }
    } else {
      ok = false;
    }
  }
  if (any_failed(!ok)) return false;
  block_argmax(gv, gi, c.s, c.t);
  // NaN logits never win a comparison: keep the index inside the vocabulary
  tok = (gi >= 0 && gi < P.V) ? gi : 0;
  return true;
}

// ---------------------------------------------------------------------------
// The persistent kernel
// ---------------------------------------------------------------------------
template <int DT, int G>
__global__ __launch_bounds__(kThreads, 1) void monokernel(const Params* __restrict__ Pp) {
  extern __shared__ __align__(16) char smem[];
  const int t = threadIdx.x, wg = blockIdx.x;
  const int n_steps = Pp->n_steps, L = Pp->L;
  int tok = Pp->in_tok;
  int done = 0;
  bool ok = true;
  for (int s = 0; s < n_steps && ok; ++s) {
    const Params& P = *opaque_s(Pp);
    const int pos = P.pos0 + s;
    if (P.forced) tok = P.forced[s];
    uint32_t* X = P.xch + (size_t)(s % kRingSets) * P.xl.words;
    {  // embedding row -> residual stream
      const Sc c = stage_ctx(Pp, smem);
      const uint16_t* er = c.P.tok_emb + (size_t)tok * c.P.d;
      for (int i = c.t; i < c.P.d; i += kThreads) c.s.xres[i] = to_f32<DT>(er[i]);
      __syncthreads();
    }
    for (int l = 0; l < L && ok; ++l) {
      ok = st_qkv<DT>(Pp, smem, l, X) && st_attn<DT, G>(Pp, smem, l, pos, X) &&
           st_merge<DT>(Pp, smem, l, pos, X) && st_wo<DT>(Pp, smem, l, X) && st_gateup<DT>(Pp, smem, l, X) &&
           st_down<DT>(Pp, smem, l, X);
    }
    if (!ok) break;
    float bv = 0.f;
    int bi = 0;
    {
      const Params& Q = *opaque_s(Pp);
      if (!Q.lm_last_only || s == Q.n_steps - 1) {
        float* lg = Q.logits ? Q.logits + (size_t)(Q.lm_last_only ? 0 : s) * Q.V : nullptr;
        if (!st_lmhead<DT>(Pp, smem, X, lg, bv, bi)) {
          ok = false;
          break;
        }
      }
    }
    // recycle the set used two steps ago, then publish this step's partial
    if (s >= 2) {
      int CL, nch;
      attn_chunking(*Pp, pos - 1, CL, nch);
      reset_set(Pp, smem, Pp->xch + (size_t)((s + 1) % kRingSets) * Pp->xl.words, nch);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (t == 0 && wg != Pp->withhold_wg) xst64(X + Pp->xl.arg + 2 * wg, pack2f(bv, __int_as_float(bi)));
    if (!gather_token(Pp, smem, X, tok)) {
      ok = false;
      break;
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (wg == 0 && t == 0) Pp->tok_out[s] = tok;
    done = s + 1;
    if (Pp->eos_id >= 0 && tok == Pp->eos_id) break;
    if (Pp->abort_after >= 0 && done >= Pp->abort_after && done < n_steps) {
      if (wg == 0 && t == 0) atomicCAS(Pp->ctl + CTL_STATUS, 0u, (uint32_t)(int32_t)KIE_ERR_ABORTED);
      break;
    }
  }
  if (wg == 0 && t == 0) {
    Pp->ctl[CTL_DONE] = (uint32_t)done;
    Pp->ctl[CTL_LAST] = (uint32_t)tok;
  }
}

// ---------------------------------------------------------------------------
// Isolated GEMV probe: y[i] = W[i % ncopy] x[i], rows split over the grid,
// one launch for all vectors.  Same engine as the decode stages.
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(kThreads, 1) void gemv_probe(const uint16_t* W, int rows, int cols, int ncopy,
                                                          const uint16_t* x, float* y, int nvec) {
  extern __shared__ __align__(16) char smem[];
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
  float* red = reinterpret_cast<float*>(smem + (size_t)cols * 2);
  float* yv = red + kRedCap;
  const int nb = gridDim.x, wg = blockIdx.x;
  const int r0 = split_lo(rows, nb, wg), r1 = split_lo(rows, nb, wg + 1);
  for (int iv = 0; iv < nvec; ++iv) {
    const int t = opaque_v((int)threadIdx.x);
    const uint16_t* Wc = W + (size_t)(iv % ncopy) * rows * cols;
    auto rowptr = [&](int r) -> const uint16_t* { return Wc + (size_t)(r0 + r) * cols; };
    auto prep = [&]() -> bool {
      const uint4* src = reinterpret_cast<const uint4*>(x + (size_t)iv * cols);
      for (int i = t; i < (cols >> 3); i += kThreads) reinterpret_cast<uint4*>(xs)[i] = src[i];
      __syncthreads();
      return true;
    };
    gemv_any<DT>(r1 - r0, cols, rowptr, prep, xs, red, yv, t);
    for (int r = t; r < r1 - r0; r += kThreads) y[(size_t)iv * rows + r0 + r] = yv[r];
    __syncthreads();
  }
}

}  // namespace kie
