// Device primitives of the monokernel: exchange-buffer access, NaN polling
// with a watchdog, wave reductions on DPP, dot2 products.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kie.h"
#include "kie_params.hpp"

namespace kie {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef __bf16 b2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Exchange memory.  Work-groups on different XCDs hand data over through
// buffers in HBM; each XCD has its own L2, and those L2s are not coherent with
// each other.  Every exchange word is therefore written and read with
// agent-scope relaxed atomics (global_store/global_load with sc1), which the
// memory model keeps coherent across the whole device.  The data is its own
// flag: a word still holding kSent (a NaN bit pattern) has not been written.
// ---------------------------------------------------------------------------
// Global (addrspace 1) views of generic pointers: global_load/global_store
// instead of flat accesses, whose counters the compiler must treat
// conservatively (a flat access may touch LDS).
#define KIE_GLOBAL __attribute__((address_space(1)))
template <class T>
__device__ __forceinline__ KIE_GLOBAL T* gptr(T* p) {
  return (KIE_GLOBAL T*)p;
}
template <class T>
__device__ __forceinline__ const KIE_GLOBAL T* gptr(const T* p) {
  return (const KIE_GLOBAL T*)p;
}

__device__ __forceinline__ uint64_t xld64(const uint32_t* p) {
  return __hip_atomic_load((KIE_GLOBAL uint64_t*)const_cast<uint32_t*>(p), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t xld32(const uint32_t* p) {
  return __hip_atomic_load((KIE_GLOBAL uint32_t*)const_cast<uint32_t*>(p), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void xst32(uint32_t* p, uint32_t v) {
  __hip_atomic_store((KIE_GLOBAL uint32_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void xst64(uint32_t* p, uint64_t v) {
  __hip_atomic_store((KIE_GLOBAL uint64_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t pack2f(float a, float b) {
  return (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32);
}
__device__ __forceinline__ float lo_f(uint64_t v) { return __uint_as_float((uint32_t)v); }
__device__ __forceinline__ float hi_f(uint64_t v) { return __uint_as_float((uint32_t)(v >> 32)); }

// fp32 payloads: a word equal to kSent is unwritten.
struct Ready32x2 {
  __device__ bool operator()(uint64_t v) const {
    return (uint32_t)v != kSent && (uint32_t)(v >> 32) != kSent;
  }
};
// 16-bit payloads (KV-cache rows): a half equal to 0xFFFF is unwritten.  A
// finite fp16/bf16 value never has that pattern (it is a NaN).
struct Ready16x4 {
  __device__ bool operator()(uint64_t v) const {
    const uint64_t x = ~v;  // unwritten halves become zero
    return ((x - 0x0001000100010001ull) & ~x & 0x8000800080008000ull) == 0;
  }
};

// Poll watchdog: a poll gives up after `limit` ticks of the 100 MHz real-time
// counter, or as soon as another work-group has recorded an error.
struct Watch {
  uint64_t limit;
  uint32_t* status;
  __device__ bool expired(uint64_t t0, int& n) const {
    if ((++n & 15) == 0 && xld32(status) != 0) return true;
    const uint64_t now = __builtin_amdgcn_s_memrealtime();
    if (now - t0 > limit) {
      atomicCAS(status, 0u, (uint32_t)(int32_t)KIE_ERR_TIMEOUT);
      return true;
    }
    return false;
  }
};

template <class Ready>
__device__ __forceinline__ bool poll64(const uint32_t* p, uint64_t& v, const Watch& w, Ready ready) {
  v = xld64(p);
  if (ready(v)) return true;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  int n = 0;
  for (;;) {
    __builtin_amdgcn_s_sleep(1);
    v = xld64(p);
    if (ready(v)) return true;
    if (w.expired(t0, n)) return false;
  }
}

// Philox4x32-10 block function (J. K. Salmon, M. A. Moraes, R. O. Dror, D. E.
// Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11): ten rounds; each
// multiplies counter words 0 and 2 by the two round constants and recombines
// the 64-bit products' halves with words 1, 3 and the key, which advances by
// the two Weyl constants before every round after the first.
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t hi0 = __umulhi(0xD2511F53u, c.x), lo0 = 0xD2511F53u * c.x;
    const uint32_t hi1 = __umulhi(0xCD9E8D57u, c.z), lo1 = 0xCD9E8D57u * c.z;
    c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
  }
  return c;
}

// ---------------------------------------------------------------------------
// Wave64 reductions on DPP (no LDS traffic).  dpp<CTRL, ROWMASK>(v) reads v
// from the lane that CTRL selects; rows outside ROWMASK receive 0.
// ---------------------------------------------------------------------------
template <int CTRL, int ROWMASK = 0xF>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWMASK, 0xF, false));
}
constexpr int DPP_QP_1032 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int DPP_QP_2301 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141;
constexpr int DPP_MIRROR = 0x140;
constexpr int DPP_BCAST15 = 0x142;
constexpr int DPP_BCAST31 = 0x143;

// Sum over aligned groups of 8 / 16 lanes; every lane receives its group sum.
__device__ __forceinline__ float sum8(float v) {
  v += dpp<DPP_QP_1032>(v);
  v += dpp<DPP_QP_2301>(v);
  v += dpp<DPP_HALF_MIRROR>(v);
  return v;
}
__device__ __forceinline__ float sum16(float v) {
  v = sum8(v);
  v += dpp<DPP_MIRROR>(v);
  return v;
}
// Sum over 32-lane halves: lane 31 holds lanes 0..31, lane 63 lanes 32..63.
__device__ __forceinline__ float sum32_tail(float v) {
  v = sum16(v);
  v += dpp<DPP_BCAST15, 0xA>(v);
  return v;
}
// Sum over the wave: lane 63 holds the total.
__device__ __forceinline__ float sum64_tail(float v) {
  v = sum32_tail(v);
  v += dpp<DPP_BCAST31, 0xC>(v);
  return v;
}
__device__ __forceinline__ float lane63(float v) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
// Max over the wave, returned to every lane.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<DPP_QP_1032>(v));
  v = fmaxf(v, dpp<DPP_QP_2301>(v));
  v = fmaxf(v, dpp<DPP_HALF_MIRROR>(v));
  v = fmaxf(v, dpp<DPP_MIRROR>(v));
  // rows 1 and 3 take the max with the previous row; rows 0/2 read 0 there,
  // so use shuffles for the cross-row part (max is not additive).
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) { return lane63(sum64_tail(v)); }

// ---------------------------------------------------------------------------
// Element conversion and dot2.  DT = KIE_F16 or KIE_BF16.
// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ float to_f32(uint32_t u16) {
  if constexpr (DT == KIE_F16) return (float)__builtin_bit_cast(_Float16, (uint16_t)u16);
  else return __uint_as_float(u16 << 16);
}
template <int DT>
__device__ __forceinline__ uint16_t to_16(float f) {
  if constexpr (DT == KIE_F16) return __builtin_bit_cast(uint16_t, (_Float16)f);
  else return __builtin_bit_cast(uint16_t, (__bf16)f);
}
template <int DT>
__device__ __forceinline__ uint32_t pack16(float a, float b) {
  return (uint32_t)to_16<DT>(a) | ((uint32_t)to_16<DT>(b) << 16);
}
// acc + sum of the 8 products of two 16-byte vectors, fp32 accumulation.
template <int DT>
__device__ __forceinline__ float dot8(const uint4& w, const uint4& x, float acc) {
  if constexpr (DT == KIE_F16) {
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, w.x), __builtin_bit_cast(h2_t, x.x), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, w.y), __builtin_bit_cast(h2_t, x.y), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, w.z), __builtin_bit_cast(h2_t, x.z), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, w.w), __builtin_bit_cast(h2_t, x.w), acc, false);
  } else {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2_t, w.x), __builtin_bit_cast(b2_t, x.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2_t, w.y), __builtin_bit_cast(b2_t, x.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2_t, w.z), __builtin_bit_cast(b2_t, x.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2_t, w.w), __builtin_bit_cast(b2_t, x.w), acc, false);
  }
  return acc;
}
// Activations fed to the dot2 unit sit in LDS as 16-byte vectors of 8
// elements.  fp16: vector k holds inputs 8k..8k+7.  bf16 keeps only 8
// significant bits, so an input x is stored as three bf16 terms
// x = b0 + b1 + b2 (b0 = bf16(x), b1 = bf16(x - b0), b2 = bf16(x - b0 - b1);
// each difference is exact in fp32): vector 3k holds the b0 of inputs
// 8k..8k+7, 3k+1 their b1, 3k+2 their b2.  Three dot2 passes then see every
// input to fp32 precision (the weights are exact), so a bf16 model's GEMVs
// are as accurate as fp32 ones.
template <int DT>
constexpr int kActWords = DT == KIE_BF16 ? 3 : 1;  // 16-byte vectors per 8 inputs

template <int DT>
__device__ __forceinline__ void act_terms(float v, uint16_t (&b)[kActWords<DT>]) {
  b[0] = to_16<DT>(v);
  if constexpr (kActWords<DT> > 1) {
    const float r1 = v - to_f32<DT>(b[0]);
    b[1] = to_16<DT>(r1);
    b[2] = to_16<DT>(r1 - to_f32<DT>(b[1]));
  }
}

template <int DT>
__device__ __forceinline__ void act_store(uint16_t* xs, int i, float v) {
  constexpr int AW = kActWords<DT>;
  uint16_t b[AW];
  act_terms<DT>(v, b);
  const int o = (i >> 3) * 8 * AW + (i & 7);
#pragma unroll
  for (int a = 0; a < AW; ++a) xs[o + 8 * a] = b[a];
}
// Inputs 2p and 2p+1.
template <int DT>
__device__ __forceinline__ void act_store2(uint16_t* xs, int p, float x0, float x1) {
  constexpr int AW = kActWords<DT>;
  uint16_t b0[AW], b1[AW];
  act_terms<DT>(x0, b0);
  act_terms<DT>(x1, b1);
  uint32_t* u = reinterpret_cast<uint32_t*>(xs);
  const int o = (p >> 2) * 4 * AW + (p & 3);
#pragma unroll
  for (int a = 0; a < AW; ++a) u[o + 4 * a] = (uint32_t)b0[a] | ((uint32_t)b1[a] << 16);
}

template <int DT>
__device__ __forceinline__ void unpack8(const uint4& v, float* f) {
  f[0] = to_f32<DT>(v.x & 0xFFFF); f[1] = to_f32<DT>(v.x >> 16);
  f[2] = to_f32<DT>(v.y & 0xFFFF); f[3] = to_f32<DT>(v.y >> 16);
  f[4] = to_f32<DT>(v.z & 0xFFFF); f[5] = to_f32<DT>(v.z >> 16);
  f[6] = to_f32<DT>(v.w & 0xFFFF); f[7] = to_f32<DT>(v.w >> 16);
}

// Weight stream load: one 16-byte vector per lane (global_load_dwordx4).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
// Non-temporal: streamed data (weights, KV rows) is not reused within a step,
// and the streaming hint measurably raises read bandwidth on this GPU.
__device__ __forceinline__ uint4 ldw(const uint16_t* p) {
  const u32x4_t v = __builtin_nontemporal_load((const KIE_GLOBAL u32x4_t*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

}  // namespace kie
