// GEMV tiling of the decode step: which weight rows each work-group streams
// and which 16-byte vectors each of its threads loads, in which order.
//
// Host and device share this code: the kernels use it to address the weight
// stream (each stage for itself, and the previous stage for its cross-stage
// prefetch), and the host runtime checks it (coverage and bounds) without a
// GPU.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "kie_params.hpp"

namespace kie {

// First of n items owned by part i of `parts` (balanced split).  32-bit: the
// host checks n * parts < 2^32 for every split it configures.
__host__ __device__ __forceinline__ int split_lo(int n, int parts, int i) {
  return (int)(((uint32_t)n * (uint32_t)i) / (uint32_t)parts);
}

__host__ __device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : v > hi ? hi : v; }

// GEMV stages in stream order.
enum : int { GS_QKV = 0, GS_WO = 1, GS_GATEUP = 2, GS_DOWN = 3, GS_LM = 4, GS_COUNT = 5 };
// Weight matrices a stage reads.
enum : int { M_Q = 0, M_K, M_V, M_O, M_GATE, M_UP, M_DOWN, M_LM, M_COUNT };

struct TileDims {
  int d, hq, hkv, hd, F, V;
};

// Output rows N and input width K of a stage.
__host__ __device__ __forceinline__ void stage_dims(const TileDims& D, int st, int& N, int& K) {
  switch (st) {
    case GS_QKV: N = (D.hq + 2 * D.hkv) * D.hd; K = D.d; break;
    case GS_WO: N = D.d; K = D.hq * D.hd; break;
    case GS_GATEUP: N = D.F; K = D.d; break;
    case GS_DOWN: N = D.d; K = D.F; break;
    default: N = D.V; K = D.d; break;
  }
}

// Rows matrix m has.
__host__ __device__ __forceinline__ int matrix_rows(const TileDims& D, int m) {
  switch (m) {
    case M_Q: return D.hq * D.hd;
    case M_K: case M_V: return D.hkv * D.hd;
    case M_O: case M_DOWN: return D.d;
    case M_GATE: case M_UP: return D.F;
    default: return D.V;
  }
}

// Lanes that read one row of vpr 16-byte vectors.  Rows of at least 64
// vectors are read by whole waves: the smallest multiple of 64 lanes (a power
// of two, at most the 512 threads) that leaves each lane at most 4 vectors of
// the row, so one lane reduction serves up to 4 vectors and the row a wave
// reads is wave-uniform.  Shorter rows (K = 256) take vpr lanes, two rows per
// wave.
__host__ __device__ __forceinline__ int lanes_per_row(int vpr) {
  if (vpr < 64) return vpr;
  int l = 64;
  while (l < kThreads && 4 * l < vpr) l <<= 1;
  return l;
}
// Vectors each lane reads per row, rounded up to 1, 2 or 4 (the GEMV width
// class; columns beyond the row are padding).
__host__ __device__ __forceinline__ int vectors_per_lane(int vpr) {
  const int l = lanes_per_row(vpr), v = (vpr + l - 1) / l;
  return v <= 1 ? 1 : v <= 2 ? 2 : 4;
}

// One thread's view of a work-group's rows in a GEMV stage.
//
// The work-group owns nrows local rows, made of up to three contiguous
// segments of weight matrices: local rows [0, n0) start at seg0, [n0, n01) at
// seg1, [n01, nrows) at seg2 (row stride K elements).  A row is read as K/8
// vectors of 8 elements by lpr = lanes_per_row(K/8) consecutive threads, each
// taking vpt = vectors_per_lane(K/8) vectors of it; rp = 512 / lpr rows are
// read per pass.  Thread t reads, for its j-th vector, local row
// (j / vpt) * rp + t / lpr and vector t % lpr + (j % vpt) * lpr of that row.
// Padding (rows beyond nrows, vectors beyond the row: the last pass, the ring
// and the column tail) reads row 0 and/or vector 0 instead; the caller
// discards it.
struct StagePlan {
  const uint16_t* seg0;
  const uint16_t* seg1;
  const uint16_t* seg2;
  int n0, n01, nrows, K, vpr, lpr, rp, vpt, sub, kl, nwr;

  __host__ __device__ __forceinline__ int passes() const { return (nrows + rp - 1) / rp; }

  __host__ __device__ __forceinline__ const uint16_t* row_vec(int row, int kv) const {
    if (row >= nrows) row = 0;
    if (kv >= vpr) kv = 0;
    const uint16_t* b = row < n0 ? seg0 + (size_t)row * K
                      : row < n01 ? seg1 + (size_t)(row - n0) * K : seg2 + (size_t)(row - n01) * K;
    return b + (size_t)kv * 8;
  }
  template <int VPT>
  __host__ __device__ __forceinline__ const uint16_t* addr(int j) const {
    const int p = j / VPT, i = j % VPT;
    return row_vec(p * rp + sub, kl + i * lpr);
  }
  __host__ __device__ __forceinline__ const uint16_t* addr(int j) const {
    const int p = j / vpt, i = j - p * vpt;
    return row_vec(p * rp + sub, kl + i * lpr);
  }
};

// Thread mapping for nrows rows of width K (segments set by the caller).
__host__ __device__ __forceinline__ StagePlan plan_rows(int nrows, int K, int t) {
  StagePlan g{};
  g.nrows = nrows;
  g.K = K;
  g.vpr = K >> 3;
  g.lpr = lanes_per_row(g.vpr);
  g.rp = kThreads / g.lpr;
  g.vpt = vectors_per_lane(g.vpr);
  g.sub = t / g.lpr;
  g.kl = t % g.lpr;
  g.nwr = g.lpr >= 64 ? g.lpr / 64 : 1;
  g.n0 = g.n01 = nrows;
  return g;
}

// Plan of GEMV stage `st` for work-group wg of nb, thread t; mats[m] = base of
// weight matrix m (row-major, K elements per row).
//   QKV:     rows [r0, r1) of the stack [Wq; Wk; Wv]
//   WO:      rows [r0, r1) of Wo        DOWN: rows [r0, r1) of W_down
//   GATEUP:  gate rows [r0, r1), then up rows [r0, r1)  (2 (r1 - r0) local rows)
//   LM:      rows [r0, r1) of the LM head
// with [r0, r1) = split of the stage's N output rows over nb work-groups.
__host__ __device__ __forceinline__ StagePlan make_stage_plan(const TileDims& D, int st, int wg, int nb, int t,
                                                              const uint16_t* const* mats) {
  int N, K;
  stage_dims(D, st, N, K);
  const int r0 = split_lo(N, nb, wg), r1 = split_lo(N, nb, wg + 1);
  const int n = r1 - r0;
  StagePlan g = plan_rows(st == GS_GATEUP ? 2 * n : n, K, t);
  const size_t Ks = (size_t)K;
  switch (st) {
    case GS_QKV: {
      const int nq = D.hq * D.hd, nk = D.hkv * D.hd;
      const int a = clampi(nq - r0, 0, n), b = clampi(nq + nk - r0, 0, n);
      g.n0 = a;
      g.n01 = b;
      // local row r >= a maps to Wk row r0 + r - nq, r >= b to Wv row r0 + r - nq - nk
      g.seg0 = mats[M_Q] + (size_t)r0 * Ks;
      g.seg1 = mats[M_K] + (size_t)clampi(r0 + a - nq, 0, r0 + a) * Ks;
      g.seg2 = mats[M_V] + (size_t)clampi(r0 + b - nq - nk, 0, r0 + b) * Ks;
      break;
    }
    case GS_WO: g.seg0 = mats[M_O] + (size_t)r0 * Ks; break;
    case GS_GATEUP:
      g.n0 = n;
      g.n01 = 2 * n;
      g.seg0 = mats[M_GATE] + (size_t)r0 * Ks;
      g.seg1 = mats[M_UP] + (size_t)r0 * Ks;
      break;
    case GS_DOWN: g.seg0 = mats[M_DOWN] + (size_t)r0 * Ks; break;
    default: g.seg0 = mats[M_LM] + (size_t)r0 * Ks; break;
  }
  return g;
}

}  // namespace kie
