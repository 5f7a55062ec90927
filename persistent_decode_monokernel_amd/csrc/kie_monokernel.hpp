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
//   LM head:  logits rows, per-work-group (max, index) partial (and, when
//             sampling, the work-group's 64 best rows as a sorted list)
//   argmax:   every work-group reduces all partials -> same next token; EOS test
//   sampling: (instead of the argmax token) work-groups 0..31 merge groups of
//             8 lists, work-group 0 merges the groups, draws and publishes
//             the token, the others poll it
//
// Code-generation note.  All stages are inlined into one kernel.  Each stage
// re-derives the thread index and the parameter pointer through an empty asm
// statement (opaque_*), so the compiler cannot hoist per-stage address
// arithmetic out of the layer loop and keep it live across all stages.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kie_device.hpp"
#include "kie_tiling.hpp"

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

// The launch parameters are read through the constant address space: they
// do not change during a launch, so every field read is a scalar load (scalar
// data cache, lgkmcnt) instead of a vector-memory load whose wait would also
// wait for the weight vectors already in flight.
typedef const __attribute__((address_space(4))) Params CParams;
__device__ __forceinline__ CParams& cparams(const Params* Pp) { return *(CParams*)opaque_s(Pp); }

// Timeline stamp k of a slot, by thread `who` of the work-group (only on the
// traced step).  k: 0 entry, 1 input arrived, 2 compute done, 3 exit.  tr is
// this work-group's row of the trace (work-group-major layout, so no grid
// size is needed here: reading gridDim is a vector-memory load of the
// dispatch packet, and waiting for it would also wait for every weight load
// in flight).
__device__ __forceinline__ void stamp(uint64_t* tr, int slot, int k, int t, int who = 0) {
  if (tr && t == who) tr[(size_t)slot * kTraceStamps + k] = __builtin_amdgcn_s_memrealtime();
}

// Wait until every store this thread issued has been performed.  Exchange and
// KV-cache stores are agent-scope (sc1, written through to memory), so once
// they are acknowledged any later publication is ordered after them for every
// other work-group; no cache write-back is needed (a release fence would write
// back this XCD's whole L2).
__device__ __forceinline__ void drain_stores() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt/lgkmcnt unconstrained
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Race test: the chosen work-group holds back every hand-off publication by
// a fixed time (the host sets it), so consumers see its words arrive late.
__device__ __forceinline__ void publish_delay(CParams& P) {
  if ((int)blockIdx.x == P.delay_wg) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (__builtin_amdgcn_s_memrealtime() - t0 < P.delay_ticks) __builtin_amdgcn_s_sleep(2);
  }
}

// The ring's first kRingSplit slots of a GEMV stage are issued ahead of the
// stage's input poll (by the previous stage, or the stage's prologue); the
// other slots right after the poll's loads, before its result is awaited.
// Loads return in issue order, so a poll issued behind the whole ring waits
// for all of it; issued behind part of it, the poll returns sooner while the
// rest of the ring keeps the weight stream going.
#ifndef KIE_RING_SPLIT
#define KIE_RING_SPLIT KIE_DEPTH
#endif
constexpr int kRingSplit = KIE_RING_SPLIT;
static_assert(kRingSplit >= 1 && kRingSplit <= kDepth, "ring split");

// Slots issued ahead of a stage's poll for a GEMV of width class VC (rows of
// at least 512 columns: kRingSplit; the narrow rows of small models keep the
// whole ring ahead -- the compiler crashed on the split form of those).
template <int VC>
constexpr int ring_split() { return VC > 0 ? kRingSplit : kDepth; }
// Issue the first RS vectors of the next GEMV stage into the ring.
template <int RS>
__device__ __forceinline__ void ring_prefetch(uint4 (&ring)[kDepth], const StagePlan& np);

// ---------------------------------------------------------------------------
// LDS view
// ---------------------------------------------------------------------------
struct Lds {
  float* xres;     // fp32 residual stream copy [d]
  uint16_t* xn;    // 16-bit activation fed to dot2 [Kmax] (bf16: three terms, see act_store)
  float* red;      // GEMV per-wave partial sums [kRedCap]
  float* yv;       // GEMV finished rows [kYCap]
  float* scr;      // aliases red/yv
  float* att;      // attention scratch: aliases xn and red/yv (both idle from the end of the
                   // QKV GEMV to the Wo poll)
  float* misc;     // 64 floats: block reductions
  int* imisc;      // 64 ints
};

__device__ __forceinline__ Lds lds_view(char* smem, CParams& P) {
  Lds s;
  s.xres = reinterpret_cast<float*>(smem + P.lds_xres);
  s.xn = reinterpret_cast<uint16_t*>(smem + P.lds_xn);
  s.red = reinterpret_cast<float*>(smem + P.lds_scr);
  s.yv = s.red + kRedCap;
  s.scr = s.red;
  s.att = reinterpret_cast<float*>(smem + P.lds_xn);
  s.misc = reinterpret_cast<float*>(smem + P.lds_misc);
  s.imisc = reinterpret_cast<int*>(s.misc + 64);
  return s;
}

// Per-stage context: everything re-derived at stage entry (see note above).
struct Sc {
  CParams& P;
  Lds s;
  Watch w;
  int t, wg, nb;
};

__device__ __forceinline__ Sc stage_ctx(const Params* Pp, char* smem) {
  CParams& P = cparams(Pp);
  return Sc{P, lds_view(smem, P), Watch{P.timeout, P.ctl + CTL_STATUS}, opaque_v((int)threadIdx.x),
            (int)blockIdx.x, P.grid};  // the grid from the parameters: a scalar load (see stamp)
}

// Work-group-wide "any thread failed" with a barrier.
__device__ __forceinline__ bool any_failed(bool failed) { return __syncthreads_or(failed ? 1 : 0) != 0; }

// Arrival-counter hand-off: the comparison protocol, compiled in only for the
// kernel instances built with HO = true (both functions are empty otherwise).
// Counter k of an exchange set starts at kSent like every other word; each
// work-group adds one once all its outputs of stage k are performed, so the
// counter reads kSent + grid when every work-group has arrived.
template <bool HO>
__device__ __forceinline__ void arrive(CParams& P, uint32_t* X, int k, int t) {
  if constexpr (!HO) return;
  drain_stores();
  __syncthreads();
  if (t == 0)
    __hip_atomic_fetch_add((KIE_GLOBAL uint32_t*)(X + P.xl.cnt + k), 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
// Wait (thread 0 polls, the work-group follows) until every work-group has
// arrived at counter k.  Ends with a barrier in counter mode.
template <bool HO>
__device__ __forceinline__ bool await_all(CParams& P, uint32_t* X, int k, const Watch& w, int t) {
  if constexpr (!HO) return true;
  bool ok = true;
  if (t == 0) {
    const uint32_t* p = X + P.xl.cnt + k;
    const uint32_t want = kSent + (uint32_t)P.grid;
    if (xld32(p) != want) {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      int n = 0;
      for (;;) {
        __builtin_amdgcn_s_sleep(1);
        if (xld32(p) == want) break;
        if (w.expired(t0, n)) {
          ok = false;
          break;
        }
      }
    }
  }
  return !any_failed(!ok);
}

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
// Batched poll of nw 8-byte exchange words src[2i..2i+1], i < nw, spread over
// the work-group (word i on thread i % 512).  Each thread issues the loads of
// a batch of its words at once and waits once, then re-polls only the words
// that were not written yet, so a vector costs about one memory round trip
// instead of one per word.  store(i, v) receives every word once.  Ends with a
// barrier; false if a poll expired.
//
// The first batch holds NB words per thread and is issued unconditionally
// (a thread past the vector re-reads its first word) and outside any loop, and
// it is first looked at outside the re-poll loop.  The compiler's waits for
// loaded registers are only exact on straight-line code: with the loads under
// branches or in a loop it waited, before each load and before the first
// look, for every older load -- the next GEMV stage's weight vectors
// included, also those that after() issues behind the batch.
constexpr int kPollBatch = 8;
constexpr int kPollD = 4;  // first batch of model-width vectors: d <= 4096 floats = 4 words per thread
struct NoAfter {
  __device__ void operator()() const {}
};
// Re-poll the words of mask `again` until all are written.
template <int NB, class Ready, class Store>
__device__ __forceinline__ bool repoll(const uint32_t* src, int base, uint32_t again, uint64_t (&v)[NB],
                                       const Watch& w, Ready ready, Store store) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  int n = 0;
  for (;;) {
    __builtin_amdgcn_s_sleep(1);
#pragma unroll
    for (int k = 0; k < NB; ++k)
      if (again & (1u << k)) v[k] = xld64(src + 2 * (size_t)(base + k * kThreads));
    __builtin_amdgcn_sched_barrier(0);
    const uint32_t pending = again;
    again = 0;
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      if (pending & (1u << k)) {
        if (ready(v[k])) store(base + k * kThreads, v[k]);
        else again |= 1u << k;
      }
    }
    if (!again) return true;
    if (w.expired(t0, n)) return false;
  }
}
// First batch: words t + k * 512, k < NB; after() runs once the loads are issued.
template <int NB, class Ready, class Store, class After>
__device__ __forceinline__ bool poll_first(const uint32_t* src, int nw, int t, const Watch& w, Ready ready,
                                           Store store, After after) {
  uint64_t v[NB];
  uint32_t pending = 0;
  const int own = t < nw ? t : 0;
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    const int i = t + k * kThreads;
    v[k] = xld64(src + 2 * (size_t)(i < nw ? i : own));
    pending |= (i < nw ? 1u : 0u) << k;
  }
  __builtin_amdgcn_sched_barrier(0);  // every load of the batch issued before any look
  after();
  __builtin_amdgcn_sched_barrier(0);
  uint32_t again = 0;
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    if (pending & (1u << k)) {
      if (ready(v[k])) store(t + k * kThreads, v[k]);
      else again |= 1u << k;
    }
  }
  return !again || repoll<NB>(src, t, again, v, w, ready, store);
}
// Later batches (vectors beyond NB * 512 words): words base + k * 512.  Which
// loads a wave issues is decided on the wave's first word (a scalar branch;
// every vector length is a multiple of 64 words).
template <class Ready, class Store>
__device__ __forceinline__ bool poll_batch(const uint32_t* src, int nw, int base, const Watch& w, Ready ready,
                                           Store store) {
  uint64_t v[kPollBatch];
  uint32_t pending = 0;
  const int b0 = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
  for (int k = 0; k < kPollBatch; ++k) {
    const int i = base + k * kThreads;
    if (b0 + k * kThreads < nw) {
      v[k] = xld64(src + 2 * (size_t)(i < nw ? i : 0));
      pending |= (i < nw ? 1u : 0u) << k;
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  uint32_t again = 0;
#pragma unroll
  for (int k = 0; k < kPollBatch; ++k) {
    if (pending & (1u << k)) {
      if (ready(v[k])) store(base + k * kThreads, v[k]);
      else again |= 1u << k;
    }
  }
  return !again || repoll<kPollBatch>(src, base, again, v, w, ready, store);
}
template <int NB = kPollBatch, class Ready, class Store, class After = NoAfter>
__device__ __forceinline__ bool poll_words(const uint32_t* src, int nw, const Watch& w, int t, Ready ready,
                                           Store store, After after = NoAfter{}) {
  static_assert(NB >= 1 && NB <= 32, "first poll batch");
  bool ok = poll_first<NB>(src, nw, t, w, ready, store, after);
  for (int base = t + NB * kThreads; base < nw && ok; base += kPollBatch * kThreads)
    ok = poll_batch(src, nw, base, w, ready, store);
  return !any_failed(!ok);
}
// Poll n fp32 words (n even) of an exchange buffer into LDS as fp32.
// NB: words per thread of the first batch (see poll_words).
template <int NB = kPollBatch, class After = NoAfter>
__device__ __forceinline__ bool poll_f32(const uint32_t* src, int n, float* dst, const Watch& w, int t,
                                         After after = NoAfter{}) {
  return poll_words<NB>(
      src, n >> 1, w, t, Ready32x2{},
      [&](int i, uint64_t v) {
        dst[2 * i] = lo_f(v);
        dst[2 * i + 1] = hi_f(v);
      },
      after);
}
// Poll n fp32 words into LDS as 16-bit activations.
template <int DT, int NB = kPollBatch, class After = NoAfter>
__device__ __forceinline__ bool poll_to16(const uint32_t* src, int n, uint16_t* dst, const Watch& w, int t,
                                          After after = NoAfter{}) {
  return poll_words<NB>(
      src, n >> 1, w, t, Ready32x2{}, [&](int i, uint64_t v) { act_store2<DT>(dst, i, lo_f(v), hi_f(v)); }, after);
}
// The RMSNorm gains of this thread's elements t + k * 512 (n <= 4096), read
// before the stage's poll: issued after it, they cost one more memory round
// trip on the hand-off's critical path.  The loads are unconditional (a lane
// past n re-reads element 0) and fenced from the code that uses them: under a
// branch the compiler converted each value right after its load, waiting for
// it and for every older load.
constexpr int kGainRegs = 8;
struct Gains {
  uint32_t v[kGainRegs];  // one 16-bit gain each
};
__device__ __forceinline__ Gains load_gains(const uint16_t* g, int n, int t) {
  Gains r;
#pragma unroll
  for (int k = 0; k < kGainRegs; ++k) {
    const int i = t + k * kThreads;
    r.v[k] = g[i < n ? i : 0];
  }
  __builtin_amdgcn_sched_barrier(0);
  return r;
}
// xn = RMSNorm(x) * g, rounded to 16 bits, with g from load_gains.  Ends with a barrier.
template <int DT>
__device__ __forceinline__ void rmsnorm_to16(const float* x, const Gains& g, int n, float eps, uint16_t* xn,
                                             float* misc, int t) {
  float ss = 0.f;
  for (int i = t; i < n; i += kThreads) ss += x[i] * x[i];
  ss = block_sum(ss, misc, t);
  const float r = 1.0f / sqrtf(ss / (float)n + eps);
#pragma unroll
  for (int k = 0; k < kGainRegs; ++k) {
    const int i = t + k * kThreads;
    if (i < n) act_store<DT>(xn, i, x[i] * r * to_f32<DT>((uint16_t)g.v[k]));
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// GEMV engine.
//
// A work-group owns `nrows` rows of K columns (StagePlan, kie_tiling.hpp).
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
// Reduce one row-partial over the lanes of its row and park it in LDS.
// WIDE: a row spans >= 64 lanes (K >= 512); else 32 lanes (K = 256).
template <bool WIDE>
__device__ __forceinline__ void gv_park(float acc, int p, const StagePlan& g, float* red, int t) {
  const int row = p * g.rp + g.sub;
  if constexpr (WIDE) {
    acc = sum64_tail(acc);
    if ((t & 63) == 63 && row < g.nrows) red[row * g.nwr + (g.kl >> 6)] = acc;
  } else {  // two rows per wave
    acc = sum32_tail(acc);
    if ((t & 31) == 31 && row < g.nrows) red[row] = acc;
  }
}

// Weight-vector addressing for tilings whose rows span whole waves (K >= 512):
// the row a wave reads is wave-uniform, so the row's address (segment select,
// row * K) is scalar arithmetic and each lane only adds its fixed byte offset
// within the row -- no per-vector vector-ALU address work.  Same mapping as
// StagePlan::addr (the host checks that one).
struct WideRows {
  // Row r (local) of the work-group lives at b0 + r * rb, plus d1 once r >=
  // n0 and d2 once r >= n01 (the later segments' bases, shifted by their first
  // local row; plain integers, so the select stays arithmetic on registers).
  uint64_t b0, d1, d2;
  int n0, n01, nrows, rp, sub, vsh;
  uint32_t rb;      // bytes per row
  uint32_t lo[4];   // this lane's byte offset of its vector i of a row (padding columns: 0)
  __device__ __forceinline__ const char* row(int r) const {
    r = r < nrows ? r : 0;
    const uint64_t m1 = r >= n0 ? ~0ull : 0ull, m2 = r >= n01 ? ~0ull : 0ull;
    return reinterpret_cast<const char*>(b0 + (m1 & d1) + (m2 & d2) + (uint64_t)(uint32_t)r * rb);
  }
  // vector i of the row read in pass p
  __device__ __forceinline__ uint4 load(int p, int i) const {
    return ldw(reinterpret_cast<const uint16_t*>(row(p * rp + sub) + lo[i]));
  }
  // j-th vector with the vectors-per-row of the plan (runtime)
  __device__ __forceinline__ uint4 load_j(int j) const {
    const int i = j & ((1 << vsh) - 1);
    const uint32_t o = i == 0 ? lo[0] : i == 1 ? lo[1] : i == 2 ? lo[2] : lo[3];
    return ldw(reinterpret_cast<const uint16_t*>(row((j >> vsh) * rp + sub) + o));
  }
};

// The plan's row fields are work-group uniform, but part of them comes out of
// vector-ALU integer division; reading them back with readfirstlane keeps the
// row arithmetic on the scalar unit.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ const char* uni(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const char*>((hi << 32) | lo);
}

__device__ __forceinline__ WideRows wide_rows(const StagePlan& g) {
  WideRows w;
  w.n0 = uni(g.n0);
  w.n01 = uni(g.n01);
  w.nrows = uni(g.nrows);
  w.rp = uni(g.rp);
  w.sub = uni(g.sub);  // lanes_per_row >= 64: uniform over the wave
  w.vsh = uni(g.vpt == 1 ? 0 : g.vpt == 2 ? 1 : 2);
  w.rb = (uint32_t)uni(g.K * 2);
  const uint64_t b0 = reinterpret_cast<uint64_t>(uni(g.seg0));
  const uint64_t b1 = reinterpret_cast<uint64_t>(uni(g.seg1)) - (uint64_t)(uint32_t)w.n0 * w.rb;
  const uint64_t b2 = reinterpret_cast<uint64_t>(uni(g.seg2)) - (uint64_t)(uint32_t)w.n01 * w.rb;
  w.b0 = b0;
  w.d1 = b1 - b0;
  w.d2 = b2 - b1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int kv = g.kl + i * g.lpr;
    w.lo[i] = (i < g.vpt && kv < g.vpr) ? (uint32_t)kv * 16u : 0u;
  }
  return w;
}

// j-th vector of any plan (the next stage's prefetch)
__device__ __forceinline__ uint4 plan_load(const StagePlan& g, const WideRows& w, int j) {
  return g.lpr >= 64 ? w.load_j(j) : ldw(g.addr(j));
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
//
// The ring is shared by consecutive GEMV stages: with `prefilled` the
// previous stage already issued this stage's first kDepth vectors, and while
// this stage drains its last block it issues the first kDepth vectors of the
// next GEMV stage (next(i) = address of that stage's vector i, or nullptr when
// there is none), so the weight stream does not stop at the hand-off.
// RS: ring slots issued ahead of prep (the decode stages: kRingSplit; the
// GEMV probe: all of them).
template <int DT, int VPT, bool WIDE, class Prep, int RS = kRingSplit>
__device__ __forceinline__ bool gemv(const StagePlan& g, Prep prep, const uint16_t* xs, float* red, float* yv, int t,
                                     uint4 (&ring)[kDepth], bool prefilled, const StagePlan next, uint64_t* tr,
                                     int slot) {
  const int J = g.passes() * VPT;
  const int Jp = (J + kDepth - 1) / kDepth * kDepth;
  static_assert(kDepth % VPT == 0, "ring blocks hold whole rows");
  const WideRows wr = WIDE ? wide_rows(g) : WideRows{};
  // vector j = pj * VPT + i of this stage
  auto wload = [&](int pj, int i) -> uint4 {
    if constexpr (WIDE) return wr.load(pj, i);
    else return ldw(g.addr<VPT>(pj * VPT + i));
  };
  const bool any = uni(Jp) > 0;
  if (any && !prefilled) {
#pragma unroll
    for (int i = 0; i < RS; ++i) ring[i] = wload(i / VPT, i % VPT);
  }
  // prep(fill) must call fill() once: it issues the ring's other slots.  No
  // branch around them (every work-group owns rows of every GEMV stage: the
  // host keeps the grid within d_model, d_ffn and the vocabulary), so the
  // compiler's wait for the poll before them stays exact.
  auto fill = [&]() {
#pragma unroll
    for (int i = RS; i < kDepth; ++i) ring[i] = wload(i / VPT, i % VPT);
  };
  if (!prep(fill)) return false;
  const bool has_next = next.nrows > 0;
  if (Jp > 0) {
    constexpr int AW = kActWords<DT>;
    uint4 xr[AW][VPT];  // the input vectors (bf16: all three terms) this thread multiplies
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int kv = g.kl + i * g.lpr;
      const uint4* v = reinterpret_cast<const uint4*>(xs) + kv * AW;
#pragma unroll
      for (int a = 0; a < AW; ++a) xr[a][i] = kv < g.vpr ? v[a] : make_uint4(0, 0, 0, 0);
    }
    auto dot = [&](const uint4& w, int i, float acc) {
#pragma unroll
      for (int a = AW - 1; a >= 0; --a) acc = dot8<DT>(w, xr[a][i % VPT], acc);  // small terms first
      return acc;
    };
    float acc = 0.f;
    int j0 = 0;
    for (; j0 + kDepth < Jp; j0 += kDepth) {
      const int p0 = (j0 + kDepth) / VPT;
#pragma unroll
      for (int i = 0; i < kDepth; ++i) {
        acc = dot(ring[i], i, acc);
        ring[i] = wload(p0 + i / VPT, i % VPT);
        if (i % VPT == VPT - 1) {
          gv_park<WIDE>(acc, (j0 + i) / VPT, g, red, t);
          acc = 0.f;
        }
      }
    }
    if (has_next) {
      const WideRows nw = next.lpr >= 64 ? wide_rows(next) : WideRows{};
#pragma unroll
      for (int i = 0; i < kDepth; ++i) {  // last block: drain, refill with the next stage
        acc = dot(ring[i], i, acc);
        if (i < RS) ring[i] = plan_load(next, nw, i);
        if (i % VPT == VPT - 1) {
          gv_park<WIDE>(acc, (j0 + i) / VPT, g, red, t);
          acc = 0.f;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < kDepth; ++i) {  // last block: drain
        acc = dot(ring[i], i, acc);
        if (i % VPT == VPT - 1) {
          gv_park<WIDE>(acc, (j0 + i) / VPT, g, red, t);
          acc = 0.f;
        }
      }
    }
  } else if (has_next) {
    const WideRows nw = next.lpr >= 64 ? wide_rows(next) : WideRows{};
#pragma unroll
    for (int i = 0; i < RS; ++i) ring[i] = plan_load(next, nw, i);
  }
  stamp(tr, slot, 2, t);
  __syncthreads();
  for (int r = t; r < g.nrows; r += kThreads) {
    float y = 0.f;
    for (int w = 0; w < g.nwr; ++w) y += red[r * g.nwr + w];
    yv[r] = y;
  }
  __syncthreads();
  return true;
}

template <int RS>
__device__ __forceinline__ void ring_prefetch(uint4 (&ring)[kDepth], const StagePlan& np) {
  if (np.nrows > 0) {
    const WideRows nw = np.lpr >= 64 ? wide_rows(np) : WideRows{};
#pragma unroll
    for (int i = 0; i < RS; ++i) ring[i] = plan_load(np, nw, i);
  }
}

// GEMV of a width class fixed at compile time: VC = 0 for K < 512 (rows of
// 32 lanes), else the vectors per thread per row (1, 2 or 4).
template <int DT, int VC, class Prep>
__device__ __forceinline__ bool gemv_cls(const StagePlan& g, Prep prep, const uint16_t* xs, float* red, float* yv,
                                         int t, uint4 (&ring)[kDepth], bool prefilled, uint64_t* tr, int slot) {
  return gemv<DT, (VC > 0 ? VC : 1), (VC > 0), Prep, ring_split<VC>()>(g, prep, xs, red, yv, t, ring, prefilled,
                                                                       StagePlan{}, tr, slot);
}

template <int DT, int RS = kDepth, class Prep>
__device__ __forceinline__ bool gemv_any(const StagePlan& g, Prep prep, const uint16_t* xs, float* red, float* yv,
                                         int t, uint4 (&ring)[kDepth], bool prefilled, const StagePlan next,
                                         uint64_t* tr = nullptr, int slot = 0) {
  // rows narrower than 512 columns keep the whole ring ahead (the compiler crashed on their split form)
  if (g.vpr < 64) return gemv<DT, 1, false, Prep, kDepth>(g, prep, xs, red, yv, t, ring, prefilled, next, tr, slot);
  if (g.vpt == 1) return gemv<DT, 1, true, Prep, RS>(g, prep, xs, red, yv, t, ring, prefilled, next, tr, slot);
  if (g.vpt == 2) return gemv<DT, 2, true, Prep, RS>(g, prep, xs, red, yv, t, ring, prefilled, next, tr, slot);
  return gemv<DT, 4, true, Prep, RS>(g, prep, xs, red, yv, t, ring, prefilled, next, tr, slot);
}


__device__ __forceinline__ const uint16_t* lw_ptr(CParams& P, int l, int k) {
  typedef const uint16_t* wptr;  // the weight table does not change during a launch either
  const __attribute__((address_space(4))) wptr* tab = (const __attribute__((address_space(4))) wptr*)P.lw;
  return tab[l * W_PER_LAYER + k];
}

// ---------------------------------------------------------------------------
// Stages
// ---------------------------------------------------------------------------

// The plan of GEMV stage `st` of layer l for this thread (tiling in
// kie_tiling.hpp; matrix bases from the weight-pointer table).
__device__ __forceinline__ StagePlan plan_stage(CParams& P, int l, int st, int t, int wg, int nb) {
  const TileDims D{P.d, P.hq, P.hkv, P.hd, P.F, P.V};
  const uint16_t* mats[M_COUNT] = {lw_ptr(P, l, W_Q),    lw_ptr(P, l, W_K),    lw_ptr(P, l, W_V),
                                   lw_ptr(P, l, W_O),    lw_ptr(P, l, W_GATE), lw_ptr(P, l, W_UP),
                                   lw_ptr(P, l, W_DOWN), P.lm_head};
  return make_stage_plan(D, st, wg, nb, t, mats);
}

// QKV projection: rows [r0, r1) of the stacked [Wq; Wk; Wv] (contiguous row
// segments of the three matrices), published unrotated in fp32.  Input x_l:
// LDS xres (layer 0: the embedding) or polled from the previous layer's xout.
template <int DT, int VD, bool HO>
__device__ KIE_INLINE bool st_qkv(const Params* Pp, char* smem, int l, uint32_t* X, uint64_t* tr, uint4 (&ring)[kDepth]) {
  const Sc c = stage_ctx(Pp, smem);
  CParams& P = c.P;
  const int slot = l * kStagesPerLayer + 0;
  stamp(tr, slot, 0, c.t);
  const int hd = P.hd, d = P.d;
  const int nq = P.hq * hd, nk = P.hkv * hd;
  const int N = nq + 2 * nk;
  const int r0 = split_lo(N, c.nb, c.wg), r1 = split_lo(N, c.nb, c.wg + 1);
  const StagePlan pl = plan_stage(P, l, GS_QKV, c.t, c.wg, c.nb);
  auto prep = [&](auto fill) -> bool {
    const Gains gn = load_gains(lw_ptr(P, l, W_ATTN_NORM), d, c.t);
    if (l == 0) fill();  // the embedding row is already in LDS
    if (l > 0 && !await_all<HO>(P, X, (l - 1) * kStagesPerLayer + 5, c.w, c.t)) return false;
    if (l > 0 && !poll_f32<kPollD>(X + P.xl.xout + (size_t)(l - 1) * d, d, c.s.xres, c.w, c.t, fill)) return false;
    rmsnorm_to16<DT>(c.s.xres, gn, d, P.eps, c.s.xn, c.s.misc, c.t);
    stamp(tr, slot, 1, c.t);
    return true;
  };
  if (!gemv_cls<DT, VD>(pl, prep, c.s.xn, c.s.red, c.s.yv, c.t, ring, l > 0, tr, slot)) return false;
  uint32_t* dst = X + P.xl.qkv + (size_t)l * N;
  publish_delay(P);
  for (int r = c.t; r < r1 - r0; r += kThreads) xst32(dst + r0 + r, __float_as_uint(c.s.yv[r]));
  arrive<HO>(P, X, l * kStagesPerLayer + 0, c.t);
  stamp(tr, slot, 3, c.t);
  return true;
}

__device__ __forceinline__ void attn_chunking(CParams& P, int n, int& CL, int& nch) {
  CL = (n + P.cmax - 1) / P.cmax;
  if (CL < kClMin) CL = kClMin;
  nch = (n + CL - 1) / CL;
}

// Online-softmax state update with one more score s and value row v:
// (m, l, o) -> (max(m, s), l e^(m-m') + e^(s-m'), o e^(m-m') + e^(s-m') v).
// Softmax statistics are kept in base 2: scores are scaled by log2(e)/sqrt(hd)
// so that exp(s - m) = exp2(s' - m'), one v_exp_f32 (about 1 ulp).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float safe_exp_diff(float a, float m) { return a == -INFINITY ? 0.f : fast_exp2(a - m); }

// Split-KV attention (flash-decoding): unit (KV head g, chunk c) computes, for
// the G query heads that read head g, the partial softmax statistics over the
// chunk's positions: m = max score, l = sum exp(s - m), o = sum exp(s - m) v
// (m kept in base-2 units, see fast_exp2).
// Rotary embedding of q and of the new k happens in registers right after the
// poll; the unit whose chunk holds the current position also appends the
// (rotated k, v) row to the KV cache.  Positions are spread over lane groups
// of hd/8 lanes (8 dimensions per lane, one position per group and pass).
// Each group keeps the online-softmax state of up to four heads at once, so a
// K/V row is read once for all of them; the groups' states then meet once in
// LDS, one thread per (head, dimension) folding them.
template <int DT, int G, bool HO>
__device__ KIE_INLINE bool st_attn(const Params* Pp, char* smem, int l, int pos, uint32_t* X, uint64_t* tr) {
  const Sc c = stage_ctx(Pp, smem);
  CParams& P = c.P;
  const int slot = l * kStagesPerLayer + 1;
  stamp(tr, slot, 0, c.t);
  const int t = c.t;
  const int hd = P.hd, hkv = P.hkv, hq = P.hq;
  const int half = hd >> 1, qd4 = hd >> 2;
  const int N = (hq + 2 * hkv) * hd;
  const int n = pos + 1;
  int CL, nch;
  attn_chunking(P, n, CL, nch);
  const int units = hkv * nch;
  constexpr int HB = G < 4 ? G : G == 8 ? 2 : 4;  // heads whose state a lane group keeps at once
  const int LPP = hd >> 3;                // lanes per position row
  const int PP = kThreads / LPP;          // lane groups = positions per pass
  const int grp = t / LPP, e8 = (t % LPP) * 8;
  const float scale = 1.4426950408889634f / sqrtf((float)hd);  // log2(e) / sqrt(hd)
  float* qs = c.s.att;                                    // [G][hd] rotated queries
  uint16_t* kv16 = reinterpret_cast<uint16_t*>(qs + G * hd);  // [2][hd] new row as stored
  float* gml = qs + G * hd + hd;                          // [PP][HB][2] per-group (m, l)
  float* go = gml + PP * HB * 2;                          // [PP][HB][hd] per-group o
  constexpr int APF = 2;                                  // passes prefetched into registers
  const uint32_t* src = X + P.xl.qkv + (size_t)l * N;
  if (c.wg < units && !await_all<HO>(P, X, l * kStagesPerLayer + 0, c.w, t)) return false;
  for (int u = c.wg; u < units; u += c.nb) {
    const int g = u % hkv, ch = u / hkv;
    const int j0 = ch * CL, j1 = min(n, j0 + CL);
    const bool has_new = pos >= j0 && pos < j1;
    const int npass = (j1 - j0 + PP - 1) / PP;
    const size_t plane = ((size_t)l * hkv + g) * P.max_seq * hd;
    uint16_t* kb = P.kc + plane;
    uint16_t* vb = P.vc + plane;
    // cached rows (written by earlier steps) do not depend on this step:
    // start streaming them before waiting for q
    uint4 kr[APF], vr[APF];
#pragma unroll
    for (int a = 0; a < APF; ++a) {
      const int j = j0 + a * PP + grp;
      if (a < npass && j < j1 && j != pos) {
        kr[a] = ldw(kb + (size_t)j * hd + e8);
        vr[a] = ldw(vb + (size_t)j * hd + e8);
      }
    }
    // poll roles: q of the G heads (pairs 2m, 2m+1 and their rotary partners
    // 2m+hd/2, 2m+1+hd/2), then the new k and v of head g
    const int nq = G * qd4, nkv = has_new ? qd4 : 0;
    const int role = t < nq ? 0 : t < nq + nkv ? 1 : t < nq + 2 * nkv ? 2 : 3;
    const int h = role == 0 ? t / qd4 : 0;
    const int m = role == 0 ? t % qd4 : role == 1 ? t - nq : role == 2 ? t - nq - nkv : 0;
    float4 rot = make_float4(1.f, 0.f, 1.f, 0.f);
    if (role <= 1) {
      const uint4 rw = ldw(reinterpret_cast<const uint16_t*>(P.rope + ((size_t)pos * half + 2 * m) * 2));
      rot = make_float4(__uint_as_float(rw.x), __uint_as_float(rw.y), __uint_as_float(rw.z), __uint_as_float(rw.w));
    }
    bool ok = true;
    if (role < 3) {
      const uint32_t* sp = role == 0 ? src + (size_t)(g * G + h) * hd
                         : role == 1 ? src + (size_t)hq * hd + (size_t)g * hd
                                     : src + (size_t)(hq + hkv) * hd + (size_t)g * hd;
      uint64_t va = xld64(sp + 2 * m), vb2 = xld64(sp + 2 * m + half);  // both in flight, one wait
      __builtin_amdgcn_sched_barrier(0);  // (the compiler had hoisted the first check above the second load)
      if (!(Ready32x2{}(va) && Ready32x2{}(vb2)))
        ok = poll64(sp + 2 * m, va, c.w, Ready32x2{}) && poll64(sp + 2 * m + half, vb2, c.w, Ready32x2{});
      float a0 = lo_f(va), a1 = hi_f(va), b0 = lo_f(vb2), b1 = hi_f(vb2);
      if (role <= 1) {  // rotate pairs (2m, 2m+hd/2) and (2m+1, 2m+1+hd/2)
        const float ra0 = a0 * rot.x - b0 * rot.y, rb0 = a0 * rot.y + b0 * rot.x;
        const float ra1 = a1 * rot.z - b1 * rot.w, rb1 = a1 * rot.w + b1 * rot.z;
        a0 = ra0; b0 = rb0; a1 = ra1; b1 = rb1;
      }
      if (role == 0) {
        float* qh = qs + h * hd;
        qh[2 * m] = a0; qh[2 * m + 1] = a1; qh[2 * m + half] = b0; qh[2 * m + 1 + half] = b1;
      } else if (ok) {
        // append to the cache for later steps; keep the stored values for now
        const uint32_t wa = pack16<DT>(a0, a1), wb = pack16<DT>(b0, b1);
        uint32_t* dst = reinterpret_cast<uint32_t*>((role == 1 ? kb : vb) + (size_t)pos * hd);
        xst32(dst + m, wa);
        xst32(dst + m + (half >> 1), wb);
        uint32_t* kv32 = reinterpret_cast<uint32_t*>(kv16) + (role == 1 ? 0 : half);
        kv32[m] = wa;
        kv32[m + (half >> 1)] = wb;
      }
    }
    if (any_failed(!ok)) return false;
    stamp(tr, slot, 1, t);
    if (has_new) {
#pragma unroll
      for (int a = 0; a < APF; ++a)
        if (a < npass && j0 + a * PP + grp == pos) {
          kr[a] = *reinterpret_cast<const uint4*>(kv16 + e8);
          vr[a] = *reinterpret_cast<const uint4*>(kv16 + hd + e8);
        }
    }
    const int ngrp = min(PP, j1 - j0);  // lane groups holding at least one position
#pragma unroll 1
    for (int hb = 0; hb < G; hb += HB) {
      float q[HB][8], mx[HB], ls[HB], o[HB][8];
#pragma unroll
      for (int h = 0; h < HB; ++h) {
        mx[h] = -INFINITY;
        ls[h] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          q[h][e] = qs[(hb + h) * hd + e8 + e];
          o[h][e] = 0.f;
        }
      }
      for (int a = 0; a < npass; ++a) {
        const int j = j0 + a * PP + grp;
        if (j >= j1) break;  // uniform per lane group
        uint4 k4, v4;
        if (a < APF) {
          k4 = kr[0];
          v4 = vr[0];
#pragma unroll
          for (int b = 1; b < APF; ++b)
            if (b == a) { k4 = kr[b]; v4 = vr[b]; }
        } else if (j == pos) {
          k4 = *reinterpret_cast<const uint4*>(kv16 + e8);
          v4 = *reinterpret_cast<const uint4*>(kv16 + hd + e8);
        } else {
          k4 = ldw(kb + (size_t)j * hd + e8);
          v4 = ldw(vb + (size_t)j * hd + e8);
        }
        float kf[8], vf[8];
        unpack8<DT>(k4, kf);
        unpack8<DT>(v4, vf);
#pragma unroll
        for (int h = 0; h < HB; ++h) {
          float sd = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) sd += q[h][e] * kf[e];
          // rows of 16 lanes (hd 128) take one more DPP step than rows of 8;
          // a select instead of a branch keeps the heads' chains interleaved
          sd = sum8(sd);
          const float sd16 = sd + dpp<DPP_MIRROR>(sd);
          sd = (hd == 128 ? sd16 : sd) * scale;
          const float mn = fmaxf(mx[h], sd);
          const float fo = safe_exp_diff(mx[h], mn), fp = fast_exp2(sd - mn);
          ls[h] = ls[h] * fo + fp;
#pragma unroll
          for (int e = 0; e < 8; ++e) o[h][e] = o[h][e] * fo + fp * vf[e];
          mx[h] = mn;
        }
      }
      if (grp < ngrp) {
#pragma unroll
        for (int h = 0; h < HB; ++h) {
          float* dst = go + (grp * HB + h) * hd + e8;
#pragma unroll
          for (int e = 0; e < 8; ++e) dst[e] = o[h][e];
          if (e8 == 0) {
            gml[(grp * HB + h) * 2] = mx[h];
            gml[(grp * HB + h) * 2 + 1] = ls[h];
          }
        }
      }
      stamp(tr, slot, 2, t);
      __syncthreads();
      // fold the groups and publish (m, l, o) of heads hb .. hb+HB-1 for this chunk
      publish_delay(P);
      uint32_t* att = X + P.xl.att;
      for (int idx = t; idx < HB * hd; idx += kThreads) {
        const int h = idx / hd, e = idx % hd;
        // eight groups' values are read before any is used (clamped indices,
        // the surplus masked), so the LDS round trips overlap
        float M = -INFINITY, Ls = 0.f, Os = 0.f;
        for (int g0 = 0; g0 < ngrp; g0 += 8) {
          float mv[8], lv[8], ov[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const int g2 = min(g0 + q, ngrp - 1);
            mv[q] = gml[(g2 * HB + h) * 2];
            lv[q] = gml[(g2 * HB + h) * 2 + 1];
            ov[q] = go[(g2 * HB + h) * hd + e];
          }
          float Mb = M;
#pragma unroll
          for (int q = 0; q < 8; ++q) Mb = fmaxf(Mb, mv[q]);
          const float r = safe_exp_diff(M, Mb);  // rescale what was folded so far
          Ls *= r;
          Os *= r;
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const float f = g0 + q < ngrp ? safe_exp_diff(mv[q], Mb) : 0.f;
            Ls += lv[q] * f;
            Os += ov[q] * f;
          }
          M = Mb;
        }
        uint32_t* rowp = att + (((size_t)l * hq + (size_t)g * G + hb + h) * P.cmax + ch) * P.astride;
        xst32(rowp + 4 + e, __float_as_uint(Os));
        if (e == 0) xst64(rowp, pack2f(M, Ls));
      }
      __syncthreads();
    }
  }
  arrive<HO>(P, X, l * kStagesPerLayer + 1, t);
  stamp(tr, slot, 3, t);
  return true;
}

// Merge of the split-KV partials.  Unit (head h, dims 8s..8s+7) runs on one
// wave; lanes walk the chunks with an online rescaling, then the wave combines.
template <int DT, bool HO>
__device__ KIE_INLINE bool st_merge(const Params* Pp, char* smem, int l, int pos, uint32_t* X, uint64_t* tr) {
  const Sc c = stage_ctx(Pp, smem);
  CParams& P = c.P;
  const int slot = l * kStagesPerLayer + 2;
  stamp(tr, slot, 0, c.t);
  const int hd = P.hd, hq = P.hq;
  int CL, nch;
  attn_chunking(P, pos + 1, CL, nch);
  const int spl = hd >> 3;
  const int units = hq * spl;
  const int wave = c.t >> 6, lane = c.t & 63;
  if (c.wg < units && !await_all<HO>(P, X, l * kStagesPerLayer + 1, c.w, c.t)) return false;
  bool ok = true;
  for (int u = c.wg + wave * c.nb; u < units; u += c.nb * kWaves) {
    const int h = u / spl, sl = u % spl;
    float m = -INFINITY, ls = 0.f, o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;
    for (int ch = lane; ch < nch && ok; ch += 64) {
      const uint32_t* rowp = X + P.xl.att + (((size_t)l * hq + h) * P.cmax + ch) * P.astride;
      const uint32_t* op = rowp + 4 + sl * 8;
      // issue all five loads, then wait once
      uint64_t mlv = xld64(rowp), o01 = xld64(op), o23 = xld64(op + 2), o45 = xld64(op + 4), o67 = xld64(op + 6);
      __builtin_amdgcn_sched_barrier(0);
      const Ready32x2 rd{};
      if (!(rd(mlv) && rd(o01) && rd(o23) && rd(o45) && rd(o67))) {
        ok = poll64(rowp, mlv, c.w, rd) && poll64(op, o01, c.w, rd) && poll64(op + 2, o23, c.w, rd) &&
             poll64(op + 4, o45, c.w, rd) && poll64(op + 6, o67, c.w, rd);
        if (!ok) break;
      }
      const float mc = lo_f(mlv), lc = hi_f(mlv);
      const float mn = fmaxf(m, mc);
      const float a = safe_exp_diff(m, mn), b = fast_exp2(mc - mn);
      ls = ls * a + lc * b;
      const float oc[8] = {lo_f(o01), hi_f(o01), lo_f(o23), hi_f(o23), lo_f(o45), hi_f(o45), lo_f(o67), hi_f(o67)};
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = o[e] * a + oc[e] * b;
      m = mn;
    }
    stamp(tr, slot, 1, c.t);
    const float M = wave_max(m);
    const float f = safe_exp_diff(m, M);
    ls = sum64_tail(ls * f);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = sum64_tail(o[e] * f);
    if (ok) publish_delay(P);
    if (lane == 63 && ok) {
      const float inv = 1.0f / ls;
      uint32_t* dst = X + P.xl.a + (size_t)l * hq * hd + (size_t)h * hd + sl * 8;
      xst64(dst, pack2f(o[0] * inv, o[1] * inv));
      xst64(dst + 2, pack2f(o[2] * inv, o[3] * inv));
      xst64(dst + 4, pack2f(o[4] * inv, o[5] * inv));
      xst64(dst + 6, pack2f(o[6] * inv, o[7] * inv));
    }
  }
  const bool failed = any_failed(!ok);
  if (!failed) arrive<HO>(P, X, l * kStagesPerLayer + 2, c.t);
  stamp(tr, slot, 3, c.t);
  return !failed;
}

// x_mid = x_l + Wo a  (rows split over work-groups).  PS (here and in the
// feed-forward stages): the stage runs as a launch of its own (stage_kernel),
// so it issues no weights for the next stage -- its registers end with it.
template <int DT, int VD, bool HO, bool PS>
__device__ KIE_INLINE bool st_wo(const Params* Pp, char* smem, int l, uint32_t* X, uint64_t* tr, uint4 (&ring)[kDepth]) {
  const Sc c = stage_ctx(Pp, smem);
  CParams& P = c.P;
  const int slot = l * kStagesPerLayer + 3;
  stamp(tr, slot, 0, c.t);
  const int d = P.d, K = P.hq * P.hd;
  const int r0 = split_lo(d, c.nb, c.wg), r1 = split_lo(d, c.nb, c.wg + 1);
  const StagePlan pl = plan_stage(P, l, GS_WO, c.t, c.wg, c.nb);
  auto prep = [&](auto fill) -> bool {
    if (!await_all<HO>(P, X, l * kStagesPerLayer + 2, c.w, c.t)) return false;
    const bool r = poll_to16<DT, kPollD>(X + P.xl.a + (size_t)l * K, K, c.s.xn, c.w, c.t, fill);
    stamp(tr, slot, 1, c.t);
    return r;
  };
  const StagePlan np = plan_stage(P, l, GS_GATEUP, c.t, c.wg, c.nb);
  if (!gemv_cls<DT, VD>(pl, prep, c.s.xn, c.s.red, c.s.yv, c.t, ring, false, tr, slot)) return false;
  uint32_t* dst = X + P.xl.xmid + (size_t)l * d;
  publish_delay(P);
  for (int r = c.t; r < r1 - r0; r += kThreads)
    xst32(dst + r0 + r, __float_as_uint(c.s.xres[r0 + r] + c.s.yv[r]));
  arrive<HO>(P, X, l * kStagesPerLayer + 3, c.t);
  if constexpr (!PS) ring_prefetch<ring_split<VD>()>(ring, np);  // after the output stores: they must not queue behind it
  stamp(tr, slot, 3, c.t);
  return true;
}

// h = silu(Wg n) * (Wu n), n = RMSNorm(x_mid) * g_ffn
template <int DT, int VD, int VF, bool HO, bool PS>
__device__ KIE_INLINE bool st_gateup(const Params* Pp, char* smem, int l, uint32_t* X, uint64_t* tr, uint4 (&ring)[kDepth]) {
  const Sc c = stage_ctx(Pp, smem);
  CParams& P = c.P;
  const int slot = l * kStagesPerLayer + 4;
  stamp(tr, slot, 0, c.t);
  const int d = P.d, F = P.F;
  const int f0 = split_lo(F, c.nb, c.wg), f1 = split_lo(F, c.nb, c.wg + 1);
  const int nf = f1 - f0;
  const StagePlan pl = plan_stage(P, l, GS_GATEUP, c.t, c.wg, c.nb);
  auto prep = [&](auto fill) -> bool {
    const Gains gn = load_gains(lw_ptr(P, l, W_FFN_NORM), d, c.t);
    if (!await_all<HO>(P, X, l * kStagesPerLayer + 3, c.w, c.t)) return false;
    if (!poll_f32<kPollD>(X + P.xl.xmid + (size_t)l * d, d, c.s.xres, c.w, c.t, fill)) return false;
    rmsnorm_to16<DT>(c.s.xres, gn, d, P.eps, c.s.xn, c.s.misc, c.t);
    stamp(tr, slot, 1, c.t);
    return true;
  };
  const StagePlan np = plan_stage(P, l, GS_DOWN, c.t, c.wg, c.nb);
  if (!gemv_cls<DT, VD>(pl, prep, c.s.xn, c.s.red, c.s.yv, c.t, ring, true, tr, slot)) return false;
  uint32_t* dst = X + P.xl.h + (size_t)l * F;
  publish_delay(P);
  for (int f = c.t; f < nf; f += kThreads) {
    const float gt = c.s.yv[f], up = c.s.yv[nf + f];
    xst32(dst + f0 + f, __float_as_uint(gt / (1.0f + expf(-gt)) * up));
  }
  arrive<HO>(P, X, l * kStagesPerLayer + 4, c.t);
  if constexpr (!PS) ring_prefetch<ring_split<VF>()>(ring, np);
  stamp(tr, slot, 3, c.t);
  return true;
}

// x_next = x_mid + Wd h
template <int DT, int VD, int VF, bool HO, bool PS>
__device__ KIE_INLINE bool st_down(const Params* Pp, char* smem, int l, uint32_t* X, uint64_t* tr, uint4 (&ring)[kDepth]) {
  const Sc c = stage_ctx(Pp, smem);
  CParams& P = c.P;
  const int slot = l * kStagesPerLayer + 5;
  stamp(tr, slot, 0, c.t);
  const int d = P.d, F = P.F;
  const int r0 = split_lo(d, c.nb, c.wg), r1 = split_lo(d, c.nb, c.wg + 1);
  const StagePlan pl = plan_stage(P, l, GS_DOWN, c.t, c.wg, c.nb);
  auto prep = [&](auto fill) -> bool {
    if (!await_all<HO>(P, X, l * kStagesPerLayer + 4, c.w, c.t)) return false;
    const bool r = poll_to16<DT, kPollBatch>(X + P.xl.h + (size_t)l * F, F, c.s.xn, c.w, c.t, fill);
    stamp(tr, slot, 1, c.t);
    return r;
  };
  const StagePlan np = l + 1 < P.L ? plan_stage(P, l + 1, GS_QKV, c.t, c.wg, c.nb)
                                   : plan_stage(P, 0, GS_LM, c.t, c.wg, c.nb);
  if (!gemv_cls<DT, VF>(pl, prep, c.s.xn, c.s.red, c.s.yv, c.t, ring, true, tr, slot)) return false;
  uint32_t* dst = X + P.xl.xout + (size_t)l * d;
  publish_delay(P);
  for (int r = c.t; r < r1 - r0; r += kThreads)
    xst32(dst + r0 + r, __float_as_uint(c.s.xres[r0 + r] + c.s.yv[r]));
  arrive<HO>(P, X, l * kStagesPerLayer + 5, c.t);
  if constexpr (!PS) ring_prefetch<ring_split<VD>()>(ring, np);
  stamp(tr, slot, 3, c.t);
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

// ---- sampling (temperature, top-k, nucleus) --------------------------------
//
// Candidate order: larger logit first, lower index on ties.  In registers a
// candidate is one 64-bit key whose unsigned order is that order: the logit's
// bits made order-preserving (sign flipped for positives, all bits for
// negatives; NaN taken as -inf) above the complemented index.  Every candidate
// has its own index (vocabulary rows, or padding indices from kPadIdx up), so
// keys are distinct and every step of the selection is a plain comparison.
__device__ __forceinline__ uint64_t cand_key(float v, int i) {
  const uint32_t u = __float_as_uint(v == v ? v : -INFINITY);
  const uint32_t h = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)h << 32) | (uint32_t)~(uint32_t)i;
}
__device__ __forceinline__ float key_value(uint64_t k) {
  const uint32_t h = (uint32_t)(k >> 32);
  return __uint_as_float((h & 0x80000000u) ? (h & 0x7FFFFFFFu) : ~h);
}
__device__ __forceinline__ int key_index(uint64_t k) { return (int)~(uint32_t)k; }

// Published lists alternate in direction so that merge trees always pair
// opposite directions.  Work-group lists (merged in groups of 8 consecutive
// ones): best-first for odd work-groups.  Group lists (wave w of work-group 0
// merges groups w, w + 8, ...): best-first when bit 3 of the group is set.
__device__ __forceinline__ bool wg_list_desc(int wg) { return wg & 1; }
__device__ __forceinline__ bool group_list_desc(int g) { return (g >> 3) & 1; }

// Padding candidates (logit -inf) get distinct indices from kPadIdx up: row
// slots of work-group wg at (wg << 10) + slot, the gatherer's padding lists
// and idle waves from kPadRest.
constexpr int kPadRest = kPadIdx + (kMaxWG << 10);

// x from lane (lane ^ S), S a power of two below 64: DPP within rows of 16
// lanes, the gfx950 row / half-wave swaps above (their two results XOR the own
// value out, whichever order they come in).
template <int S>
__device__ __forceinline__ uint32_t lane_xor(uint32_t x, int lane) {
  if constexpr (S == 1) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
  } else if constexpr (S == 2) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
  } else if constexpr (S == 4) {
    const int up = __builtin_amdgcn_update_dpp(0, (int)x, 0x104, 0xF, 0xF, false);  // row_shl:4, lane + 4
    const int dn = __builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);  // row_shr:4, lane - 4
    return (uint32_t)((lane & 4) ? dn : up);
  } else if constexpr (S == 8) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x128, 0xF, 0xF, false);  // row_ror:8
  } else if constexpr (S == 16) {
    const auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return p[0] ^ p[1] ^ x;
  } else {
    const auto p = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return p[0] ^ p[1] ^ x;
  }
}

// Compare-exchange with lane (lane ^ S): the lower lane of each pair keeps the
// larger key in a best-first (desc) block, the smaller one otherwise.
template <int S>
__device__ __forceinline__ void cas_step(uint64_t& k, int lane, bool desc) {
  const uint64_t p = ((uint64_t)lane_xor<S>((uint32_t)(k >> 32), lane) << 32) | lane_xor<S>((uint32_t)k, lane);
  const bool keep_max = ((lane & S) == 0) == desc;
  k = ((p > k) == keep_max) ? p : k;
}

// Lists of 64 keys (lane j = entry j) sorted in opposite directions: their
// concatenation is bitonic, so the lane-wise larger key is the 64 best of the
// union, itself bitonic; six compare-exchange steps at distances 32 .. 1 sort
// it best-first (desc) or worst-first.
__device__ __forceinline__ void merge_lists(uint64_t& a, uint64_t b, int lane, bool desc) {
  a = b > a ? b : a;
  cas_step<32>(a, lane, desc);
  cas_step<16>(a, lane, desc);
  cas_step<8>(a, lane, desc);
  cas_step<4>(a, lane, desc);
  cas_step<2>(a, lane, desc);
  cas_step<1>(a, lane, desc);
}

// Sort 64 keys (lane j holds one) best-first (desc) or worst-first: a bitonic
// network over blocks of 2, 4, ..., 64 lanes; below 64 the blocks alternate
// direction so that neighbouring blocks form a bitonic block of the next size.
template <int B>
__device__ __forceinline__ void sort_stage(uint64_t& k, int lane, bool desc) {
  const bool d = B == 64 ? desc : (desc != ((lane & B) != 0));
  if constexpr (B >= 64) cas_step<32>(k, lane, d);
  if constexpr (B >= 32) cas_step<16>(k, lane, d);
  if constexpr (B >= 16) cas_step<8>(k, lane, d);
  if constexpr (B >= 8) cas_step<4>(k, lane, d);
  if constexpr (B >= 4) cas_step<2>(k, lane, d);
  cas_step<1>(k, lane, d);
}
__device__ __forceinline__ void sort64(uint64_t& k, int lane, bool desc) {
  sort_stage<2>(k, lane, desc);
  sort_stage<4>(k, lane, desc);
  sort_stage<8>(k, lane, desc);
  sort_stage<16>(k, lane, desc);
  sort_stage<32>(k, lane, desc);
  sort_stage<64>(k, lane, desc);
}

// Pairwise merge tree over N lists in registers (N a power of two; list k is
// worst-first for even k, best-first for odd k).  Pair m of every round is
// written worst-first for even m, best-first for odd m; the last merge gives
// direction `last_desc`.  The merges of a round are independent and overlap.
template <int N>
__device__ __forceinline__ void merge_tree(uint64_t (&k)[N], int lane, bool last_desc) {
#pragma unroll
  for (int span = 1; span < N; span *= 2) {
#pragma unroll
    for (int a = 0; a < N; a += 2 * span)
      merge_lists(k[a], k[a + span], lane, 2 * span == N ? last_desc : ((a / (2 * span)) & 1) != 0);
  }
}

// Padding list in direction `desc`: indices base + rank, rank = lane (best
// first) or 63 - lane.
__device__ __forceinline__ uint64_t pad_list(int base, int lane, bool desc) {
  return cand_key(-INFINITY, base + (desc ? lane : kCand - 1 - lane));
}

// This work-group's 64 best rows (n <= 1024 logits in yv): wave w sorts rows
// 64w + lane (and 512 + 64w + lane); the waves' lists meet in a merge tree in
// wave 0 (over the smallest power of two of waves that holds every row),
// which publishes the list, direction wg_list_desc(wg), as (logit, index) pairs.
// Ranks past the row count are padding.
__device__ __forceinline__ void publish_candidates(const float* yv, int n, int v0, uint32_t* dst, int wg, int t,
                                                   float* lds) {
  const int lane = t & 63, wv = t >> 6;
  auto key = [&](int r) { return r < n ? cand_key(yv[r], v0 + r) : cand_key(-INFINITY, kPadIdx + (wg << 10) + r); };
  const int used = n > 512 ? kWaves : n > 256 ? 8 : n > 128 ? 4 : n > 64 ? 2 : 1;  // lists in the tree
  uint64_t* lk = reinterpret_cast<uint64_t*>(lds);
  if (wv < used) {
    uint64_t k = key(64 * wv + lane);
    sort64(k, lane, (wv & 1) != 0);
    if (n > 512) {
      uint64_t k2 = key(512 + 64 * wv + lane);
      sort64(k2, lane, (wv & 1) == 0);
      merge_lists(k, k2, lane, (wv & 1) != 0);
    }
    lk[wv * kCand + lane] = k;
  }
  __syncthreads();
  if (wv == 0) {
    uint64_t k;
    if (used == 1) {  // wave 0 sorted worst-first: a best-first list takes its entries in reverse
      k = lk[wg_list_desc(wg) ? kCand - 1 - lane : lane];
    } else if (used == 2) {
      uint64_t kk[2] = {lk[lane], lk[kCand + lane]};
      merge_tree<2>(kk, lane, wg_list_desc(wg));
      k = kk[0];
    } else if (used == 4) {
      uint64_t kk[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) kk[w] = lk[w * kCand + lane];
      merge_tree<4>(kk, lane, wg_list_desc(wg));
      k = kk[0];
    } else {
      uint64_t kk[kWaves];
#pragma unroll
      for (int w = 0; w < kWaves; ++w) kk[w] = lk[w * kCand + lane];
      merge_tree<kWaves>(kk, lane, wg_list_desc(wg));
      k = kk[0];
    }
    xst64(dst + 2 * lane, pack2f(key_value(k), __int_as_float(key_index(k))));
  }
  __syncthreads();
}

// Poll-load entry `lane` of list `l` of an exchange array of lists and make it
// a key; false (for the whole wave) when a poll gave up.
__device__ __forceinline__ bool load_list(const uint32_t* src, int l, int lane, uint64_t& k, const Watch& w) {
  const uint32_t* p = src + ((size_t)l * kCand + lane) * 2;
  uint64_t e = xld64(p);
  const bool got = Ready32x2{}(e) || poll64(p, e, w, Ready32x2{});
  k = cand_key(lo_f(e), __float_as_int(hi_f(e)));
  return __all(got);
}

// Work-group g < ceil(grid / 8): merge the lists of work-groups 8g .. 8g+7
// (wave w loads one; missing ones are padding) in a tree in wave 0 and
// publish the group's 64 best, direction group_list_desc(g).
__device__ KIE_INLINE bool group_merge(const Params* Pp, char* smem, uint32_t* X) {
  const Sc c = stage_ctx(Pp, smem);
  CParams& P = c.P;
  const int lane = c.t & 63, wv = c.t >> 6, g = c.wg, l = 8 * g + wv;
  uint64_t k = pad_list(kPadRest + l * kCand, lane, wg_list_desc(l));
  bool ok = l >= c.nb || load_list(X + P.xl.cand, l, lane, k, c.w);
  if (any_failed(!ok)) return false;
  uint64_t* lk = reinterpret_cast<uint64_t*>(c.s.red);  // red/yv are idle after the LM head
  lk[wv * kCand + lane] = k;
  __syncthreads();
  if (wv == 0) {
    uint64_t k8[kWaves];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) k8[w] = lk[w * kCand + lane];
    merge_tree<kWaves>(k8, lane, group_list_desc(g));
    publish_delay(P);
    xst64(X + P.xl.cand2 + ((size_t)g * kCand + lane) * 2, pack2f(key_value(k8[0]), __int_as_float(key_index(k8[0]))));
  }
  __syncthreads();
  return true;
}

// Work-group 0: gather the group lists and reduce them to the global 64 best,
// then wave 0 draws.  Wave w loads groups w, w + 8, ... (all in flight) and
// merges them in a register tree; the eight waves' lists meet in a second tree
// in wave 0.  Draw: weights exp2((z - z0) * log2(e) / T) over the first
// samp_k, inclusive prefix sums S across lanes, nucleus n = 1 + #{S_j < top_p *
// S_{k-1}}, u from Philox4x32-10 (counter (pos, 0, 0, 0)), token = entry
// #{j < n : S_j <= u S_{n-1}}.
constexpr int kGroupsPerWave = kMaxWG / 8 / kWaves;  // 16 group lists per wave at most
__device__ KIE_INLINE bool gather_sample(const Params* Pp, char* smem, uint32_t* X, int pos, int& tok,
                                          uint64_t* tr) {
  const Sc c = stage_ctx(Pp, smem);
  CParams& P = c.P;
  const int slot = P.L * kStagesPerLayer + 2;
  stamp(tr, slot, 0, c.t);
  const int lane = c.t & 63, wv = c.t >> 6, ng = (c.nb + 7) / 8;
  const uint32_t* src = X + P.xl.cand2;
  uint64_t kk[kGroupsPerWave];
  uint64_t e[kGroupsPerWave];
#pragma unroll
  for (int k = 0; k < kGroupsPerWave; ++k) {  // issue every load first
    const int g = wv + 8 * k;
    e[k] = g < ng ? xld64(src + ((size_t)g * kCand + lane) * 2) : 0ull;
  }
  bool ok = true;
#pragma unroll
  for (int k = 0; k < kGroupsPerWave; ++k) {
    const int g = wv + 8 * k;
    if (g < ng) {
      if (ok) {
        const bool got = Ready32x2{}(e[k]) || poll64(src + ((size_t)g * kCand + lane) * 2, e[k], c.w, Ready32x2{});
        ok = __all(got);
      }
      kk[k] = cand_key(lo_f(e[k]), __float_as_int(hi_f(e[k])));
    } else {  // padding list in the direction group g would have had
      kk[k] = pad_list(kPadRest + (kMaxWG + g) * kCand, lane, group_list_desc(g));
    }
  }
  if (any_failed(!ok)) return false;
  uint64_t run;
  if (ng <= 8) {
    run = kk[0];
  } else if (ng <= 16) {
    uint64_t k2[2] = {kk[0], kk[1]};
    merge_tree<2>(k2, lane, (wv & 1) != 0);
    run = k2[0];
  } else if (ng <= 32) {
    uint64_t k4[4] = {kk[0], kk[1], kk[2], kk[3]};
    merge_tree<4>(k4, lane, (wv & 1) != 0);
    run = k4[0];
  } else {
    merge_tree<kGroupsPerWave>(kk, lane, (wv & 1) != 0);
    run = kk[0];
  }
  if (ng <= 8 && (wv & 1) != group_list_desc(wv))  // one group per wave: already in the list's direction
    run = __shfl(run, kCand - 1 - lane);
  stamp(tr, slot, 1, c.t);
  uint64_t* lk = reinterpret_cast<uint64_t*>(c.s.red);  // the waves' lists (red/yv are idle after the LM head)
  lk[wv * kCand + lane] = run;
  __syncthreads();
  if (wv == 0) {
    uint64_t k8[kWaves];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) k8[w] = lk[w * kCand + lane];
    merge_tree<kWaves>(k8, lane, true);
    const float v = key_value(k8[0]);
    const int i = key_index(k8[0]);
    const int K = P.samp_k;
    const float z0 = __shfl(v, 0);
    float S = lane < K ? __builtin_amdgcn_exp2f((v - z0) * P.samp_scale) : 0.f;
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
      const float o = __shfl_up(S, s);
      if (lane >= s) S += o;
    }
    const float total = __shfl(S, K - 1);
    const int n = 1 + (int)__popcll(__ballot(lane < K && S < P.samp_top_p * total));
    const float Sn = __shfl(S, n - 1);
    const uint4 x = philox4x32_10(make_uint4((uint32_t)pos, 0u, 0u, 0u), P.samp_key0, P.samp_key1);
    const float r = (float)(x.x >> 8) * 0x1p-24f * Sn;
    int j = (int)__popcll(__ballot(lane < n && S <= r));
    j = j < n ? j : n - 1;
    const int tk = __shfl(i, j);
    if (lane == 0) c.s.imisc[0] = tk;
  }
  __syncthreads();
  stamp(tr, slot, 2, c.t);
  const int tk = c.s.imisc[0];
  __syncthreads();
  tok = (tk >= 0 && tk < P.V) ? tk : 0;
  stamp(tr, slot, 3, c.t);
  return true;
}

// The sampled token: work-groups 0 .. ceil(grid/8)-1 merge groups of lists,
// work-group 0 draws the token and publishes it, the others poll it.
__device__ KIE_INLINE bool sampled_token(const Params* Pp, char* smem, uint32_t* X, int pos, int& tok, uint64_t* tr) {
  if ((int)blockIdx.x < (cparams(Pp).grid + 7) / 8 && !group_merge(Pp, smem, X)) return false;
  if (blockIdx.x == 0) {
    if (!gather_sample(Pp, smem, X, pos, tok, tr)) return false;
    publish_delay(cparams(Pp));
    if (threadIdx.x == 0) xst64(X + cparams(Pp).xl.stok, pack2f(__int_as_float(tok), 0.f));
    return true;
  }
  const Sc c = stage_ctx(Pp, smem);
  const int slot = c.P.L * kStagesPerLayer + 2;
  stamp(tr, slot, 0, c.t);
  bool ok = true;
  if (c.t == 0) {
    uint64_t v = 0;
    ok = poll64(X + c.P.xl.stok, v, c.w, Ready32x2{});
    c.s.imisc[0] = __float_as_int(lo_f(v));
  }
  if (any_failed(!ok)) return false;
  const int tk = c.s.imisc[0];
  __syncthreads();
  tok = (tk >= 0 && tk < c.P.V) ? tk : 0;
  stamp(tr, slot, 3, c.t);
  return true;
}

// LM head on this work-group's vocabulary rows; logits optionally written.
// The host guarantees ceil(V / grid) rows fit the LDS partial-sum buffers.
template <int DT, int VD, bool HO>
__device__ KIE_INLINE bool st_lmhead(const Params* Pp, char* smem, uint32_t* X, float* logits, float& best_v,
                                     int& best_i, uint64_t* tr, uint4 (&ring)[kDepth]) {
  const Sc c = stage_ctx(Pp, smem);
  CParams& P = c.P;
  const int slot = P.L * kStagesPerLayer;
  stamp(tr, slot, 0, c.t);
  const int d = P.d, V = P.V;
  const int v0 = split_lo(V, c.nb, c.wg), v1 = split_lo(V, c.nb, c.wg + 1);
  const StagePlan pl = plan_stage(P, 0, GS_LM, c.t, c.wg, c.nb);
  auto prep = [&](auto fill) -> bool {
    if (!await_all<HO>(P, X, (P.L - 1) * kStagesPerLayer + 5, c.w, c.t)) return false;
    const Gains gn = load_gains(P.final_norm, d, c.t);
    if (!poll_f32<kPollD>(X + P.xl.xout + (size_t)(P.L - 1) * d, d, c.s.xres, c.w, c.t, fill)) return false;
    rmsnorm_to16<DT>(c.s.xres, gn, d, P.eps, c.s.xn, c.s.misc, c.t);
    stamp(tr, slot, 1, c.t);
    return true;
  };
  if (!gemv_cls<DT, VD>(pl, prep, c.s.xn, c.s.red, c.s.yv, c.t, ring, true, tr, slot)) return false;
  float bv = -INFINITY;
  int bi = 0x7FFFFFFF;
  for (int r = c.t; r < v1 - v0; r += kThreads) {
    const float y = c.s.yv[r];
    if (logits) logits[v0 + r] = y;
    if (arg_better(y, v0 + r, bv, bi)) {
      bv = y;
      bi = v0 + r;
    }
  }
  if (P.samp_k > 0) {
    publish_delay(P);
    publish_candidates(c.s.yv, v1 - v0, v0, X + P.xl.cand + (size_t)c.wg * kCand * 2, c.wg, c.t, c.s.red);
  }
  block_argmax(bv, bi, c.s, c.t);
  best_v = bv;
  best_i = bi;
  stamp(tr, slot, 3, c.t);
  return true;
}

// Reset this work-group's share of exchange set `Xr` to the NaN pattern, with
// threads [t_lo, kThreads).  Xr is the set of step s-1 while this is step s.
// Why no work-group still reads it: every work-group owns at least one row of
// every vector a step-s hand-off polls (the host keeps the grid at most
// d_model and d_ffn wide), so this work-group could only reach step s's
// recycling after every other work-group published step-s words, i.e. after
// each had left step s-1 -- including the argmax and sampling words it reads
// in step s-1's tail, after publishing its own partial.  Set Xr is written
// again at step s+2, by work-groups that have gathered this work-group's step
// s+1 partial, which is published only after these stores were performed.
__device__ KIE_INLINE void reset_set(const Params* Pp, char* smem, uint32_t* Xr, int nch_prev, int t_lo,
                                     uint64_t* tr) {
  const Sc c = stage_ctx(Pp, smem);
  CParams& P = c.P;
  if (c.t < t_lo) return;
  const uint32_t tt = c.t - t_lo, nt = kThreads - t_lo;
  const uint64_t sent2 = ~0ull;
  {  // dense part, 8-byte units (the host keeps every count below 2^32 / grid)
    const uint32_t dense2 = (uint32_t)(P.xl.dense >> 1);
    const uint32_t a = split_lo(dense2, c.nb, c.wg), b = split_lo(dense2, c.nb, c.wg + 1);
    for (uint32_t k = a + tt; k < b; k += nt) xst64(Xr + 2 * (size_t)k, sent2);
  }
  if (nch_prev > 0) {  // the chunks of every (layer, head) block that were in use
    const uint32_t per = (uint32_t)(nch_prev * P.astride / 2);  // 8-byte units per block
    const uint32_t blocks = (uint32_t)(P.L * P.hq);
    const uint32_t b0 = split_lo(blocks, c.nb, c.wg), b1 = split_lo(blocks, c.nb, c.wg + 1);
    uint32_t* att = Xr + P.xl.att;
    for (uint32_t blk = b0; blk < b1; ++blk) {
      uint32_t* base = att + (size_t)blk * P.cmax * P.astride;
      for (uint32_t k = tt; k < per; k += nt) xst64(base + 2 * (size_t)k, sent2);
    }
  }
  stamp(tr, P.L * kStagesPerLayer + 1, 2, c.t, t_lo);
}

// Gather the per-work-group (max, index) partials -> the greedy token (also
// the end-of-step marker when sampling chooses the token instead).  Every
// work-group reduces the same values in the same order, so all agree.
template <bool HO>
__device__ KIE_INLINE bool gather_token(const Params* Pp, char* smem, uint32_t* X, int& tok, uint64_t* tr) {
  const Sc c = stage_ctx(Pp, smem);
  const int slot = c.P.L * kStagesPerLayer + 1;
  stamp(tr, slot, 0, c.t);
  CParams& P = c.P;
  float gv = -INFINITY;
  int gi = 0x7FFFFFFF;
  bool ok = true;
  if (!await_all<HO>(P, X, P.L * kStagesPerLayer, c.w, c.t)) return false;
  for (int w = c.t; w < c.nb && c.t < kThreads / 2; w += kThreads / 2) {
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
  stamp(tr, slot, 1, c.t);
  block_argmax(gv, gi, c.s, c.t);
  // NaN logits never win a comparison: keep the index inside the vocabulary
  tok = (gi >= 0 && gi < P.V) ? gi : 0;
  stamp(tr, slot, 3, c.t);
  return true;
}

// ---------------------------------------------------------------------------
// The persistent kernel
// ---------------------------------------------------------------------------
// HO: the arrival-counter hand-off (the comparison protocol) instead of the
// NaN-polled data alone.
template <int DT, int G, int VD, int VF, bool HO>
__global__ __launch_bounds__(kThreads, 1) void monokernel(const Params* __restrict__ Pp) {
  extern __shared__ __align__(16) char smem[];
  const int t = threadIdx.x, wg = blockIdx.x;
  const int n_steps = Pp->n_steps, L = Pp->L;
  int tok = Pp->in_tok;
  int done = 0;
  bool ok = true;
  uint4 ring[kDepth];  // weight-stream ring shared by consecutive GEMV stages
  for (int s = 0; s < n_steps && ok; ++s) {
    CParams& P = cparams(Pp);
    const int pos = P.pos0 + s;
    if (P.forced) tok = P.forced[s];
    uint32_t* X = P.xch + (size_t)(s % kRingSets) * P.xl.words;
    uint64_t* tr = (P.trace && s == P.trace_step)
                       ? P.trace + (size_t)wg * (P.L * kStagesPerLayer + 3) * kTraceStamps
                       : nullptr;
    const bool lm_only = cparams(Pp).lm_only != 0;
    if (lm_only) {  // the LM head's first weight vectors (no down stage issued them)
      const Sc c = stage_ctx(Pp, smem);
      ring_prefetch<ring_split<VD>()>(ring, plan_stage(c.P, 0, GS_LM, c.t, c.wg, c.nb));
    } else {  // embedding row -> residual stream
      const Sc c = stage_ctx(Pp, smem);
      const uint16_t* er = c.P.tok_emb + (size_t)tok * c.P.d;
      for (int i = c.t; i < c.P.d; i += kThreads) c.s.xres[i] = to_f32<DT>(er[i]);
      __syncthreads();
    }
    for (int l = 0; l < L && ok && !lm_only; ++l) {
      ok = st_qkv<DT, VD, HO>(Pp, smem, l, X, tr, ring) && st_attn<DT, G, HO>(Pp, smem, l, pos, X, tr) &&
           st_merge<DT, HO>(Pp, smem, l, pos, X, tr) && st_wo<DT, VD, HO, false>(Pp, smem, l, X, tr, ring) &&
           st_gateup<DT, VD, VF, HO, false>(Pp, smem, l, X, tr, ring) &&
           st_down<DT, VD, VF, HO, false>(Pp, smem, l, X, tr, ring);
    }
    if (!ok) break;
    float bv = 0.f;
    int bi = 0;
    bool lm = false;
    {
      CParams& Q = cparams(Pp);
      lm = !Q.lm_last_only || s == Q.n_steps - 1;
      if (lm) {
        float* lg = Q.logits ? Q.logits + (size_t)(Q.lm_last_only ? 0 : s) * Q.V : nullptr;
        if (!st_lmhead<DT, VD, HO>(Pp, smem, X, lg, bv, bi, tr, ring)) {
          ok = false;
          break;
        }
      }
    }
    // publish this step's partial once everything this step wrote is performed
    drain_stores();
    publish_delay(cparams(Pp));
    __syncthreads();
    if (t == 0 && wg != Pp->withhold_wg) xst64(X + Pp->xl.arg + 2 * wg, pack2f(bv, __int_as_float(bi)));
    arrive<HO>(cparams(Pp), X, L * kStagesPerLayer, t);
    // the upper half of the work-group recycles the previous step's exchange
    // set while the lower half gathers the partials (grid <= kThreads / 2)
    if (s >= 1) {
      int CL, nch;
      attn_chunking(cparams(Pp), pos, CL, nch);
      reset_set(Pp, smem, Pp->xch + (size_t)((s + 2) % kRingSets) * Pp->xl.words, nch, kThreads / 2, tr);
    }
    if (!gather_token<HO>(Pp, smem, X, tok, tr)) {
      ok = false;
      break;
    }
    if (lm && cparams(Pp).samp_k > 0 && !sampled_token(Pp, smem, X, pos, tok, tr)) {
      ok = false;
      break;
    }
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
// The same stages as separate launches (the launch-tax comparison): launch
// (s, l, st) runs stage st of layer l of decode step s (st 0..5 = qkv, attn,
// merge, wo, gate/up, down; 6 = LM head and the argmax partial; 7 = exchange
// recycling and the token).  Each launch starts after the previous one has
// finished, so every poll finds its words already written; what the
// persistent kernel keeps on chip across stages (the residual row in LDS, the
// next stage's first weight vectors in registers) is reloaded here.  Greedy
// decode only, no end-of-sequence stop (the host checks both).
// ---------------------------------------------------------------------------
template <int DT, int G, int VD, int VF>
__global__ __launch_bounds__(kThreads, 1) void stage_kernel(const Params* __restrict__ Pp, int s, int l, int st) {
  extern __shared__ __align__(16) char smem[];
  const Sc c = stage_ctx(Pp, smem);
  CParams& P = c.P;
  const int pos = P.pos0 + s;
  uint32_t* X = P.xch + (size_t)(s % kRingSets) * P.xl.words;
  uint4 ring[kDepth];
  auto load_embedding = [&]() {
    const int tok = P.forced ? P.forced[s] : s == 0 ? P.in_tok : Pp->tok_out[s - 1];
    const uint16_t* er = P.tok_emb + (size_t)tok * P.d;
    for (int i = c.t; i < P.d; i += kThreads) c.s.xres[i] = to_f32<DT>(er[i]);
    __syncthreads();
  };
  auto own_prefetch = [&](int lay, int gs) {
    const StagePlan np = plan_stage(P, lay, gs, c.t, c.wg, c.nb);
    if (gs == GS_DOWN) ring_prefetch<ring_split<VF>()>(ring, np);
    else ring_prefetch<ring_split<VD>()>(ring, np);
  };
  bool ok = true;
  switch (st) {
    case 0:
      if (l == 0) load_embedding();
      else own_prefetch(l, GS_QKV);
      ok = st_qkv<DT, VD, false>(Pp, smem, l, X, nullptr, ring);
      break;
    case 1: ok = st_attn<DT, G, false>(Pp, smem, l, pos, X, nullptr); break;
    case 2: ok = st_merge<DT, false>(Pp, smem, l, pos, X, nullptr); break;
    case 3:  // the residual x_l that the Wo outputs add to
      if (l == 0) load_embedding();
      else ok = poll_f32(X + P.xl.xout + (size_t)(l - 1) * P.d, P.d, c.s.xres, c.w, c.t);
      ok = ok && st_wo<DT, VD, false, true>(Pp, smem, l, X, nullptr, ring);
      break;
    case 4:
      own_prefetch(l, GS_GATEUP);
      ok = st_gateup<DT, VD, VF, false, true>(Pp, smem, l, X, nullptr, ring);
      break;
    case 5:  // the residual x_mid that the down outputs add to
      ok = poll_f32(X + P.xl.xmid + (size_t)l * P.d, P.d, c.s.xres, c.w, c.t);
      own_prefetch(l, GS_DOWN);
      ok = ok && st_down<DT, VD, VF, false, true>(Pp, smem, l, X, nullptr, ring);
      break;
    case 6: {
      own_prefetch(0, GS_LM);
      float bv = 0.f;
      int bi = 0;
      float* lg = P.logits ? P.logits + (size_t)s * P.V : nullptr;
      ok = st_lmhead<DT, VD, false>(Pp, smem, X, lg, bv, bi, nullptr, ring);
      drain_stores();
      __syncthreads();
      if (ok && c.t == 0) xst64(X + P.xl.arg + 2 * c.wg, pack2f(bv, __int_as_float(bi)));
      break;
    }
    default: {
      if (s >= 1) {
        int CL, nch;
        attn_chunking(P, pos, CL, nch);
        reset_set(Pp, smem, P.xch + (size_t)((s + 2) % kRingSets) * P.xl.words, nch, kThreads / 2, nullptr);
      }
      int tok = 0;
      ok = gather_token<false>(Pp, smem, X, tok, nullptr);
      if (ok && c.wg == 0 && c.t == 0) {
        Pp->tok_out[s] = tok;
        Pp->ctl[CTL_DONE] = (uint32_t)(s + 1);
        Pp->ctl[CTL_LAST] = (uint32_t)tok;
      }
      break;
    }
  }
  (void)ok;  // a failed poll has recorded its status in the control words
}

// ---------------------------------------------------------------------------
// Isolated GEMV probe: y[i] = W[i % ncopy] x[i], rows split over the grid,
// one launch for all vectors.  Same engine as the decode stages.
//
// INPUT_FIRST = false (stage order): each product issues its first weight
// block, then reads its input vector, as a decode stage whose weights were
// prefetched before its input arrived by hand-off.  Loads return in issue
// order, so the input waits behind that block.
// INPUT_FIRST = true: each product reads its input vector first and issues
// the whole weight block right behind it (the order when the input is at
// hand), so the input returns one round trip later while the weights stream.
// ---------------------------------------------------------------------------
constexpr int kProbeXv = 4;  // input vectors per thread: cols <= 16384 = 4 * 512 * 8

template <int DT>
__device__ __forceinline__ void probe_x_to_lds(uint16_t* xs, const uint4 (&xv)[kProbeXv], int nv8, int t) {
  constexpr int AW = kActWords<DT>;  // the probe's input is 16-bit already: bf16 residual terms are zero
#pragma unroll
  for (int k = 0; k < kProbeXv; ++k) {
    const int i = t + k * kThreads;
    if (i < nv8) {
      reinterpret_cast<uint4*>(xs)[i * AW] = xv[k];
      for (int a = 1; a < AW; ++a) reinterpret_cast<uint4*>(xs)[i * AW + a] = make_uint4(0, 0, 0, 0);
    }
  }
}

template <int DT, bool INPUT_FIRST>
__global__ __launch_bounds__(kThreads, 1) void gemv_probe(const uint16_t* W, int rows, int cols, int ncopy,
                                                          const uint16_t* x, float* y, int nvec) {
  extern __shared__ __align__(16) char smem[];
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
  float* red = reinterpret_cast<float*>(smem + (size_t)cols * 2 * kActWords<DT>);
  float* yv = red + kRedCap;
  const int nb = gridDim.x, wg = blockIdx.x;
  const int r0 = split_lo(rows, nb, wg), r1 = split_lo(rows, nb, wg + 1);
  const int nv8 = cols >> 3;
  for (int iv = 0; iv < nvec; ++iv) {
    const int t = opaque_v((int)threadIdx.x);
    StagePlan pl = plan_rows(r1 - r0, cols, t);
    pl.seg0 = W + (size_t)(iv % ncopy) * rows * cols + (size_t)r0 * cols;
    auto prep = [&](auto fill) -> bool {
      const uint4* src = reinterpret_cast<const uint4*>(x + (size_t)iv * cols);
      uint4 xv[kProbeXv];
#pragma unroll
      for (int k = 0; k < kProbeXv; ++k) {
        const int i = t + k * kThreads;
        xv[k] = i < nv8 ? src[i] : make_uint4(0, 0, 0, 0);
      }
      fill();  // the rest of the ring (all of it with INPUT_FIRST) right behind the input's loads
      probe_x_to_lds<DT>(xs, xv, nv8, t);
      __syncthreads();
      return true;
    };
    uint4 ring[kDepth];
    gemv_any<DT, INPUT_FIRST ? 0 : kDepth>(pl, prep, xs, red, yv, t, ring, false, StagePlan{});
    for (int r = t; r < r1 - r0; r += kThreads) y[(size_t)iv * rows + r0 + r] = yv[r];
    __syncthreads();
  }
}

}  // namespace kie
