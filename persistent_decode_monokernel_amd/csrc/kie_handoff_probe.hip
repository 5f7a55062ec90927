// Hand-off latency probe: the decode kernel's exchange form (8-byte
// agent-scope stores, polled with agent-scope loads and s_sleep 1 between
// polls) timed alone, as a ping between two work-groups or as an all-to-all
// round across the grid, with and without weight-style streaming beside it.
#include "kie_device.hpp"

#include <cstdio>
#include <cstdlib>
#include <vector>

namespace kie {
namespace {

constexpr uint64_t kWaitLimit = 1000000;     // ticks of the 100 MHz counter per wait (10 ms)
constexpr uint64_t kStreamLimit = 20000000;  // streamers stop after 200 ms at the latest
constexpr int kChunk = 32;                   // ring iterations between checks of the stop flag
constexpr int kRecWords = 6;                 // per work-group record

// Scratch layout in 8-byte words.
constexpr int kAbortW = 0;         // set by a wait that ran out of time
constexpr int kDoneW = 1;          // the exchange finished: streamers elsewhere stop
constexpr int kSinkW = 2;          // keeps the streamed data live
constexpr int kPingW = 16;         // work-group a's word; b's is 16 words (128 B) further
constexpr int kSlotW = 64;         // all-to-all: one word per work-group, `stride` words apart;
                                   // the records follow the slots (exchange ticks, XCC id,
                                   // stream start, end, vectors streamed, ok)
constexpr int kMaxStride = 16;

struct ProbeArgs {
  const uint4* buf;
  uint64_t nvec;
  uint64_t* s;    // scratch, zeroed before the launch
  uint64_t* rec;  // s + kSlotW + stride * grid
  int kind, a, b, rounds, where, stride;
};

__device__ __forceinline__ uint64_t now() { return __builtin_amdgcn_s_memrealtime(); }
__device__ __forceinline__ uint64_t ld(const uint64_t* p) { return xld64(reinterpret_cast<const uint32_t*>(p)); }
__device__ __forceinline__ void st(uint64_t* p, uint64_t v) { xst64(reinterpret_cast<uint32_t*>(p), v); }

// Wait until *p >= r; false on timeout (then the abort word is set) or abort.
__device__ __forceinline__ bool wait_ge(const uint64_t* p, uint64_t r, uint64_t* s) {
  if (ld(p) >= r) return true;
  const uint64_t t0 = now();
  for (int n = 1;; ++n) {
    __builtin_amdgcn_s_sleep(1);
    if (ld(p) >= r) return true;
    if ((n & 15) == 0 && ld(s + kAbortW) != 0) return false;
    if (now() - t0 > kWaitLimit) {
      st(s + kAbortW, 1);
      return false;
    }
  }
}

// Two work-groups, one thread each: a stores round r, b answers r once it
// sees it.  Rounds 1 and 2 are untimed; a's record holds the ticks of the rest.
__device__ __forceinline__ void ping(const ProbeArgs& p, bool is_a, uint64_t warm) {
  uint64_t* mine = p.s + kPingW + (is_a ? 0 : 16);
  const uint64_t* theirs = p.s + kPingW + (is_a ? 16 : 0);
  const uint64_t t0 = now();
  while (now() - t0 < warm) __builtin_amdgcn_s_sleep(10);
  bool ok = true;
  uint64_t ts = now();
  for (int r = 1; r <= p.rounds + 2 && ok; ++r) {
    if (r == 3) ts = now();
    if (is_a) st(mine, r);
    ok = wait_ge(theirs, r, p.s);
    if (!is_a && ok) st(mine, r);
  }
  const uint64_t te = now();
  uint64_t* rec = p.rec + (uint64_t)blockIdx.x * kRecWords;
  if (is_a) {
    rec[0] = ok ? te - ts : 0;
    st(p.s + kDoneW, 1);
  }
  rec[5] = ok ? 1 : 0;
}

// Wave 0 of every work-group: lane 0 publishes round r in the work-group's
// slot, every lane polls its grid/64 slots together (loads issued before any
// is checked), re-polling only those still behind.
__device__ __forceinline__ void all_to_all(const ProbeArgs& p, int grid) {
  const int lane = threadIdx.x;
  constexpr int kMaxPer = kMaxWG / 64;
  const int per = (grid + 63) / 64;
  bool ok = true;
  uint64_t ts = now();
  for (int r = 1; r <= p.rounds + 2 && ok; ++r) {
    if (r == 3) ts = now();
    if (lane == 0) st(p.s + kSlotW + (uint64_t)blockIdx.x * p.stride, r);
    bool rdy[kMaxPer];
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j) rdy[j] = j >= per || lane + 64 * j >= grid;
    bool failed = false;
    const uint64_t tw = now();
    for (int n = 1;; ++n) {
      // Every word of the lane is re-read each round, under a scalar test
      // only (per is the same for the whole grid): with the loads under a
      // per-lane test, the compiler waited for each load before issuing the
      // next, and a round cost one memory round trip per word.
      uint64_t v[kMaxPer];
#pragma unroll
      for (int j = 0; j < kMaxPer; ++j)
        if (j < per) v[j] = ld(p.s + kSlotW + (uint64_t)min(lane + 64 * j, grid - 1) * p.stride);
      __builtin_amdgcn_sched_barrier(0);
      bool all = true;
#pragma unroll
      for (int j = 0; j < kMaxPer; ++j) {
        if (j < per) rdy[j] = rdy[j] || v[j] >= (uint64_t)r;
        all = all && rdy[j];
      }
      if (all) break;
      if ((n & 15) == 0 && ld(p.s + kAbortW) != 0) { failed = true; break; }
      if (now() - tw > kWaitLimit) {
        st(p.s + kAbortW, 1);
        failed = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    ok = __ballot(failed) == 0;
  }
  const uint64_t te = now();
  if (lane == 0) {
    uint64_t* rec = p.rec + (uint64_t)blockIdx.x * kRecWords;
    rec[0] = ok ? te - ts : 0;
    rec[5] = ok ? 1 : 0;
  }
}

// nt threads (index tt) stream the work-group's contiguous share in chunks of
// (kChunk + 1) * D slots of nt vectors, D non-temporal dwordx4 loads in flight
// per thread, wrapping within the share; between chunks they check the stop
// condition.  The host guarantees a share of at least one chunk.
template <int D>
__device__ __forceinline__ void stream(const ProbeArgs& p, int grid, int nt, int tt, volatile uint32_t* lds_stop, bool own) {
  const uint64_t share = p.nvec / grid, base = share * blockIdx.x, nslot = share / nt;
  constexpr uint64_t kSpan = (uint64_t)(kChunk + 1) * D;
  const uint64_t t0 = now();
  uint32_t acc = 0;
  uint64_t slot = 0, chunks = 0;
  for (;;) {
    if (slot + kSpan > nslot) slot = 0;
    const uint4* q = p.buf + base + slot * nt + tt;
    uint4 ring[D];
#pragma unroll
    for (int k = 0; k < D; ++k) ring[k] = ldw(reinterpret_cast<const uint16_t*>(q + (uint64_t)k * nt));
#pragma unroll 1
    for (int c = 1; c <= kChunk; ++c) {
      q += (uint64_t)D * nt;
#pragma unroll
      for (int k = 0; k < D; ++k) {
        acc ^= ring[k].x ^ ring[k].y ^ ring[k].z ^ ring[k].w;
        ring[k] = ldw(reinterpret_cast<const uint16_t*>(q + (uint64_t)k * nt));
      }
    }
#pragma unroll
    for (int k = 0; k < D; ++k) acc ^= ring[k].x ^ ring[k].y ^ ring[k].z ^ ring[k].w;
    slot += kSpan;
    ++chunks;
    const bool stop = own ? *lds_stop != 0 : (ld(p.s + kDoneW) != 0 || ld(p.s + kAbortW) != 0);
    if (stop || now() - t0 > kStreamLimit) break;
  }
  if (tt == 0) {
    uint64_t* rec = p.rec + (uint64_t)blockIdx.x * kRecWords;
    rec[2] = t0;
    rec[3] = now();
    rec[4] = chunks * kSpan * nt;
  }
  if (acc == 0x9E3779B9u) p.s[kSinkW] = acc;  // practically never: keeps the loads
}

template <int D>
__global__ __launch_bounds__(kThreads, 1) void handoff_probe(ProbeArgs p) {
  __shared__ uint32_t lds_stop;
  const int wg = blockIdx.x, t = threadIdx.x, grid = gridDim.x;
  if (t == 0) lds_stop = 0;
  __syncthreads();
  const bool exch = p.kind == KIE_PROBE_ALL_TO_ALL || wg == p.a || wg == p.b;
  const bool own = (p.where & KIE_PROBE_STREAM_OWN) != 0;
  const bool others = (p.where & KIE_PROBE_STREAM_OTHERS) != 0;
  if (exch && t == 0)
    p.rec[(uint64_t)wg * kRecWords + 1] = __builtin_amdgcn_s_getreg((3 << 11) | 20);  // HW_REG_XCC_ID[3:0]
  if (exch) {
    if (t < 64) {
      if (p.kind == KIE_PROBE_ALL_TO_ALL) all_to_all(p, grid);
      else if (t == 0) ping(p, wg == p.a, p.where != KIE_PROBE_STREAM_NONE ? 3000 : 500);
      if (t == 0) *(volatile uint32_t*)&lds_stop = 1;
    } else if (own) {
      stream<D>(p, grid, kThreads - 64, t - 64, &lds_stop, true);
    }
  } else if (others) {
    stream<D>(p, grid, kThreads, t, &lds_stop, false);
  }
}

const void* handoff_probe_fn(int depth) {
  switch (depth) {
    case 1: return reinterpret_cast<const void*>(&handoff_probe<1>);
    case 2: return reinterpret_cast<const void*>(&handoff_probe<2>);
    case 3: return reinterpret_cast<const void*>(&handoff_probe<3>);
    case 4: return reinterpret_cast<const void*>(&handoff_probe<4>);
    case 8: return reinterpret_cast<const void*>(&handoff_probe<8>);
  }
  return nullptr;
}

__global__ void zero_words(uint64_t* p, uint64_t n) {
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (uint64_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

}  // namespace
}  // namespace kie

using namespace kie;

#define PROBE_HIP(call)                                  \
  do {                                                   \
    hipError_t e_ = (call);                              \
    if (e_ != hipSuccess) {                              \
      if (getenv("KIE_VERBOSE"))                         \
        fprintf(stderr, "kie: %s failed: %s\n", #call, hipGetErrorString(e_)); \
      return KIE_ERR_HIP;                                \
    }                                                    \
  } while (0)

extern "C" kie_status kie_handoff_probe(int32_t kind, int32_t wg_a, int32_t wg_b, int32_t rounds,
                                        int32_t slot_stride, int32_t stream_depth, int32_t stream_where, const void* buf_dev,
                                        size_t bytes, uint64_t* scratch_dev, size_t scratch_bytes,
                                        void* hip_stream, kie_handoff_probe_result* out) {
  if (!out || !scratch_dev || (reinterpret_cast<uintptr_t>(scratch_dev) & 7)) return KIE_ERR_ARG;
  if (kind != KIE_PROBE_PING && kind != KIE_PROBE_ALL_TO_ALL) return KIE_ERR_ARG;
  if (rounds < 1 || rounds > 100000 || stream_where < 0 || stream_where > 3) return KIE_ERR_ARG;
  if (slot_stride < 1 || slot_stride > kMaxStride || (slot_stride & (slot_stride - 1))) return KIE_ERR_ARG;
  if (kind == KIE_PROBE_ALL_TO_ALL && (stream_where & KIE_PROBE_STREAM_OTHERS)) return KIE_ERR_ARG;
  const bool streams = stream_where != KIE_PROBE_STREAM_NONE;
  const void* fn = handoff_probe_fn(streams ? stream_depth : 1);
  if (!fn) return KIE_ERR_ARG;
  if (streams && (!buf_dev || (reinterpret_cast<uintptr_t>(buf_dev) & 15))) return KIE_ERR_ARG;
  int dev = 0;
  PROBE_HIP(hipGetDevice(&dev));
  hipDeviceProp_t prop;
  PROBE_HIP(hipGetDeviceProperties(&prop, dev));
  const int grid = prop.multiProcessorCount < kMaxWG ? prop.multiProcessorCount : kMaxWG;
  if (kind == KIE_PROBE_PING && (wg_a < 0 || wg_b < 0 || wg_a >= grid || wg_b >= grid || wg_a == wg_b))
    return KIE_ERR_ARG;
  const uint64_t rec_w = kSlotW + (uint64_t)slot_stride * grid;
  const size_t need = (size_t)(rec_w + (uint64_t)kRecWords * grid) * 8;
  if (scratch_bytes < need) return KIE_ERR_CAPACITY;
  // every streaming work-group's share holds at least one chunk of slots of
  // 512 vectors (the wider of the two streaming widths, 512 and 448 threads)
  if (streams && bytes / 16 / grid / kThreads < (uint64_t)(kChunk + 1) * stream_depth) return KIE_ERR_CAPACITY;
  int khz = 0;
  PROBE_HIP(hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev));
  if (khz <= 0) khz = 100000;

  hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
  const uint64_t nwords = need / 8;
  hipLaunchKernelGGL(zero_words, dim3(64), dim3(256), 0, st, scratch_dev, nwords);
  PROBE_HIP(hipGetLastError());
  ProbeArgs p{reinterpret_cast<const uint4*>(buf_dev), streams ? bytes / 16 : 0, scratch_dev, scratch_dev + rec_w,
              kind, kind == KIE_PROBE_PING ? wg_a : -1, kind == KIE_PROBE_PING ? wg_b : -1, rounds, stream_where,
              slot_stride};
  void* args[] = {&p};
  PROBE_HIP(hipLaunchCooperativeKernel(fn, dim3(grid), dim3(kThreads), args, 0, st));
  std::vector<uint64_t> rec((size_t)kRecWords * grid), hdr(2);
  PROBE_HIP(hipMemcpyAsync(rec.data(), scratch_dev + rec_w, rec.size() * 8, hipMemcpyDeviceToHost, st));
  PROBE_HIP(hipMemcpyAsync(hdr.data(), scratch_dev, 16, hipMemcpyDeviceToHost, st));
  PROBE_HIP(hipStreamSynchronize(st));

  const double us_per_tick = 1000.0 / khz;
  kie_handoff_probe_result r{};
  r.grid = grid;
  r.completed = hdr[kAbortW] == 0;
  if (kind == KIE_PROBE_PING) {
    r.exchange_us = rec[(size_t)wg_a * kRecWords] * us_per_tick / rounds;
    r.exchange_max_us = r.exchange_us;
    r.xcc_a = (int32_t)rec[(size_t)wg_a * kRecWords + 1];
    r.xcc_b = (int32_t)rec[(size_t)wg_b * kRecWords + 1];
  } else {
    double sum = 0, mx = 0;
    for (int w = 0; w < grid; ++w) {
      const double us = rec[(size_t)w * kRecWords] * us_per_tick / rounds;
      sum += us;
      mx = us > mx ? us : mx;
      if (rec[(size_t)w * kRecWords + 5] == 0) r.completed = 0;
    }
    r.exchange_us = sum / grid;
    r.exchange_max_us = mx;
    r.xcc_a = (int32_t)rec[1];
    r.xcc_b = grid > 1 ? (int32_t)rec[kRecWords + 1] : r.xcc_a;
  }
  uint64_t t0 = ~0ull, t1 = 0, vec = 0;
  for (int w = 0; w < grid; ++w) {
    const uint64_t* q = &rec[(size_t)w * kRecWords];
    if (q[4] == 0) continue;
    t0 = q[2] < t0 ? q[2] : t0;
    t1 = q[3] > t1 ? q[3] : t1;
    vec += q[4];
  }
  if (vec && t1 > t0) r.stream_gbps = vec * 16.0 / ((t1 - t0) * us_per_tick * 1e-6) / 1e9;
  *out = r;
  return KIE_OK;
}
