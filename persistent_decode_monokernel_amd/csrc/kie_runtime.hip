// Host runtime behind include/kie.h: validation, workspace layout, the rotary
// table, weight registration, the persistent launches, status mapping.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "kie.h"
#include "kie_params.hpp"
#include "kie_prefill.hpp"
#include "kie_tiling.hpp"

namespace kie {
const void* monokernel_fn_f16_g1(int vd, int vf);
const void* monokernel_fn_f16_g2(int vd, int vf);
const void* monokernel_fn_f16_g4(int vd, int vf);
const void* monokernel_fn_f16_g8(int vd, int vf);
const void* monokernel_fn_bf16_g1(int vd, int vf);
const void* monokernel_fn_bf16_g2(int vd, int vf);
const void* monokernel_fn_bf16_g4(int vd, int vf);
const void* monokernel_fn_bf16_g8(int vd, int vf);
const void* monokernel_counters_fn_f16_g4(int vd, int vf);
const void* monokernel_counters_fn_bf16_g4(int vd, int vf);
const void* stage_kernel_fn_f16_g1(int vd, int vf);
const void* stage_kernel_fn_f16_g2(int vd, int vf);
const void* stage_kernel_fn_f16_g4(int vd, int vf);
const void* stage_kernel_fn_f16_g8(int vd, int vf);
const void* stage_kernel_fn_bf16_g1(int vd, int vf);
const void* stage_kernel_fn_bf16_g2(int vd, int vf);
const void* stage_kernel_fn_bf16_g4(int vd, int vf);
const void* stage_kernel_fn_bf16_g8(int vd, int vf);
const void* gemv_probe_fn(int dtype, bool input_first);
const void* stream_probe_fn(int depth);
hipError_t launch_fill(uint32_t* p, uint64_t n, uint32_t v, hipStream_t st);
}  // namespace kie

using namespace kie;

namespace {

constexpr uint64_t kDefaultTimeout = 200000000ull;  // 2 s at 100 MHz

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool pow2_between(int v, int lo, int hi) { return v >= lo && v <= hi && (v & (v - 1)) == 0; }

// A GEMV input width the engine tiles: a power of two in [256, 4096] (rows of
// <= 512 vectors) or a multiple of 256 up to 16384 (rows of up to 4 vectors per
// thread).
bool k_ok(int k) { return pow2_between(k, 256, 4096) || (k > 4096 && k <= 16384 && k % 256 == 0); }

int attn_cmax(const kie_config& c) {
  int m = kAttnUnits / c.n_kv_heads;
  return m < 1 ? 1 : m;
}

int attn_cl_cap(const kie_config& c) {
  const int cmax = attn_cmax(c);
  int cl = (c.max_seq + cmax - 1) / cmax;
  return cl < kClMin ? kClMin : cl;
}

XchLayout xch_layout(const kie_config& c) {
  XchLayout x{};
  const uint64_t L = c.n_layers, d = c.d_model, qd = (uint64_t)c.n_heads * c.head_dim, F = c.d_ffn;
  uint64_t o = 0;
  auto take = [&](uint64_t words) {
    const uint64_t at = o;
    o = align_up(o + words, 4);
    return at;
  };
  x.xmid = take(L * d);
  x.xout = take(L * d);
  x.qkv = take(L * (qd + 2ull * c.n_kv_heads * c.head_dim));
  x.a = take(L * qd);
  x.h = take(L * F);
  x.arg = take(2 * (uint64_t)kMaxWG);
  x.cand = take(2ull * kMaxWG * kCand);
  x.cand2 = take(2ull * (kMaxWG / 8) * kCand);
  x.stok = take(2);
  x.cnt = take(L * kStagesPerLayer + 1);
  x.dense = o;
  x.att = take(L * c.n_heads * (uint64_t)attn_cmax(c) * (c.head_dim + 4));
  x.words = align_up(o, 64);
  return x;
}

struct Layout {
  size_t params, rope, lw, kc, vc, xch, ctl, tok, forced, total;
  size_t pf_x, pf_xn, pf_qkv, pf_a, pf_h, pf_p;  // matrix-core prompt path (0 bytes when unsupported)
  int pf_chunk;
  size_t kv_plane_bytes;
  XchLayout xl;
};

Layout make_layout(const kie_config& c) {
  Layout y{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  y.kv_plane_bytes = (size_t)c.n_layers * c.n_kv_heads * c.max_seq * c.head_dim * 2;
  y.xl = xch_layout(c);
  y.params = take(sizeof(Params));
  y.rope = take((size_t)c.max_seq * (c.head_dim / 2) * 2 * sizeof(float));
  y.lw = take((size_t)c.n_layers * W_PER_LAYER * sizeof(void*));
  y.kc = take(y.kv_plane_bytes);
  y.vc = take(y.kv_plane_bytes);
  y.xch = take((size_t)kRingSets * y.xl.words * 4);
  y.ctl = take(CTL_WORDS * 4);
  y.tok = take((size_t)c.max_seq * 4);
  y.forced = take((size_t)c.max_seq * 4);
  y.pf_chunk = prefill_supported(c) ? (c.max_seq < kPfChunk ? c.max_seq : kPfChunk) : 0;
  {
    const size_t pc = (size_t)y.pf_chunk, qd = (size_t)c.n_heads * c.head_dim, kvd = (size_t)c.n_kv_heads * c.head_dim;
    const size_t ab = y.pf_chunk > 0 ? prefill_act_bytes(c) : 0;  // activation element: fp16, or fp32 (bf16)
    y.pf_x = take(pc * c.d_model * 4);
    y.pf_xn = take(pc * c.d_model * ab);
    y.pf_qkv = take(pc * (qd + 2 * kvd) * 4);
    y.pf_a = take(pc * qd * ab);
    y.pf_h = take(pc * c.d_ffn * ab);
    y.pf_p = take(y.pf_chunk > 0 ? prefill_part_floats(c, y.pf_chunk) * 4 : 0);
  }
  y.total = o;
  return y;
}

struct LdsPlan {
  int xres, xn, scr, misc, bytes;
};

LdsPlan lds_plan(const kie_config& c) {
  LdsPlan p{};
  const int qd = c.n_heads * c.head_dim;
  int kmax = c.d_model;
  if (qd > kmax) kmax = qd;
  if (c.d_ffn > kmax) kmax = c.d_ffn;
  const int G = c.n_heads / c.n_kv_heads;
  const size_t gemv_scr = (size_t)(kRedCap + kYCap) * 4;
  // attention scratch, from the xn offset over xn and scr: rotated queries
  // [G][hd], the new row [2][hd] 16-bit, per lane group (m, l) and o for up
  // to 4 heads at once (2 when 8 query heads share a KV head), lane groups = 512 / (hd / 8)
  const size_t hb = G < 4 ? G : G == 8 ? 2 : 4, groups = (size_t)kThreads / (c.head_dim / 8);
  const size_t attn_scr = ((size_t)G * c.head_dim + (size_t)c.head_dim + groups * hb * 2 +
                           groups * hb * c.head_dim) * 4;
  size_t o = 0;
  p.xres = 0;
  o = align_up((size_t)c.d_model * 4, 16);
  p.xn = (int)o;
  const size_t xn_bytes = align_up((size_t)kmax * 2 * (c.dtype == KIE_BF16 ? 3 : 1), 16);  // bf16: three terms
  o += xn_bytes;
  p.scr = (int)o;
  const size_t scr_bytes = attn_scr > xn_bytes + gemv_scr ? attn_scr - xn_bytes : gemv_scr;
  o = align_up(o + scr_bytes, 16);
  p.misc = (int)o;
  o += 128 * 4;
  p.bytes = (int)o;
  return p;
}

// GEMV width class of an input width K: 0 for K < 512 (32 lanes per row),
// else the vectors each thread reads per row (1, 2 or 4).
int width_class(int K) {
  const int vpr = K / 8;
  return vpr < 64 ? 0 : vectors_per_lane(vpr);
}

// The kernel instance for a shape: dtype, query heads per KV head, width class
// of d_model (= that of n_heads*head_dim) and of d_ffn.
const void* monokernel_fn(const kie_config& c) {
  const int G = c.n_heads / c.n_kv_heads, vd = width_class(c.d_model), vf = width_class(c.d_ffn);
  const bool f16 = c.dtype == KIE_F16;
  switch (G) {
    case 1: return f16 ? monokernel_fn_f16_g1(vd, vf) : monokernel_fn_bf16_g1(vd, vf);
    case 2: return f16 ? monokernel_fn_f16_g2(vd, vf) : monokernel_fn_bf16_g2(vd, vf);
    case 4: return f16 ? monokernel_fn_f16_g4(vd, vf) : monokernel_fn_bf16_g4(vd, vf);
    case 8: return f16 ? monokernel_fn_f16_g8(vd, vf) : monokernel_fn_bf16_g8(vd, vf);
  }
  return nullptr;
}

// The arrival-counter instance of a shape, or null where none is built.
const void* monokernel_counters_fn(const kie_config& c) {
  const int G = c.n_heads / c.n_kv_heads, vd = width_class(c.d_model), vf = width_class(c.d_ffn);
  if (G != 4) return nullptr;
  return c.dtype == KIE_F16 ? monokernel_counters_fn_f16_g4(vd, vf) : monokernel_counters_fn_bf16_g4(vd, vf);
}

// The per-stage instance of the same shape (one launch per stage).
const void* stage_kernel_fn(const kie_config& c) {
  const int G = c.n_heads / c.n_kv_heads, vd = width_class(c.d_model), vf = width_class(c.d_ffn);
  const bool f16 = c.dtype == KIE_F16;
  switch (G) {
    case 1: return f16 ? stage_kernel_fn_f16_g1(vd, vf) : stage_kernel_fn_bf16_g1(vd, vf);
    case 2: return f16 ? stage_kernel_fn_f16_g2(vd, vf) : stage_kernel_fn_bf16_g2(vd, vf);
    case 4: return f16 ? stage_kernel_fn_f16_g4(vd, vf) : stage_kernel_fn_bf16_g4(vd, vf);
    case 8: return f16 ? stage_kernel_fn_f16_g8(vd, vf) : stage_kernel_fn_bf16_g8(vd, vf);
  }
  return nullptr;
}

}  // namespace

struct kie_engine {
  kie_config cfg{};
  Layout lay{};
  LdsPlan lds{};
  int device = 0;
  int cu_count = 0;
  int grid = 0;
  hipStream_t stream = nullptr;
  char* ws = nullptr;
  bool have_weights = false;
  const uint16_t* tok_emb = nullptr;
  const uint16_t* final_norm = nullptr;
  const uint16_t* lm_head = nullptr;
  bool have_seq = false;
  int pos = 0;
  int pending = -1;
  uint64_t timeout = kDefaultTimeout;
  int abort_after = -1;
  int withhold_wg = -1;
  int delay_wg = -1;          // race test: work-group whose publications are delayed
  int handoff = kHandoffNan;  // hand-off protocol of the persistent launches
  int launch_mode = KIE_LAUNCH_PERSISTENT;  // kie_decode: persistent kernel or one launch per stage
  uint64_t delay_ticks = 0;
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  float last_ms = 0.f;
  int last_steps = 0;
  Params params_host{};
  uint64_t* trace = nullptr;
  int trace_step = 0;
  std::vector<const uint16_t*> wtab;  // host copy of the per-layer weight table
  int prefill_mode = KIE_PREFILL_AUTO;
  int prefill_chunk = 0;  // positions per matrix-core chunk; 0 = the workspace's (lay.pf_chunk)
  int samp_k = 0;         // sampling (kie_set_sampling); 0 = greedy
  float samp_scale = 0.f, samp_top_p = 1.f;
  uint64_t samp_seed = 0;
  bool is_static = false;  // static storage on the static workspace (kie_create_static)
};

extern "C" const char* kie_status_string(kie_status s) {
  switch (s) {
    case KIE_OK: return "ok";
    case KIE_ERR_ARG: return "invalid argument";
    case KIE_ERR_STATE: return "call out of order";
    case KIE_ERR_CAPACITY: return "capacity exceeded";
    case KIE_ERR_UNSUPPORTED: return "unsupported shape";
    case KIE_ERR_HIP: return "HIP runtime error";
    case KIE_ERR_TIMEOUT: return "device poll timed out";
    case KIE_ERR_ABORTED: return "aborted on request";
  }
  return "unknown status";
}

extern "C" kie_status kie_config_validate(const kie_config* c) {
  if (!c) return KIE_ERR_ARG;
  if (c->n_layers < 1 || c->d_model < 1 || c->n_heads < 1 || c->n_kv_heads < 1 || c->head_dim < 1 ||
      c->d_ffn < 1 || c->vocab < 1 || c->max_seq < 1)
    return KIE_ERR_ARG;
  if (!(c->rms_eps > 0.f) || !std::isfinite(c->rms_eps) || !(c->rope_base > 1.f) || !std::isfinite(c->rope_base))
    return KIE_ERR_ARG;
  if (c->dtype != KIE_F16 && c->dtype != KIE_BF16) return KIE_ERR_ARG;
  if (c->head_dim != 64 && c->head_dim != 128) return KIE_ERR_UNSUPPORTED;
  if (c->n_heads % c->n_kv_heads != 0) return KIE_ERR_UNSUPPORTED;
  const int G = c->n_heads / c->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return KIE_ERR_UNSUPPORTED;
  if (c->n_kv_heads > kAttnUnits) return KIE_ERR_UNSUPPORTED;
  if (!k_ok(c->d_model) || !k_ok(c->n_heads * c->head_dim) || !k_ok(c->d_ffn)) return KIE_ERR_UNSUPPORTED;
  // compiled kernel instances: d_model <= 4096 with n_heads*head_dim in the
  // same width class, d_ffn >= 512 in a class at least d_model's
  {
    const int vd = width_class(c->d_model), vf = width_class(c->d_ffn);
    if (c->d_model > 4096 || width_class(c->n_heads * c->head_dim) != vd || vf == 0 || vf < vd)
      return KIE_ERR_UNSUPPORTED;
  }
  if ((long long)c->vocab * c->d_model >= (1ll << 40)) return KIE_ERR_UNSUPPORTED;
  if (lds_plan(*c).bytes > 160 * 1024) return KIE_ERR_UNSUPPORTED;
  return KIE_OK;
}

extern "C" size_t kie_workspace_bytes(const kie_config* c) {
  if (kie_config_validate(c) != KIE_OK) return 0;
  return make_layout(*c).total;
}

static kie_status hip_fail(hipError_t e, const char* what) {
  if (getenv("KIE_VERBOSE")) fprintf(stderr, "kie: %s failed: %s\n", what, hipGetErrorString(e));
  return KIE_ERR_HIP;
}

#define KIE_HIP(call)                                      \
  do {                                                     \
    hipError_t e_ = (call);                                \
    if (e_ != hipSuccess) return hip_fail(e_, #call);      \
  } while (0)

// Can `grid` work-groups run the shape: every GEMV stage's rows per
// work-group fit the LDS partial sums, the step tail's gather covers the grid,
// and the index arithmetic stays within 32 bits.
static bool grid_fits(const kie_config& c, const Layout& lay, int grid) {
  if (grid < 1 || grid > kMaxWG || grid > kThreads / 2) return false;
  // every work-group owns a row of each vector a hand-off polls (the
  // exchange-set recycling relies on it) and of every GEMV stage (the weight
  // ring is filled without a per-work-group test)
  if (grid > c.d_model || grid > c.d_ffn || grid > c.vocab) return false;
  auto fits = [&](long long rows, int K) {
    const int vpr = K / 8, lpr = vpr < kThreads ? vpr : kThreads, nwr = lpr >= 64 ? lpr / 64 : 1;
    return rows <= kYCap && rows * nwr <= kRedCap;
  };
  auto per = [&](long long n) { return (n + grid - 1) / grid; };
  const long long qkv = (long long)(c.n_heads + 2 * c.n_kv_heads) * c.head_dim;
  return fits(per(qkv), c.d_model) && fits(per(c.d_model), c.n_heads * c.head_dim) &&
         fits(2 * per(c.d_ffn), c.d_model) && fits(per(c.d_model), c.d_ffn) && fits(per(c.vocab), c.d_model) &&
         (uint64_t)c.vocab * grid < (1ull << 32) && (lay.xl.dense / 2) * grid < (1ull << 32) &&
         (uint64_t)c.d_ffn * grid < (1ull << 32);
}

// Rotary table, built in double precision (angle(p, i) = p * base^(-2i/hd)),
// copied to the device in pieces through a stack buffer (no host allocation).
static hipError_t write_rope(const kie_config& c, char* dst_dev, hipStream_t st) {
  const int half = c.head_dim / 2;
  constexpr int kChunk = 4096;  // floats per piece
  float buf[kChunk];
  const size_t total = (size_t)c.max_seq * half * 2;
  for (size_t at = 0; at < total; at += kChunk) {
    const size_t n = total - at < (size_t)kChunk ? total - at : (size_t)kChunk;
    for (size_t k = 0; k < n; k += 2) {
      const size_t e = (at + k) / 2;
      const int p = (int)(e / half), i = (int)(e % half);
      const double ang = (double)p * std::pow((double)c.rope_base, -2.0 * i / c.head_dim);
      buf[k] = (float)std::cos(ang);
      buf[k + 1] = (float)std::sin(ang);
    }
    hipError_t he = hipMemcpyAsync(dst_dev + at * sizeof(float), buf, n * sizeof(float), hipMemcpyHostToDevice, st);
    if (he == hipSuccess) he = hipStreamSynchronize(st);  // buf is reused by the next piece
    if (he != hipSuccess) return he;
  }
  return hipSuccess;
}

// Engine construction shared by kie_create and kie_create_static: `e` is
// default-constructed storage the caller owns; with_events creates the HIP
// events that time each persistent launch.
static kie_status create_impl(kie_engine* e, const kie_config* cfg, void* workspace_dev, size_t ws_bytes,
                              void* hip_stream, bool with_events) {
  const kie_status v = kie_config_validate(cfg);
  if (v != KIE_OK) return v;
  if (!workspace_dev || (reinterpret_cast<uintptr_t>(workspace_dev) & 255) != 0) return KIE_ERR_ARG;
  const Layout lay = make_layout(*cfg);
  if (ws_bytes < lay.total) return KIE_ERR_CAPACITY;

  int dev = 0;
  KIE_HIP(hipGetDevice(&dev));
  hipDeviceProp_t prop;
  KIE_HIP(hipGetDeviceProperties(&prop, dev));
  int coop = 0;
  KIE_HIP(hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev));
  if (!coop) return KIE_ERR_UNSUPPORTED;

  e->cfg = *cfg;
  e->lay = lay;
  e->lds = lds_plan(*cfg);
  e->device = dev;
  e->cu_count = prop.multiProcessorCount;
  e->stream = reinterpret_cast<hipStream_t>(hip_stream);
  e->ws = reinterpret_cast<char*>(workspace_dev);

  const void* fn = monokernel_fn(*cfg);
  hipError_t he = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, e->lds.bytes);
  // the arrival-counter instance, where this shape has one
  if (he == hipSuccess && monokernel_counters_fn(*cfg))
    he = hipFuncSetAttribute(monokernel_counters_fn(*cfg), hipFuncAttributeMaxDynamicSharedMemorySize, e->lds.bytes);
  int per_cu = 0;
  if (he == hipSuccess) he = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, e->lds.bytes);
  if (he != hipSuccess) return hip_fail(he, "occupancy");
  if (per_cu < 1) return KIE_ERR_UNSUPPORTED;
  he = hipFuncSetAttribute(stage_kernel_fn(*cfg), hipFuncAttributeMaxDynamicSharedMemorySize, e->lds.bytes);
  if (he != hipSuccess) return hip_fail(he, "stage kernel");
  // One resident work-group per compute unit.
  e->grid = e->cu_count < kMaxWG ? e->cu_count : kMaxWG;
  if (!grid_fits(*cfg, lay, e->grid)) return KIE_ERR_UNSUPPORTED;

  he = write_rope(*cfg, e->ws + lay.rope, e->stream);
  if (he == hipSuccess) he = launch_fill(reinterpret_cast<uint32_t*>(e->ws + lay.ctl), CTL_WORDS, 0u, e->stream);
  if (he == hipSuccess && with_events) he = hipEventCreate(&e->ev0);
  if (he == hipSuccess && with_events) he = hipEventCreate(&e->ev1);
  if (he == hipSuccess) he = hipStreamSynchronize(e->stream);
  if (he != hipSuccess) return hip_fail(he, "create");
  return KIE_OK;
}

static void release_events(kie_engine* e) {
  if (e->ev0) (void)hipEventDestroy(e->ev0);
  if (e->ev1) (void)hipEventDestroy(e->ev1);
  e->ev0 = e->ev1 = nullptr;
}

extern "C" kie_status kie_create(const kie_config* cfg, void* workspace_dev, size_t ws_bytes, void* hip_stream,
                                 kie_engine** out) {
  if (!out) return KIE_ERR_ARG;
  *out = nullptr;
  kie_engine* e = new (std::nothrow) kie_engine();
  if (!e) return KIE_ERR_ARG;
  const kie_status st = create_impl(e, cfg, workspace_dev, ws_bytes, hip_stream, true);
  if (st != KIE_OK) {
    release_events(e);
    delete e;
    return st;
  }
  *out = e;
  return KIE_OK;
}

// ---- the static workspace (kie_create_static) -----------------------------
//
// For callers that cannot allocate device memory.  The workspace is this
// file-scope device array: every GPU the library runs on holds its own copy
// (KIE_STATIC_WORKSPACE_BYTES) until the process ends.  In host code the
// array's name is only a host-side handle; its device address on each GPU is
// looked up once per device with hipGetSymbolAddress and kept in
// g_scratch_dev, which is what every launch and copy uses.  The engine handle
// lives in static storage too, one per device.
static __device__ __align__(256) unsigned char scratch[KIE_STATIC_WORKSPACE_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_static_mu;
void* g_scratch_dev[kMaxDevices];  // device address of `scratch` on each GPU (null until looked up)
alignas(kie_engine) unsigned char g_static_store[kMaxDevices][sizeof(kie_engine)];
bool g_static_live[kMaxDevices];
}  // namespace

extern "C" kie_status kie_create_static(const kie_config* cfg, void* hip_stream, kie_engine** out) {
  if (!out) return KIE_ERR_ARG;
  *out = nullptr;
  const kie_status v = kie_config_validate(cfg);
  if (v != KIE_OK) return v;
  const size_t need = make_layout(*cfg).total;
  if (need > (size_t)KIE_STATIC_WORKSPACE_BYTES) {
    if (getenv("KIE_VERBOSE"))
      fprintf(stderr, "kie_create_static: workspace of %zu bytes exceeds the static %zu bytes\n", need,
              (size_t)KIE_STATIC_WORKSPACE_BYTES);
    return KIE_ERR_CAPACITY;
  }
  int dev = 0;
  KIE_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return KIE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_static_mu);
  if (g_static_live[dev]) return KIE_ERR_STATE;  // this GPU's static engine is still in use
  if (!g_scratch_dev[dev]) {  // once per device, with that device current
    void* p = nullptr;
    KIE_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255) != 0) return KIE_ERR_HIP;
    g_scratch_dev[dev] = p;
  }
  kie_engine* e = new (g_static_store[dev]) kie_engine();  // placement: no allocation
  e->is_static = true;
  const kie_status st = create_impl(e, cfg, g_scratch_dev[dev], (size_t)KIE_STATIC_WORKSPACE_BYTES, hip_stream,
                                    false);
  if (st != KIE_OK) {
    e->~kie_engine();
    return st;
  }
  g_static_live[dev] = true;
  *out = e;
  return KIE_OK;
}

extern "C" void kie_destroy(kie_engine* e) {
  if (!e) return;
  release_events(e);
  if (e->is_static) {
    std::lock_guard<std::mutex> lock(g_static_mu);
    const int dev = e->device;
    e->~kie_engine();
    if (dev >= 0 && dev < kMaxDevices) g_static_live[dev] = false;
    return;
  }
  delete e;
}

extern "C" kie_status kie_load_weights(kie_engine* e, const kie_weights* w) {
  if (!e || !w) return KIE_ERR_ARG;
  const int L = e->cfg.n_layers;
  if (!w->tok_emb || !w->final_norm || !w->lm_head || !w->attn_norm || !w->wq || !w->wk || !w->wv || !w->wo ||
      !w->ffn_norm || !w->w_gate || !w->w_up || !w->w_down)
    return KIE_ERR_ARG;
  std::vector<const void*> tab((size_t)L * W_PER_LAYER);
  for (int l = 0; l < L; ++l) {
    const void* p[W_PER_LAYER] = {w->attn_norm[l], w->wq[l], w->wk[l], w->wv[l], w->wo[l],
                                  w->ffn_norm[l], w->w_gate[l], w->w_up[l], w->w_down[l]};
    for (int k = 0; k < W_PER_LAYER; ++k) {
      if (!p[k] || (reinterpret_cast<uintptr_t>(p[k]) & 15) != 0) return KIE_ERR_ARG;
      tab[(size_t)l * W_PER_LAYER + k] = p[k];
    }
  }
  for (const void* p : {w->tok_emb, w->final_norm, w->lm_head})
    if ((reinterpret_cast<uintptr_t>(p) & 15) != 0) return KIE_ERR_ARG;
  KIE_HIP(hipMemcpyAsync(e->ws + e->lay.lw, tab.data(), tab.size() * sizeof(void*), hipMemcpyHostToDevice, e->stream));
  KIE_HIP(hipStreamSynchronize(e->stream));
  e->wtab.assign(tab.size(), nullptr);
  for (size_t i = 0; i < tab.size(); ++i) e->wtab[i] = reinterpret_cast<const uint16_t*>(tab[i]);
  e->tok_emb = reinterpret_cast<const uint16_t*>(w->tok_emb);
  e->final_norm = reinterpret_cast<const uint16_t*>(w->final_norm);
  e->lm_head = reinterpret_cast<const uint16_t*>(w->lm_head);
  e->have_weights = true;
  e->have_seq = false;
  e->pos = 0;
  e->pending = -1;
  return KIE_OK;
}

static Params base_params(const kie_engine* e) {
  const kie_config& c = e->cfg;
  Params P{};
  P.L = c.n_layers; P.d = c.d_model; P.hq = c.n_heads; P.hkv = c.n_kv_heads; P.hd = c.head_dim;
  P.F = c.d_ffn; P.V = c.vocab; P.max_seq = c.max_seq; P.eps = c.rms_eps;
  P.cmax = attn_cmax(c); P.astride = c.head_dim + 4; P.cl_cap = attn_cl_cap(c);
  P.tok_emb = e->tok_emb; P.final_norm = e->final_norm; P.lm_head = e->lm_head;
  P.lw = reinterpret_cast<const uint16_t* const*>(e->ws + e->lay.lw);
  P.kc = reinterpret_cast<uint16_t*>(e->ws + e->lay.kc);
  P.vc = reinterpret_cast<uint16_t*>(e->ws + e->lay.vc);
  P.rope = reinterpret_cast<const float*>(e->ws + e->lay.rope);
  P.xch = reinterpret_cast<uint32_t*>(e->ws + e->lay.xch);
  P.xl = e->lay.xl;
  P.ctl = reinterpret_cast<uint32_t*>(e->ws + e->lay.ctl);
  P.tok_out = reinterpret_cast<int*>(e->ws + e->lay.tok);
  P.abort_after = -1;
  P.withhold_wg = e->withhold_wg;
  P.delay_wg = e->delay_wg;
  P.delay_ticks = e->delay_ticks;
  P.timeout = e->timeout;
  P.trace = e->trace;
  P.trace_step = e->trace_step;
  P.lds_xres = e->lds.xres; P.lds_xn = e->lds.xn; P.lds_scr = e->lds.scr; P.lds_misc = e->lds.misc;
  P.lds_bytes = e->lds.bytes;
  P.grid = e->grid;
  P.samp_k = e->samp_k;
  P.samp_scale = e->samp_scale;
  P.samp_top_p = e->samp_top_p;
  P.samp_key0 = (uint32_t)e->samp_seed;
  P.samp_key1 = (uint32_t)(e->samp_seed >> 32);
  return P;
}

// Reset control words and exchange sets, launch the persistent kernel, wait,
// and read back status / steps done / last token.
// x_last (device fp32, d_model values) or null: the final residual an
// LM-head-only launch starts from, placed in set 0's last-layer xout.
static kie_status run_persistent(kie_engine* e, Params& P, int* done, int* last, const float* x_last = nullptr) {
  KIE_HIP(launch_fill(P.ctl, CTL_WORDS, 0u, e->stream));
  KIE_HIP(launch_fill(P.xch, (uint64_t)kRingSets * P.xl.words, kSent, e->stream));
  if (x_last)
    KIE_HIP(hipMemcpyAsync(P.xch + P.xl.xout + (size_t)(P.L - 1) * P.d, x_last, (size_t)P.d * 4,
                           hipMemcpyDeviceToDevice, e->stream));
  // The kernel reads its parameters from the workspace (scalar loads).
  Params* dev_params = reinterpret_cast<Params*>(e->ws + e->lay.params);
  e->params_host = P;  // stays valid until the copy below has run (the call synchronises)
  KIE_HIP(hipMemcpyAsync(dev_params, &e->params_host, sizeof(Params), hipMemcpyHostToDevice, e->stream));
  void* args[] = {&dev_params};
  if (e->ev0) KIE_HIP(hipEventRecord(e->ev0, e->stream));
  // the arrival-counter instance when chosen (not for an LM-head-only launch:
  // no stage before it arrives at a counter)
  const void* fn = e->handoff == kHandoffCounters && !P.lm_only ? monokernel_counters_fn(e->cfg)
                                                                 : monokernel_fn(e->cfg);
  KIE_HIP(hipLaunchCooperativeKernel(fn, dim3(e->grid), dim3(kThreads), args, (unsigned)P.lds_bytes, e->stream));
  if (e->ev1) KIE_HIP(hipEventRecord(e->ev1, e->stream));
  uint32_t ctl[4] = {0, 0, 0, 0};
  KIE_HIP(hipMemcpyAsync(ctl, P.ctl, sizeof(ctl), hipMemcpyDeviceToHost, e->stream));
  KIE_HIP(hipStreamSynchronize(e->stream));
  float ms = 0.f;
  if (e->ev0 && e->ev1 && hipEventElapsedTime(&ms, e->ev0, e->ev1) == hipSuccess) e->last_ms = ms;
  *done = (int)ctl[CTL_DONE];
  *last = (int)ctl[CTL_LAST];
  e->last_steps = *done;
  const int32_t st = (int32_t)ctl[CTL_STATUS];
  if (st == 0) return KIE_OK;
  if (st == KIE_ERR_ABORTED) return KIE_ERR_ABORTED;
  return KIE_ERR_TIMEOUT;
}

// kie_decode's steps as one launch per stage (stage_kernel): 6 per layer, the
// LM head, and the token.  Plain launches in a host loop, or the same launches
// captured once into a HIP graph and replayed (capture and instantiation happen
// before the timed region).  The events bracket only the launches.
static kie_status run_per_stage(kie_engine* e, Params& P, int* done, int* last) {
  const int L = e->cfg.n_layers;
  KIE_HIP(launch_fill(P.ctl, CTL_WORDS, 0u, e->stream));
  KIE_HIP(launch_fill(P.xch, (uint64_t)kRingSets * P.xl.words, kSent, e->stream));
  Params* dev_params = reinterpret_cast<Params*>(e->ws + e->lay.params);
  e->params_host = P;
  KIE_HIP(hipMemcpyAsync(dev_params, &e->params_host, sizeof(Params), hipMemcpyHostToDevice, e->stream));
  const void* fn = stage_kernel_fn(e->cfg);
  auto launch_all = [&](hipStream_t stream) -> hipError_t {
    for (int s = 0; s < P.n_steps; ++s)
      for (int k = 0; k < L * kStagesPerLayer + 2; ++k) {
        int ss = s, l = k < L * kStagesPerLayer ? k / kStagesPerLayer : 0;
        int st = k < L * kStagesPerLayer ? k % kStagesPerLayer : 6 + (k - L * kStagesPerLayer);
        void* args[] = {&dev_params, &ss, &l, &st};
        const hipError_t he = hipLaunchKernel(fn, dim3(e->grid), dim3(kThreads), args, (size_t)e->lds.bytes,
                                              stream);
        if (he != hipSuccess) return he;
      }
    return hipSuccess;
  };
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  hipError_t he = hipSuccess;
  if (e->launch_mode == KIE_LAUNCH_PER_STAGE_GRAPH) {
    // captured on a stream of its own (the engine's may be the null stream,
    // which cannot be captured), replayed on the engine's
    hipStream_t cs = nullptr;
    he = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
    if (he == hipSuccess) he = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
    if (he == hipSuccess) {
      const hipError_t hl = launch_all(cs);
      he = hipStreamEndCapture(cs, &graph);
      if (he == hipSuccess) he = hl;
    }
    if (cs) (void)hipStreamDestroy(cs);
    if (he == hipSuccess) he = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  }
  if (he == hipSuccess && e->ev0) he = hipEventRecord(e->ev0, e->stream);
  if (he == hipSuccess) he = exec ? hipGraphLaunch(exec, e->stream) : launch_all(e->stream);
  if (he == hipSuccess && e->ev1) he = hipEventRecord(e->ev1, e->stream);
  uint32_t ctl[4] = {0, 0, 0, 0};
  if (he == hipSuccess) he = hipMemcpyAsync(ctl, P.ctl, sizeof(ctl), hipMemcpyDeviceToHost, e->stream);
  if (he == hipSuccess) he = hipStreamSynchronize(e->stream);
  if (exec) (void)hipGraphExecDestroy(exec);
  if (graph) (void)hipGraphDestroy(graph);
  KIE_HIP(he);
  float ms = 0.f;
  if (e->ev0 && e->ev1 && hipEventElapsedTime(&ms, e->ev0, e->ev1) == hipSuccess) e->last_ms = ms;
  *done = (int)ctl[CTL_DONE];
  *last = (int)ctl[CTL_LAST];
  e->last_steps = *done;
  return ctl[CTL_STATUS] == 0 ? KIE_OK : KIE_ERR_TIMEOUT;
}

extern "C" kie_status kie_set_launch_mode(kie_engine* e, int32_t mode) {
  if (!e || (mode != KIE_LAUNCH_PERSISTENT && mode != KIE_LAUNCH_PER_STAGE && mode != KIE_LAUNCH_PER_STAGE_GRAPH))
    return KIE_ERR_ARG;
  e->launch_mode = mode;
  return KIE_OK;
}

extern "C" kie_status kie_prefill(kie_engine* e, const int32_t* prompt_host, int32_t n_prompt,
                                  int32_t* next_token_host, float* logits_dev) {
  if (!e || !prompt_host || !next_token_host) return KIE_ERR_ARG;
  if (!e->have_weights) return KIE_ERR_STATE;
  if (n_prompt < 1) return KIE_ERR_ARG;
  if (n_prompt > e->cfg.max_seq) return KIE_ERR_CAPACITY;
  for (int i = 0; i < n_prompt; ++i)
    if (prompt_host[i] < 0 || prompt_host[i] >= e->cfg.vocab) return KIE_ERR_ARG;
  e->have_seq = false;
  KIE_HIP(hipMemcpyAsync(e->ws + e->lay.forced, prompt_host, (size_t)n_prompt * 4, hipMemcpyHostToDevice, e->stream));
  const int* forced = reinterpret_cast<const int*>(e->ws + e->lay.forced);
  // every position on the matrix cores (when the shape allows), then one
  // persistent launch that runs only the LM head on the last position's
  // residual; else every position as a forced step of the persistent kernel
  int first = 0;
  const float* x_last = nullptr;
  if (e->prefill_mode == KIE_PREFILL_AUTO && e->lay.pf_chunk > 0 && n_prompt >= 2) {
    const kie_config& c = e->cfg;
    PrefillCtx x{};
    x.cfg = c;
    x.stream = e->stream;
    x.tok_emb = e->tok_emb;
    x.wtab = e->wtab.data();
    x.rope = reinterpret_cast<const float*>(e->ws + e->lay.rope);
    x.kc = reinterpret_cast<uint16_t*>(e->ws + e->lay.kc);
    x.vc = reinterpret_cast<uint16_t*>(e->ws + e->lay.vc);
    x.X = reinterpret_cast<float*>(e->ws + e->lay.pf_x);
    x.Xn = e->ws + e->lay.pf_xn;
    x.QKV = reinterpret_cast<float*>(e->ws + e->lay.pf_qkv);
    x.A = e->ws + e->lay.pf_a;
    x.H = e->ws + e->lay.pf_h;
    x.P = reinterpret_cast<float*>(e->ws + e->lay.pf_p);
    const int chunk = e->prefill_chunk > 0 ? e->prefill_chunk : e->lay.pf_chunk;
    int M = 0;
    for (int p0 = 0; p0 < n_prompt; p0 += chunk) {
      M = n_prompt - p0 < chunk ? n_prompt - p0 : chunk;
      KIE_HIP(prefill_chunk(x, forced + p0, p0, M));
    }
    x_last = x.X + (size_t)(M - 1) * c.d_model;  // the last chunk's last row
    first = n_prompt - 1;
  }
  Params P = base_params(e);
  P.pos0 = first;
  P.eos_id = -1;
  P.in_tok = prompt_host[first];
  P.lm_last_only = 1;
  P.logits = logits_dev;
  if (x_last) {  // the LM head alone
    P.lm_only = 1;
    P.n_steps = 1;
  } else {
    P.forced = forced;
    P.n_steps = n_prompt;
  }
  int done = 0, last = 0;
  const kie_status st = run_persistent(e, P, &done, &last, x_last);
  if (st != KIE_OK) return st;
  if (done != P.n_steps) return KIE_ERR_TIMEOUT;
  e->pos = n_prompt;
  e->pending = last;
  e->have_seq = true;
  *next_token_host = last;
  return KIE_OK;
}

extern "C" kie_status kie_set_prefill_mode(kie_engine* e, int32_t mode) {
  if (!e || (mode != KIE_PREFILL_AUTO && mode != KIE_PREFILL_DECODE_LOOP)) return KIE_ERR_ARG;
  e->prefill_mode = mode;
  return KIE_OK;
}

extern "C" kie_status kie_set_grid(kie_engine* e, int32_t grid) {
  if (!e || grid < 0) return KIE_ERR_ARG;
  const int full = e->cu_count < kMaxWG ? e->cu_count : kMaxWG;
  if (grid == 0) grid = full;
  if (grid > full) return KIE_ERR_ARG;
  if (!grid_fits(e->cfg, e->lay, grid) || kie_check_tiling(&e->cfg, grid, 0) != KIE_OK) return KIE_ERR_UNSUPPORTED;
  e->grid = grid;
  return KIE_OK;
}

extern "C" kie_status kie_set_prefill_chunk(kie_engine* e, int32_t positions) {
  if (!e || positions < 0) return KIE_ERR_ARG;
  if (positions > e->lay.pf_chunk) return KIE_ERR_CAPACITY;
  e->prefill_chunk = positions;
  return KIE_OK;
}

extern "C" kie_status kie_set_sampling(kie_engine* e, float temperature, int32_t top_k, float top_p,
                                       uint64_t seed) {
  if (!e || std::isnan(temperature)) return KIE_ERR_ARG;
  if (temperature <= 0.f) {
    e->samp_k = 0;
    return KIE_OK;
  }
  if (top_k < 1 || top_k > kCand || top_k > e->cfg.vocab || !(top_p > 0.f && top_p <= 1.f) ||
      !std::isfinite(1.0f / temperature))
    return KIE_ERR_ARG;
  e->samp_k = top_k;
  e->samp_scale = 1.4426950408889634f / temperature;
  e->samp_top_p = top_p;
  e->samp_seed = seed;
  return KIE_OK;
}

extern "C" kie_status kie_decode(kie_engine* e, int32_t n_steps, int32_t eos_id, int32_t* tokens_host,
                                 int32_t* n_generated, float* logits_dev) {
  if (!e || !n_generated || (n_steps > 0 && !tokens_host) || n_steps < 0) return KIE_ERR_ARG;
  if (eos_id >= e->cfg.vocab) return KIE_ERR_ARG;
  if (!e->have_weights || !e->have_seq) return KIE_ERR_STATE;
  if ((long long)e->pos + n_steps > e->cfg.max_seq) return KIE_ERR_CAPACITY;
  const int abort_after = e->abort_after;
  e->abort_after = -1;
  if (n_steps == 0 || abort_after == 0) {  // nothing to run; the sequence is unchanged
    *n_generated = 0;
    return n_steps > 0 ? KIE_ERR_ABORTED : KIE_OK;
  }
  Params P = base_params(e);
  P.pos0 = e->pos;
  P.n_steps = n_steps;
  P.eos_id = eos_id < 0 ? -1 : eos_id;
  P.in_tok = e->pending;
  P.lm_last_only = 0;
  P.logits = logits_dev;
  P.abort_after = abort_after;
  int done = 0, last = 0;
  const bool per_stage = e->launch_mode != KIE_LAUNCH_PERSISTENT;
  if (per_stage) {
    // greedy, fixed step count, default hand-offs, no timeline
    if (e->samp_k > 0 || P.eos_id >= 0 || abort_after >= 0 || e->withhold_wg >= 0) return KIE_ERR_UNSUPPORTED;
    P.trace = nullptr;
    P.delay_wg = -1;
  }
  const kie_status st = per_stage ? run_per_stage(e, P, &done, &last) : run_persistent(e, P, &done, &last);
  if (st == KIE_ERR_HIP) return st;
  if (done > 0) {
    KIE_HIP(hipMemcpy(tokens_host, P.tok_out, (size_t)done * 4, hipMemcpyDeviceToHost));
  }
  *n_generated = done;
  if (st == KIE_OK || st == KIE_ERR_ABORTED) {
    e->pos += done;
    if (done > 0) e->pending = last;
  } else {
    e->have_seq = false;  // a poll expired mid-step: the cache row of that step may be partial
  }
  return st;
}

extern "C" kie_status kie_import_kv(kie_engine* e, const void* k_dev, const void* v_dev, int32_t n_pos,
                                    int32_t pending_token) {
  if (!e) return KIE_ERR_ARG;
  if (!e->have_weights) return KIE_ERR_STATE;
  if (n_pos < 0 || pending_token < 0 || pending_token >= e->cfg.vocab) return KIE_ERR_ARG;
  if (n_pos >= e->cfg.max_seq) return KIE_ERR_CAPACITY;
  if (n_pos > 0 && (!k_dev || !v_dev)) return KIE_ERR_ARG;
  const kie_config& c = e->cfg;
  uint16_t* kc = reinterpret_cast<uint16_t*>(e->ws + e->lay.kc);
  uint16_t* vc = reinterpret_cast<uint16_t*>(e->ws + e->lay.vc);
  if (n_pos > 0) {
    const size_t row = (size_t)n_pos * c.head_dim * 2, pitch = (size_t)c.max_seq * c.head_dim * 2;
    const size_t planes = (size_t)c.n_layers * c.n_kv_heads;
    KIE_HIP(hipMemcpy2DAsync(kc, pitch, k_dev, row, row, planes, hipMemcpyDeviceToDevice, e->stream));
    KIE_HIP(hipMemcpy2DAsync(vc, pitch, v_dev, row, row, planes, hipMemcpyDeviceToDevice, e->stream));
  }
  KIE_HIP(hipStreamSynchronize(e->stream));
  e->pos = n_pos;
  e->pending = pending_token;
  e->have_seq = true;
  return KIE_OK;
}

extern "C" kie_status kie_export_kv(kie_engine* e, void* k_dev, void* v_dev, int32_t* n_pos_io,
                                    int32_t* pending_token) {
  if (!e || !n_pos_io || !pending_token) return KIE_ERR_ARG;
  if (!e->have_seq) return KIE_ERR_STATE;
  if (*n_pos_io < e->pos) return KIE_ERR_CAPACITY;
  if (e->pos > 0 && (!k_dev || !v_dev)) return KIE_ERR_ARG;
  const kie_config& c = e->cfg;
  if (e->pos > 0) {
    const size_t row = (size_t)e->pos * c.head_dim * 2, pitch = (size_t)c.max_seq * c.head_dim * 2;
    const size_t planes = (size_t)c.n_layers * c.n_kv_heads;
    KIE_HIP(hipMemcpy2DAsync(k_dev, row, e->ws + e->lay.kc, pitch, row, planes, hipMemcpyDeviceToDevice, e->stream));
    KIE_HIP(hipMemcpy2DAsync(v_dev, row, e->ws + e->lay.vc, pitch, row, planes, hipMemcpyDeviceToDevice, e->stream));
    KIE_HIP(hipStreamSynchronize(e->stream));
  }
  *n_pos_io = e->pos;
  *pending_token = e->pending;
  return KIE_OK;
}

extern "C" kie_status kie_get_info(const kie_engine* e, kie_info* out) {
  if (!e || !out) return KIE_ERR_ARG;
  out->grid = e->grid;
  out->block = kThreads;
  out->lds_bytes = e->lds.bytes;
  out->cu_count = e->cu_count;
  out->attn_max_chunks = attn_cmax(e->cfg);
  out->pos = e->pos;
  out->last_kernel_ms = e->last_ms;
  out->last_steps = e->last_steps;
  return KIE_OK;
}

extern "C" kie_status kie_set_poll_timeout(kie_engine* e, uint64_t ticks) {
  if (!e) return KIE_ERR_ARG;
  e->timeout = ticks ? ticks : kDefaultTimeout;
  return KIE_OK;
}

extern "C" kie_status kie_set_abort_after(kie_engine* e, int32_t abort_after_steps) {
  if (!e || abort_after_steps < -1) return KIE_ERR_ARG;
  e->abort_after = abort_after_steps;
  return KIE_OK;
}

extern "C" kie_status kie_set_withhold(kie_engine* e, int32_t wg) {
  if (!e || wg < -1) return KIE_ERR_ARG;
  e->withhold_wg = wg;
  return KIE_OK;
}

extern "C" kie_status kie_set_handoff(kie_engine* e, int32_t mode) {
  if (!e || (mode != KIE_HANDOFF_NAN_POLL && mode != KIE_HANDOFF_COUNTERS)) return KIE_ERR_ARG;
  if (mode == KIE_HANDOFF_COUNTERS && !monokernel_counters_fn(e->cfg)) return KIE_ERR_UNSUPPORTED;
  e->handoff = mode == KIE_HANDOFF_COUNTERS ? kHandoffCounters : kHandoffNan;
  return KIE_OK;
}

extern "C" kie_status kie_set_delay(kie_engine* e, int32_t wg, uint64_t ticks) {
  if (!e || wg < -1) return KIE_ERR_ARG;
  if (ticks > 100000000ull) return KIE_ERR_ARG;  // at most 1 s per publication
  e->delay_wg = wg;
  e->delay_ticks = ticks;
  return KIE_OK;
}

// After a launch of S >= 2 completed steps, the exchange sets of steps S-2
// and S-3 (set indices (S-2) % 3 and S % 3) must hold the NaN pattern in every
// word: the first was recycled during step S-1, the second during step S-2
// (or never used).  Counts the words that do not.
extern "C" kie_status kie_check_idle_sets(const kie_engine* e, uint64_t* dirty_words) {
  if (!e || !dirty_words) return KIE_ERR_ARG;
  const int S = e->last_steps;
  if (S < 2) return KIE_ERR_STATE;
  const size_t words = e->lay.xl.words;
  std::vector<uint32_t> host(words);
  uint64_t dirty = 0;
  for (int set : {(S - 2) % kRingSets, S % kRingSets}) {
    const char* src = e->ws + e->lay.xch + (size_t)set * words * 4;
    KIE_HIP(hipMemcpyAsync(host.data(), src, words * 4, hipMemcpyDeviceToHost, e->stream));
    KIE_HIP(hipStreamSynchronize(e->stream));
    for (uint32_t w : host) dirty += w != kSent;
  }
  *dirty_words = dirty;
  return KIE_OK;
}

extern "C" kie_status kie_gemv_probe(const void* W_dev, int32_t rows, int32_t cols, int32_t n_copies,
                                     const void* x_dev, float* y_dev, int32_t n_vec, int32_t dtype,
                                     int32_t input_first, void* hip_stream, float* kernel_ms) {
  if (!W_dev || !x_dev || !y_dev || rows < 1 || n_copies < 1 || n_vec < 0) return KIE_ERR_ARG;
  if (input_first != 0 && input_first != 1) return KIE_ERR_ARG;
  if (dtype != KIE_F16 && dtype != KIE_BF16) return KIE_ERR_ARG;
  if (!k_ok(cols)) return KIE_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(W_dev) & 15) || (reinterpret_cast<uintptr_t>(x_dev) & 15)) return KIE_ERR_ARG;
  if (n_vec == 0) {
    if (kernel_ms) *kernel_ms = 0.f;
    return KIE_OK;
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
  int dev = 0;
  KIE_HIP(hipGetDevice(&dev));
  hipDeviceProp_t prop;
  KIE_HIP(hipGetDeviceProperties(&prop, dev));
  int grid = prop.multiProcessorCount;
  if (grid > rows) grid = rows;
  const size_t lds = (size_t)cols * 2 * (dtype == KIE_BF16 ? 3 : 1) + (size_t)(kRedCap + kYCap) * 4;
  const int max_rows = (rows + grid - 1) / grid;
  const int vpr = cols / 8, lpr = vpr < kThreads ? vpr : kThreads, nwr = lpr >= 64 ? lpr / 64 : 1;
  if ((long long)max_rows * nwr > kRedCap || max_rows > kYCap) return KIE_ERR_UNSUPPORTED;
  const void* fn = gemv_probe_fn(dtype, input_first != 0);
  KIE_HIP(hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
  hipEvent_t a, b;
  KIE_HIP(hipEventCreate(&a));
  KIE_HIP(hipEventCreate(&b));
  const uint16_t* W = reinterpret_cast<const uint16_t*>(W_dev);
  const uint16_t* x = reinterpret_cast<const uint16_t*>(x_dev);
  int r = rows, c = cols, nc = n_copies, nv = n_vec;
  void* args[] = {&W, &r, &c, &nc, &x, &y_dev, &nv};
  hipError_t he = hipEventRecord(a, st);
  if (he == hipSuccess) he = hipLaunchKernel(fn, dim3(grid), dim3(kThreads), args, lds, st);
  if (he == hipSuccess) he = hipEventRecord(b, st);
  if (he == hipSuccess) he = hipStreamSynchronize(st);
  float ms = 0.f;
  if (he == hipSuccess) he = hipEventElapsedTime(&ms, a, b);
  (void)hipEventDestroy(a);
  (void)hipEventDestroy(b);
  if (he != hipSuccess) return hip_fail(he, "gemv probe");
  if (kernel_ms) *kernel_ms = ms;
  return KIE_OK;
}

extern "C" kie_status kie_stream_probe(const void* buf_dev, size_t bytes, int32_t depth, int32_t reps,
                                       uint32_t* sink_dev, void* hip_stream, float* kernel_ms) {
  if (!buf_dev || !sink_dev || reps < 1 || (reinterpret_cast<uintptr_t>(buf_dev) & 15)) return KIE_ERR_ARG;
  const void* fn = stream_probe_fn(depth);
  if (!fn) return KIE_ERR_ARG;
  hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
  int dev = 0;
  KIE_HIP(hipGetDevice(&dev));
  hipDeviceProp_t prop;
  KIE_HIP(hipGetDeviceProperties(&prop, dev));
  const int grid = prop.multiProcessorCount < kMaxWG ? prop.multiProcessorCount : kMaxWG;
  // every work-group reads whole passes of 512 vectors, at least `depth` of them
  if (bytes / 16 < (uint64_t)grid * kThreads * (uint64_t)depth) return KIE_ERR_CAPACITY;
  const uint4* buf = reinterpret_cast<const uint4*>(buf_dev);
  uint64_t nvec = bytes / 16;
  int rp = reps;
  void* args[] = {&buf, &nvec, &rp, &sink_dev};
  hipEvent_t a, b;
  KIE_HIP(hipEventCreate(&a));
  KIE_HIP(hipEventCreate(&b));
  hipError_t he = hipEventRecord(a, st);
  if (he == hipSuccess) he = hipLaunchCooperativeKernel(fn, dim3(grid), dim3(kThreads), args, 0, st);
  if (he == hipSuccess) he = hipEventRecord(b, st);
  if (he == hipSuccess) he = hipStreamSynchronize(st);
  float ms = 0.f;
  if (he == hipSuccess) he = hipEventElapsedTime(&ms, a, b);
  (void)hipEventDestroy(a);
  (void)hipEventDestroy(b);
  if (he != hipSuccess) return hip_fail(he, "stream probe");
  if (kernel_ms) *kernel_ms = ms;
  return KIE_OK;
}

extern "C" size_t kie_trace_words(const kie_engine* e) {
  if (!e) return 0;
  return (size_t)(e->cfg.n_layers * kStagesPerLayer + 3) * e->grid * kTraceStamps;
}

extern "C" kie_status kie_set_trace(kie_engine* e, uint64_t* trace_dev, int32_t step) {
  if (!e || step < 0) return KIE_ERR_ARG;
  if (trace_dev && (reinterpret_cast<uintptr_t>(trace_dev) & 7)) return KIE_ERR_ARG;
  e->trace = trace_dev;
  e->trace_step = step;
  return KIE_OK;
}

// Host check of the GEMV tiling (kie_tiling.hpp) for cfg on `grid`
// work-groups: every vector a thread loads lies inside its weight matrix and
// on a row boundary grid; every in-range vector is the (row, column) the stage
// definition assigns to it; with `full`, every vector of every matrix is
// loaded exactly once by the grid (sampled work-groups otherwise).
extern "C" kie_status kie_check_tiling(const kie_config* cfg, int32_t grid, int32_t full) {
  const kie_status v = kie_config_validate(cfg);
  if (v != KIE_OK) return v;
  if (grid < 1 || grid > kMaxWG) return KIE_ERR_ARG;
  const kie_config& c = *cfg;
  const TileDims D{c.d_model, c.n_heads, c.n_kv_heads, c.head_dim, c.d_ffn, c.vocab};
  const uintptr_t kSpan = (uintptr_t)1 << 40;  // fake, disjoint matrix bases
  const uint16_t* mats[M_COUNT];
  for (int m = 0; m < M_COUNT; ++m) mats[m] = reinterpret_cast<const uint16_t*>((uintptr_t)(m + 1) * kSpan);
  const bool verbose = getenv("KIE_VERBOSE") != nullptr;
  auto fail = [&](const char* what, int st, int wg, int t, int j) {
    if (verbose) fprintf(stderr, "kie_check_tiling: %s (stage %d wg %d thread %d vector %d)\n", what, st, wg, t, j);
    return KIE_ERR_UNSUPPORTED;
  };
  std::vector<std::vector<uint8_t>> seen;
  if (full) {
    seen.resize(M_COUNT);
    for (int m = 0; m < M_COUNT; ++m) {
      int N, K;
      stage_dims(D, m == M_Q || m == M_K || m == M_V ? GS_QKV : m == M_O ? GS_WO
                      : m == M_GATE || m == M_UP ? GS_GATEUP : m == M_DOWN ? GS_DOWN : GS_LM, N, K);
      seen[m].assign((size_t)matrix_rows(D, m) * (K / 8), 0);
    }
  }
  std::vector<int> wgs;
  if (full) {
    for (int w = 0; w < grid; ++w) wgs.push_back(w);
  } else {
    for (int w : {0, 1, grid / 2, grid - 2, grid - 1})
      if (w >= 0 && w < grid && (wgs.empty() || wgs.back() != w)) wgs.push_back(w);
  }
  for (int st = 0; st < GS_COUNT; ++st) {
    int N, K;
    stage_dims(D, st, N, K);
    for (int wg : wgs) {
      const int r0 = split_lo(N, grid, wg), r1 = split_lo(N, grid, wg + 1), n = r1 - r0;
      for (int t = 0; t < kThreads; ++t) {
        const StagePlan g = make_stage_plan(D, st, wg, grid, t, mats);
        if (g.nrows > kYCap || (long long)g.nrows * g.nwr > kRedCap) return fail("rows exceed LDS", st, wg, t, -1);
        if (g.nrows == 0) continue;
        const int J = g.passes() * g.vpt, Jp = (J + kDepth - 1) / kDepth * kDepth;
        for (int j = 0; j < Jp + kDepth; ++j) {  // + the prefetch reach of the previous stage
          const uintptr_t a = reinterpret_cast<uintptr_t>(g.addr(j));
          const int m = (int)(a / kSpan) - 1;
          if (m < 0 || m >= M_COUNT) return fail("address outside every matrix", st, wg, t, j);
          const uint64_t e = (a - (uintptr_t)(m + 1) * kSpan) / 2;
          if ((a & 15) != 0 || e % 8 != 0) return fail("misaligned vector", st, wg, t, j);
          if (e + 8 > (uint64_t)matrix_rows(D, m) * K) return fail("vector beyond its matrix", st, wg, t, j);
          const int p = j / g.vpt, i = j % g.vpt;
          const int row = p * g.rp + g.sub, kv = g.kl + i * g.lpr;
          if (row >= g.nrows || kv >= g.vpr || j >= J) continue;  // padding: any in-bounds vector
          int em, erow;
          switch (st) {
            case GS_QKV: {
              const int gr = r0 + row, nq = D.hq * D.hd, nk = D.hkv * D.hd;
              em = gr < nq ? M_Q : gr < nq + nk ? M_K : M_V;
              erow = gr < nq ? gr : gr < nq + nk ? gr - nq : gr - nq - nk;
              break;
            }
            case GS_WO: em = M_O; erow = r0 + row; break;
            case GS_GATEUP: em = row < n ? M_GATE : M_UP; erow = r0 + (row < n ? row : row - n); break;
            case GS_DOWN: em = M_DOWN; erow = r0 + row; break;
            default: em = M_LM; erow = r0 + row; break;
          }
          if (m != em || e != (uint64_t)erow * K + (uint64_t)kv * 8) return fail("wrong vector", st, wg, t, j);
          if (full) {
            uint8_t& s = seen[m][(size_t)erow * (K / 8) + kv];
            if (s) return fail("vector loaded twice", st, wg, t, j);
            s = 1;
          }
        }
      }
    }
  }
  if (full)
    for (int m = 0; m < M_COUNT; ++m)
      for (uint8_t s : seen[m])
        if (!s) return fail("vector never loaded", -1, -1, -1, m);
  return KIE_OK;
}
