// Parameters and layout shared by the host runtime and the device kernels.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace kie {

constexpr int kThreads = 512;            // threads per work-group (8 wave64)
constexpr int kWaves = kThreads / 64;
constexpr int kMaxWG = 1024;             // upper bound on the persistent grid
constexpr int kRingSets = 3;             // exchange sets rotating over decode steps
constexpr int kClMin = 16;               // shortest split-KV chunk (positions)
constexpr int kAttnUnits = 256;          // target (KV head, chunk) units per layer
constexpr int kRedCap = 8192;            // LDS floats for per-wave GEMV partial sums
constexpr int kYCap = 1024;              // LDS floats for finished GEMV rows
#ifndef KIE_DEPTH
#define KIE_DEPTH 8
#endif
constexpr int kDepth = KIE_DEPTH;       // weight vectors in flight per thread (a multiple of 4)
constexpr uint32_t kSent = 0xFFFFFFFFu;  // NaN pattern that marks "not written yet"
constexpr int kCand = 64;                // sampling: candidates per work-group list and in the global list
constexpr int kPadIdx = 0x40000000;      // sampling: indices of padding candidates (logit -inf) start here
constexpr int kStagesPerLayer = 6;       // qkv, attn, merge, wo, gate/up, down
constexpr int kTraceStamps = 4;          // per (slot, work-group): entry, input, compute done, exit
constexpr int kHandoffNan = 0, kHandoffCounters = 1;

// per-layer weight slots in the device pointer table
enum : int {
  W_ATTN_NORM = 0, W_Q, W_K, W_V, W_O, W_FFN_NORM, W_GATE, W_UP, W_DOWN, W_PER_LAYER
};

// control words
enum : int { CTL_STATUS = 0, CTL_DONE = 1, CTL_LAST = 2, CTL_WORDS = 64 };

// Word offsets of the sub-buffers of one exchange set (fp32 words).
struct XchLayout {
  uint64_t xmid;   // [L][d]        residual after attention
  uint64_t xout;   // [L][d]        residual after the feed-forward block
  uint64_t qkv;    // [L][(Hq+2Hkv)*hd] q, k, v before the rotary embedding
  uint64_t a;      // [L][Hq*hd]    merged attention output
  uint64_t h;      // [L][F]        silu(gate) * up
  uint64_t arg;    // [kMaxWG][2]   per-work-group (max logit, index)
  uint64_t cand;   // [kMaxWG][kCand][2] per-work-group sampling candidates (logit, index), sorted
  uint64_t cand2;  // [kMaxWG / 8][kCand][2] the same, merged over groups of 8 work-groups
  uint64_t stok;   // [2]           sampled token (work-group 0 draws it)
  uint64_t cnt;    // [L * kStagesPerLayer + 1] arrival counters (counter hand-off mode)
  uint64_t att;    // [L][Hq][cmax][astride]  split-KV partials (m, l, pad, pad, o[hd])
  uint64_t dense;  // words before att (reset wholesale)
  uint64_t words;  // total words of one set
};

struct Params {
  // model
  int L, d, hq, hkv, hd, F, V, max_seq;
  float eps;
  int cmax, astride, cl_cap;
  // weights (16-bit words of the engine dtype)
  const uint16_t* tok_emb;
  const uint16_t* final_norm;
  const uint16_t* lm_head;
  const uint16_t* const* lw;  // device table [L][W_PER_LAYER]
  // workspace
  uint16_t* kc;               // [L][Hkv][max_seq][hd]
  uint16_t* vc;
  const float* rope;          // [max_seq][hd/2][2] = (cos, sin)
  uint32_t* xch;              // kRingSets exchange sets
  XchLayout xl;
  uint32_t* ctl;              // control words
  int* tok_out;               // [n_steps] emitted tokens
  float* logits;              // [n_steps][V] or [1][V] (prefill) or null
  const int* forced;          // prompt tokens (prefill) or null
  // launch
  int pos0, n_steps, eos_id, in_tok, abort_after, lm_last_only, withhold_wg;
  // 1: one step that runs only the LM head and the token choice, on a final
  // residual the host placed in exchange set 0's last-layer xout (the prompt
  // path's last position); no layers, no embedding
  int lm_only;
  // race test: work-group delay_wg waits delay_ticks (100 MHz) before it
  // publishes any hand-off output (-1: off)
  int delay_wg;
  uint64_t delay_ticks;
  // sampling: samp_k = 0 greedy; else top-k (<= kCand), log2(e) / temperature,
  // nucleus mass, Philox4x32-10 key
  int samp_k;
  float samp_scale, samp_top_p;
  uint32_t samp_key0, samp_key1;
  // per-token timeline: step `trace_step` of the launch is stamped into
  // trace[((slot) * grid + wg) * kTraceStamps + k], slot = layer *
  // kStagesPerLayer + stage (then kStagesPerLayer*L + {0: LM head, 1: step
  // tail}); k = 0 entry, 1 input arrived, 2 compute done, 3 exit; ticks of the
  // 100 MHz real-time counter.
  uint64_t* trace;
  int trace_step;
  uint64_t timeout;           // poll deadline, ticks of the 100 MHz counter
  // dynamic LDS layout (bytes)
  int lds_xres, lds_xn, lds_scr, lds_misc, lds_bytes;
  int grid;                   // work-groups of the launch (gridDim.x, read as a kernel parameter)
};

}  // namespace kie
