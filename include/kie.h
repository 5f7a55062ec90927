/*
 * kie.h -- C ABI of the persistent batch-1 decode monokernel for one AMD
 * MI355X (gfx950).
 *
 * What the library computes.  Greedy autoregressive decoding of one request
 * (batch 1) through a dense, pre-norm, decoder-only transformer (RMSNorm,
 * rotary position embedding, grouped-query attention, SwiGLU feed-forward,
 * untied LM head).  Every decode step of a kie_decode() call -- embedding,
 * all layers, LM head, greedy argmax and the EOS test -- runs inside ONE
 * grid-resident persistent kernel, which loops over tokens without returning
 * to the host and without a kernel launch per token or per layer.  This is the
 * "monokernel" of the Kog Inference Engine pages: revietech.ru, "Kog
 * vyzhimayet maksimum iz GPU: 3000 tokenov/s", section "Chto takoye
 * monokernel" (one resident program covering prefill, decode, LM-head
 * sampling and the EOS check, no CPU return, no per-token launch); remio.ai,
 * "Kog stawia na glebsza optymalizacje GPU...", section "Dlaczego Kog idzie
 * glebiej" (the decode sequence lives in one persistent kernel); lehuy.net,
 * "Kog dat toc do suy luan 3.000 token/giay...", section "Giai phap
 * Monokernel" (launch cost removed, CPU-GPU synchronisation minimised).
 *
 * Work-groups hand data to each other through device buffers that are
 * pre-filled with a NaN bit pattern; consumers poll the data words themselves
 * until they stop being NaN, instead of counting arrivals with atomics
 * (revietech.ru page, section "Chto takoye monokernel", the paragraph on
 * synchronisation).  Projections at batch 1 are matrix-vector products run on
 * the packed dot2 vector ALU instructions, not on matrix cores (revietech.ru
 * page, section "Arkhitektura i osobennosti", first bullet, and its FAQ).
 *
 * Conventions shared by every entry point
 *  - Memory.  The caller owns every device buffer: weights and the workspace.
 *    The library never allocates or frees device memory; the opaque engine
 *    handle (host memory) is the only object it owns.  (kie_create_static
 *    uses a static workspace that is part of the loaded library instead.)
 *  - Pointers marked _dev are device pointers, _host are host pointers.
 *  - Matrices are row-major [out][in] (PyTorch nn.Linear layout), elements of
 *    the engine dtype (IEEE fp16 or bf16 as raw 16-bit words).
 *  - Calls are synchronous on the stream given to kie_create(): they return
 *    after the GPU work finished, so their status covers failures found by the
 *    kernel itself (a poll that timed out).
 *  - Threads.  An engine must be used by one host thread at a time.  Two
 *    engines on one GPU must not run kie_prefill/kie_decode concurrently: the
 *    persistent kernel occupies every compute unit.
 *  - Errors.  Every call returns a kie_status; on any error no output argument
 *    is written unless stated otherwise.
 */
#ifndef KIE_H
#define KIE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  kie_status_string() gives a short English text. */
typedef enum {
  KIE_OK = 0,
  KIE_ERR_ARG = -1,         /* null pointer, size or range error in arguments */
  KIE_ERR_STATE = -2,       /* call out of order (decode before prefill ...) */
  KIE_ERR_CAPACITY = -3,    /* position would exceed max_seq, workspace too small */
  KIE_ERR_UNSUPPORTED = -4, /* shape the kernels do not implement */
  KIE_ERR_HIP = -5,         /* a HIP runtime call failed (no device, launch error) */
  KIE_ERR_TIMEOUT = -6,     /* a device-side poll exceeded its deadline */
  KIE_ERR_ABORTED = -7      /* the kernel stopped on the engine's abort request */
} kie_status;

typedef enum { KIE_F16 = 1, KIE_BF16 = 2 } kie_dtype;

/* Model shape.  Supported (kie_config_validate() reports anything else as
 * KIE_ERR_UNSUPPORTED):
 *   head_dim in {64, 128}; n_heads / n_kv_heads in {1, 2, 4, 8}; n_kv_heads <= 256;
 *   d_model and n_heads*head_dim powers of two in [256, 4096], both below 512
 *   or both at least 512;
 *   d_ffn a power of two in [512, 4096] or a multiple of 256 in (4096, 16384],
 *   and at most 4096 when d_model is 256;
 *   vocab * d_model < 2^40; the kernel's LDS plan within 160 KiB;
 *   vocab >= 1; max_seq >= 1. */
typedef struct {
  int32_t n_layers;
  int32_t d_model;
  int32_t n_heads;     /* query heads Hq */
  int32_t n_kv_heads;  /* key/value heads Hkv */
  int32_t head_dim;    /* hd */
  int32_t d_ffn;       /* SwiGLU hidden width F */
  int32_t vocab;       /* V */
  int32_t max_seq;     /* KV-cache capacity in positions */
  float rms_eps;       /* RMSNorm epsilon, e.g. 1e-5 */
  float rope_base;     /* rotary base, e.g. 10000 */
  int32_t dtype;       /* kie_dtype of weights, KV cache and activations fed to dot2 */
} kie_config;

/* Device pointers to the weights, all of engine dtype.  The library borrows
 * them: the caller keeps them alive and unchanged until kie_destroy() or the
 * next kie_load_weights().  Per-layer fields point to host arrays of
 * n_layers device pointers (the arrays are copied during the call).
 *   tok_emb   [vocab][d_model]          lm_head   [vocab][d_model]
 *   final_norm[d_model]
 *   attn_norm [d_model]                 ffn_norm  [d_model]
 *   wq [Hq*hd][d_model]   wk, wv [Hkv*hd][d_model]   wo [d_model][Hq*hd]
 *   w_gate, w_up [d_ffn][d_model]       w_down [d_model][d_ffn]          */
typedef struct {
  const void* tok_emb;
  const void* final_norm;
  const void* lm_head;
  const void* const* attn_norm;
  const void* const* wq;
  const void* const* wk;
  const void* const* wv;
  const void* const* wo;
  const void* const* ffn_norm;
  const void* const* w_gate;
  const void* const* w_up;
  const void* const* w_down;
} kie_weights;

typedef struct kie_engine kie_engine; /* opaque, owned by the library */

/* Short static text for a status code; never NULL. */
const char* kie_status_string(kie_status s);

/* Host-only check of a configuration: KIE_OK, KIE_ERR_ARG (null or a value
 * out of range) or KIE_ERR_UNSUPPORTED.  Touches no GPU. */
kie_status kie_config_validate(const kie_config* cfg);

/* Bytes of device workspace kie_create() needs for cfg (0 if cfg is invalid).
 * Covers the KV cache [2][n_layers][Hkv][max_seq][hd] of engine dtype, the
 * rotary table, the NaN-initialised exchange buffers and control words.
 * Touches no GPU. */
size_t kie_workspace_bytes(const kie_config* cfg);

/* Create an engine on the current HIP device.  workspace_dev: device buffer of
 * ws_bytes >= kie_workspace_bytes(cfg), 256-byte aligned, owned by the caller
 * and kept alive until kie_destroy().  hip_stream: a hipStream_t, or NULL for
 * the default stream; every call of this engine runs on it.  Writes the rotary
 * table into the workspace.  On success *out is a new handle.
 * Source: the pages define no API.  They state the problem this call sets up --
 * one request (batch 1) served by one program resident on the GPU
 * (revietech.ru page, section "Chto takoye monokernel") -- and the rest follows
 * the stated target's boundary (create / load weights / prefill / decode /
 * destroy, device memory owned by the caller). */
kie_status kie_create(const kie_config* cfg, void* workspace_dev, size_t ws_bytes,
                      void* hip_stream, kie_engine** out);

/* Bytes of the library's static device workspace (64 MiB) used by
 * kie_create_static(). */
#define KIE_STATIC_WORKSPACE_BYTES (64u << 20)

/* kie_create() for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * engine's workspace is a static device array inside the library instead of a
 * caller buffer, and the handle lives in static storage.  The call allocates
 * nothing (no hipMalloc / hipFree, no host heap) and creates no HIP events
 * (kie_info.last_kernel_ms stays 0 for such an engine).
 *   KIE_ERR_CAPACITY when kie_workspace_bytes(cfg) > KIE_STATIC_WORKSPACE_BYTES.
 *   KIE_ERR_STATE while this GPU's static engine exists (one per GPU: every GPU
 *   the library runs on holds its own static workspace, of that size, until
 *   the process ends).
 * The engine is then used and released (kie_destroy) like any other; the
 * workspace keeps the last engine's contents, and everything a launch needs
 * cleared is cleared by the library before it.  Engines of one GPU share the
 * array: a static engine must not run while another static engine of the same
 * GPU is alive, and calls that overlap on one GPU race. */
kie_status kie_create_static(const kie_config* cfg, void* hip_stream, kie_engine** out);

/* Register the weights (device pointers, see kie_weights).  Resets the
 * sequence: a kie_prefill() or kie_import_kv() must follow before decoding.
 * Errors: KIE_ERR_ARG for a null or misaligned (not 16-byte) pointer.
 * Source: the pages define no API; the weights are streamed from device
 * memory layer by layer on every token (revietech.ru page, section "Tsifry
 * proizvoditelnosti": batch-1 decode is bound by HBM bandwidth), so they stay
 * resident and borrowed, as the stated target's boundary has it. */
kie_status kie_load_weights(kie_engine* e, const kie_weights* w);

/* Run the prompt through the model (see kie_set_prefill_mode for how).  By
 * default, where the shape allows (2 or more positions), every prompt position
 * runs as dense matrix-core products, and one launch of the persistent kernel
 * then runs only the LM head and the token choice on the last position's
 * residual.  Otherwise every position is a step of the persistent decode
 * kernel with the prompt token fed instead of a sampled one.
 * Starts a new sequence: the KV cache is rewritten from position 0.
 *   prompt_host[n_prompt]: token ids in [0, vocab), 1 <= n_prompt <= max_seq.
 *   next_token_host: receives the token after the last prompt position (greedy,
 *   or drawn as kie_set_sampling chose).
 *   logits_dev: NULL, or device float[vocab] receiving the logits of the last
 *   prompt position.
 * After success the engine holds pos = n_prompt and the new token pending. */
kie_status kie_prefill(kie_engine* e, const int32_t* prompt_host, int32_t n_prompt,
                       int32_t* next_token_host, float* logits_dev);

/* How kie_prefill() runs the prompt.  KIE_PREFILL_AUTO (default): every
 * position as dense products on the matrix cores (GEMMs and flash attention;
 * fp16 activations for fp16 models, fp32 activations split into three bf16
 * terms for bf16 models; shapes whose projection widths are multiples of 128
 * and prompts of 2 or more positions -- others fall back to the decode loop),
 * then one launch of the persistent kernel that runs only the LM head and the
 * token choice on the last position, which yields the logits and the first
 * token.  KIE_PREFILL_DECODE_LOOP: every prompt
 * position as a forced step of the persistent decode kernel.  The pages put
 * prompt processing inside the resident program (revietech.ru page, section
 * "Chto takoye monokernel"); both modes leave the same sequence state (up to
 * rounding order). */
typedef enum { KIE_PREFILL_AUTO = 0, KIE_PREFILL_DECODE_LOOP = 1 } kie_prefill_mode;
kie_status kie_set_prefill_mode(kie_engine* e, int32_t mode);

/* Work-groups of the persistent kernel: 0 (default) = one per compute unit;
 * 1 <= grid <= compute units runs on a subset (the pages' kernel deliberately
 * uses 256 of MI300X's 304 CUs: revietech.ru page, section "Arkhitektura i
 * osobennosti").  KIE_ERR_ARG above the compute-unit count,
 * KIE_ERR_UNSUPPORTED when a stage's rows per work-group would not fit LDS.
 * Results do not depend on the grid beyond rounding order.  Takes effect at
 * the next kie_prefill / kie_decode. */
kie_status kie_set_grid(kie_engine* e, int32_t grid);

/* Prompt positions per matrix-core chunk in KIE_PREFILL_AUTO (each chunk runs
 * every layer before the next starts).  The workspace holds the activations of
 * min(max_seq, 8192) positions; 0 (default) uses all of them, a smaller value
 * trades throughput for shorter launch sequences.  KIE_ERR_CAPACITY above the
 * workspace's chunk (0 for shapes without the matrix-core path), KIE_ERR_ARG
 * below 0.  Same results for every chunk size up to rounding order. */
kie_status kie_set_prefill_chunk(kie_engine* e, int32_t positions);

/* How the emitted tokens are chosen from the LM-head logits (by kie_decode
 * and for kie_prefill's next token).  The pages end every token with LM-head
 * sampling and the end-of-sequence check on the device (revietech.ru page,
 * section "Chto takoye monokernel") without naming a rule; this is the rule
 * taken.
 *   temperature <= 0: greedy, the first index of the largest logit (default;
 *   top_k, top_p and seed are then ignored).
 *   temperature > 0: candidates are the top_k largest logits (ties to the
 *   lower index), 1 <= top_k <= min(64, vocab); weights exp((z - zmax) /
 *   temperature); the nucleus is the shortest prefix of the candidates, in
 *   that order, whose weight reaches the fraction top_p (0 < top_p <= 1) of
 *   their total; the token is the first nucleus candidate whose cumulative
 *   weight exceeds u times the nucleus weight.  u = (x >> 8) * 2^-24, x the
 *   first output word of Philox4x32-10 (Salmon et al., SC'11) with counter
 *   (p, 0, 0, 0) and key (seed low 32 bits, seed high 32 bits), p the position
 *   of the token fed to the step: the sequence does not depend on how decoding
 *   is split into calls.  Weights and sums are fp32 on the device.
 * KIE_ERR_ARG for arguments out of range (the previous setting stays). */
kie_status kie_set_sampling(kie_engine* e, float temperature, int32_t top_k, float top_p, uint64_t seed);

/* Decode of up to n_steps tokens (greedy unless kie_set_sampling chose
 * otherwise) in ONE persistent kernel launch.
 * Step i feeds the pending token at position pos+i and emits token i.  If
 * eos_id >= 0 and a step emits eos_id, that token is written and counted and
 * the loop stops.
 *   tokens_host[n_steps]: receives the emitted tokens.
 *   n_generated: receives the number of emitted tokens (<= n_steps).
 *   logits_dev: NULL, or device float[n_steps][vocab] receiving the logits of
 *   every executed step (parity mode; costs extra writes).
 * Requires a prefilled sequence and pos + n_steps <= max_seq (else
 * KIE_ERR_CAPACITY before any launch).  Repeated calls continue the sequence.
 * On KIE_ERR_ABORTED (see kie_set_abort_after) tokens_host and n_generated
 * hold the steps that completed and the sequence stays valid: pos advanced by
 * n_generated and the last emitted token is pending, so decoding can go on.
 * On KIE_ERR_TIMEOUT they hold the completed steps too, but the step that
 * timed out may have left a partial KV-cache row: the sequence must be
 * restarted by kie_prefill() or kie_import_kv() (KIE_ERR_STATE until then).
 * Source: one resident kernel runs every step -- layers, LM-head sampling and
 * the end-of-sequence check -- without returning to the CPU or launching a
 * kernel per token (revietech.ru page, section "Chto takoye monokernel");
 * n_steps and the host arrays are the stated target's boundary. */
kie_status kie_decode(kie_engine* e, int32_t n_steps, int32_t eos_id, int32_t* tokens_host,
                      int32_t* n_generated, float* logits_dev);

/* Release the handle.  NULL-safe.  Frees no caller memory.  The pages define
 * no API; this closes the stated target's create / destroy pair. */
void kie_destroy(kie_engine* e);

/* ---- sequence state: checkpoint / resume -------------------------------- */

/* Replace the sequence state: positions [0, n_pos) of the KV cache are copied
 * from k_dev and v_dev, device arrays [n_layers][Hkv][n_pos][hd] of engine
 * dtype (keys already rotated), pos becomes n_pos and pending_token the token
 * the next decode step feeds.  0 <= n_pos < max_seq. */
kie_status kie_import_kv(kie_engine* e, const void* k_dev, const void* v_dev, int32_t n_pos,
                         int32_t pending_token);

/* Copy the current KV cache rows [0, pos) out to k_dev / v_dev, device arrays
 * [n_layers][Hkv][pos][hd] sized by the caller from *n_pos_io on input (the
 * capacity in positions); on output *n_pos_io = pos and *pending_token = the
 * token the next decode step feeds (-1 if none). */
kie_status kie_export_kv(kie_engine* e, void* k_dev, void* v_dev, int32_t* n_pos_io,
                         int32_t* pending_token);

/* ---- diagnostics ---------------------------------------------------------- */

typedef struct {
  int32_t grid;           /* work-groups of the persistent kernel (one per CU) */
  int32_t block;          /* threads per work-group */
  int32_t lds_bytes;      /* dynamic LDS per work-group */
  int32_t cu_count;       /* compute units reported by the device */
  int32_t attn_max_chunks;/* split-KV chunks per KV head at most */
  int32_t pos;            /* current sequence length */
  float last_kernel_ms;   /* duration of the last persistent launch, HIP events
                             recorded on the engine stream around that launch */
  int32_t last_steps;     /* loop iterations the last launch executed */
} kie_info;

kie_status kie_get_info(const kie_engine* e, kie_info* out);

/* Deadline of every device-side poll, in ticks of the 100 MHz real-time
 * counter (default 2e8 = 2 s).  A poll that exceeds it makes every
 * work-group leave the kernel and the call return KIE_ERR_TIMEOUT.  A tiny
 * value forces that path from the host (failure-handling tests).  0 restores
 * the default. */
kie_status kie_set_poll_timeout(kie_engine* e, uint64_t ticks);

/* Ask the next kie_decode() to stop after abort_after_steps completed steps
 * (-1 = never), returning KIE_ERR_ABORTED with the partial tokens.  The
 * request is consumed by that call. */
kie_status kie_set_abort_after(kie_engine* e, int32_t abort_after_steps);

/* Fault injection for failure-handling tests: work-group `wg` of the next
 * persistent launches never publishes its end-of-step partial, so every other
 * work-group's poll for it must expire and the call must return
 * KIE_ERR_TIMEOUT (after the poll deadline) with every work-group having left
 * the kernel.  -1 (default) disables it. */
kie_status kie_set_withhold(kie_engine* e, int32_t wg);

/* Race test: the next persistent launches make work-group `wg` wait `ticks`
 * of the 100 MHz counter (at most 1e8) before each of its hand-off
 * publications (QKV, attention partials, merge, Wo, gate/up, down, the LM
 * head's argmax partial and sampling lists, the sampled token), so every
 * consumer of its words sees them arrive late.  The results must not change
 * (tests compare tokens and logits bit for bit).  wg = -1 turns it off. */
kie_status kie_set_delay(kie_engine* e, int32_t wg, uint64_t ticks);

/* Hand-off protocol of the next persistent launches (a measurement switch).
 * Source: revietech.ru, "Kog vyzhimayet maksimum iz GPU: 3000 tokenov/s",
 * section "Chto takoye monokernel", the synchronisation paragraph: work-groups
 * poll buffers pre-filled with NaN instead of counting arrivals with atomics.
 *   KIE_HANDOFF_NAN_POLL (default): the data is its own flag; a consumer polls
 *     exactly the words it needs.
 *   KIE_HANDOFF_COUNTERS: the alternative that passage sets aside, for
 *     comparison.  After each stage every work-group waits until its own
 *     stores are performed and adds one to the stage's counter (an agent-scope
 *     atomic); consumers wait until all work-groups have arrived, then read.
 * The counter protocol is a separate kernel instance, built for the shapes it
 * is measured on (4 query heads per KV head, model width and d_ffn both in
 * the four-vectors-per-lane GEMV class: the ~2B and ~8B shapes among them);
 * KIE_ERR_UNSUPPORTED for other shapes.  An
 * LM-head-only launch of kie_prefill always uses the default protocol.
 * Results are bit-identical in both modes.  KIE_ERR_ARG for another mode. */
#define KIE_HANDOFF_NAN_POLL 0
#define KIE_HANDOFF_COUNTERS 1
kie_status kie_set_handoff(kie_engine* e, int32_t mode);

/* How kie_decode runs its steps (a measurement switch).
 * Source: revietech.ru, "Kog vyzhimayet maksimum iz GPU: 3000 tokenov/s",
 * section "Chto takoye monokernel": every separate kernel launch costs a fixed
 * setup time, which the single resident kernel removes.
 *   KIE_LAUNCH_PERSISTENT (default): one persistent launch for all steps.
 *   KIE_LAUNCH_PER_STAGE: the same stage code as one launch per stage per
 *     token (6 per layer, the LM head, the token), queued from a host loop.
 *   KIE_LAUNCH_PER_STAGE_GRAPH: the same launches captured once into a HIP
 *     graph and replayed as one graph launch (capture before the timing).
 *     Each call creates a capture stream and a graph of 6 x n_layers + 2
 *     nodes per step (host-side HIP objects, released before it returns): a
 *     measurement mode, not for callers that cannot allocate.
 * The per-stage modes take greedy decode with eos_id < 0 and no fault
 * injection (else KIE_ERR_UNSUPPORTED); tokens and logits equal the
 * persistent kernel's bit for bit.  KIE_ERR_ARG for another mode. */
#define KIE_LAUNCH_PERSISTENT 0
#define KIE_LAUNCH_PER_STAGE 1
#define KIE_LAUNCH_PER_STAGE_GRAPH 2
kie_status kie_set_launch_mode(kie_engine* e, int32_t mode);

/* Race test of the exchange-set recycling: after a launch that completed S >= 2
 * steps, the two exchange sets not used by its last step must hold the NaN
 * pattern in every word (one was recycled during the last step, the other
 * during the step before it, or never used).  *dirty_words receives the count
 * of words that do not (0 when the invariant holds).  KIE_ERR_STATE if the last
 * launch completed fewer than 2 steps.  Copies the sets to the host. */
kie_status kie_check_idle_sets(const kie_engine* e, uint64_t* dirty_words);

/* Per-token timeline.  kie_trace_words(e) = uint64 words a trace buffer
 * needs: (n_layers*6 + 3) slots x grid work-groups x 4 stamps.  After
 * kie_set_trace(e, buf, step), every persistent launch of the engine stamps
 * loop iteration `step` (relative to the launch) into buf: for slot s (layer l
 * stage k at s = 6*l + k with k = 0 QKV, 1 attention, 2 merge, 3 Wo,
 * 4 gate/up, 5 down; then s = 6*L LM head, 6*L + 1 step tail: partial
 * published / partials gathered / exchange set recycled / token known) and
 * work-group w, buf[(w*S + s)*4 + j] (S = n_layers*6 + 3 slots per work-group)
 * holds the 100 MHz real-time counter at
 * stage entry (j = 0), when the stage's input had arrived (j = 1), when its
 * arithmetic was done (j = 2) and at stage exit (j = 3).  Thread 0 of each
 * work-group writes them (the recycling stamp: thread 256); entries a
 * work-group does not reach are left untouched.  buf = NULL turns tracing off
 * (the default). */
size_t kie_trace_words(const kie_engine* e);
kie_status kie_set_trace(kie_engine* e, uint64_t* trace_dev, int32_t step);

/* Host-only self-check of the weight-stream tiling for cfg on `grid`
 * work-groups (no GPU): every 16-byte vector each thread of each GEMV stage
 * (QKV, Wo, gate/up, down, LM head) loads -- including the vectors the
 * previous stage prefetches -- lies inside its weight matrix, in-range
 * vectors are exactly the (row, column) the stage owns, and with full != 0
 * every vector of every matrix is loaded exactly once by the grid (else a
 * sample of work-groups is checked).  KIE_OK, or KIE_ERR_UNSUPPORTED on the
 * first violation (described on stderr when KIE_VERBOSE is set). */
kie_status kie_check_tiling(const kie_config* cfg, int32_t grid, int32_t full);

/* ---- isolated GEMV probe -------------------------------------------------- */

/* y[i] = W * x[i] for i < n_vec, in ONE persistent launch of the same GEMV
 * engine the decode kernel uses (dwordx4 weight streaming, dot2 with fp32
 * accumulation, per-row split-K reduction inside each work-group).  W_dev
 * [n_copies][rows][cols] of dtype: vector i uses copy i % n_copies (several
 * copies defeat the memory-side cache).  x_dev [n_vec][cols] of dtype;
 * y_dev [n_vec][rows] float.  cols a multiple of 256; rows >= 1.
 * input_first = 0 (stage order): each product issues its first block of
 * weight vectors, then reads its input vector, as a decode stage whose
 * weights were prefetched before its input arrived by hand-off.
 * input_first = 1: each product reads its input vector first and issues its
 * weight vectors right behind it (the order when the input is at hand).
 * Both orders give the same y.
 * *kernel_ms receives the launch duration (HIP events) if not NULL.
 * Runs on hip_stream (NULL = default) and synchronises it.  KIE_ERR_ARG for a
 * NULL or misaligned pointer, a bad size, dtype or input_first flag. */
kie_status kie_gemv_probe(const void* W_dev, int32_t rows, int32_t cols, int32_t n_copies,
                          const void* x_dev, float* y_dev, int32_t n_vec, int32_t dtype,
                          int32_t input_first, void* hip_stream, float* kernel_ms);

/* ---- read-stream probe --------------------------------------------------- */

/* The HBM read-stream ceiling the decode kernel's GEMVs are measured against:
 * batch-1 decode is bound by memory bandwidth (revietech.ru page, section
 * "Tsifry proizvoditelnosti"), and what a kernel can actually stream is below
 * the published peak.  ONE grid-wide launch (one work-group of 512 threads per
 * compute unit) reads buf_dev (bytes, 16-byte aligned; choose it larger than
 * the 256 MB memory-side cache) reps times with the decode kernel's load form
 * (non-temporal dwordx4), `depth` loads in flight per thread (1, 2, 3, 4, 6 or
 * 8: 8 KiB to 64 KiB per compute unit).  Each work-group reads whole passes of
 * 512 vectors of its contiguous share; bytes read = grid * 512 * 16 *
 * floor(bytes / 16 / grid / 512) * reps.  sink_dev: device uint32[1024] the
 * kernel may write (keeps the loads; normally untouched).  *kernel_ms: launch
 * time (HIP events on hip_stream).  KIE_ERR_ARG for a bad depth or pointer,
 * KIE_ERR_CAPACITY when the buffer gives a work-group fewer than `depth` passes. */
kie_status kie_stream_probe(const void* buf_dev, size_t bytes, int32_t depth, int32_t reps,
                            uint32_t* sink_dev, void* hip_stream, float* kernel_ms);

/* ---- matrix-core GEMM probe ----------------------------------------------- */

/* One product of the prompt path's matrix-core GEMM alone, in exactly the
 * launch sequence kie_prefill uses for it (batch-1 decode is bound by memory
 * bandwidth, the prompt by compute: revietech.ru page, section "Tsifry
 * proizvoditelnosti"; the prompt goes to the matrix cores):
 *   KIE_GEMM_STORE:  C = A W^T        (the QKV projection)
 *   KIE_GEMM_ADD:    C += A W^T       (Wo, down: the residual add)
 *   KIE_GEMM_SWIGLU: H = silu(A W^T) * (A W2^T)   (gate W, up W2)
 * A_dev [M][K]: fp16 for dtype KIE_F16; fp32 for KIE_BF16 (split into three
 * bf16 terms, one product each, as the prompt path does).  W_dev, W2_dev
 * [N][K] of dtype (W2_dev only for SWIGLU).  out_dev: C fp32 [M][N] (STORE,
 * ADD) or H [M][N] (SWIGLU; fp16 for KIE_F16, fp32 for KIE_BF16).  1 <= M <=
 * 65536, K a multiple of 64 up to 65536, N up to 65536 and a multiple of 128
 * (STORE, ADD) or 64 (SWIGLU), M * N < 2^31; every pointer 16-byte aligned.
 * fp16 products run on 256 x 256 tiles when that grid fills the GPU (at least
 * 256 tiles; gate/up + SwiGLU 512), on 128 x 128 tiles otherwise.
 * With fewer than 512 output tiles of 128 x 128, STORE and ADD split the
 * reduction into S <= 4 slices whose fp32 partial products go to part_dev
 * (at least S * M * N * 4 bytes, KIE_ERR_CAPACITY otherwise; unused when S =
 * 1) and are added in order; *slices receives S if not NULL.  The product
 * runs `reps` times back to back (ADD accumulates every time); *kernel_ms
 * receives the mean time per product (HIP events on hip_stream, which the
 * call synchronises).  KIE_ERR_ARG for anything out of range. */
enum { KIE_GEMM_STORE = 0, KIE_GEMM_ADD = 1, KIE_GEMM_SWIGLU = 2 };
kie_status kie_gemm_probe(int32_t op, int32_t dtype, const void* A_dev, int32_t M, int32_t K,
                          const void* W_dev, const void* W2_dev, int32_t N, void* out_dev, void* part_dev,
                          size_t part_bytes, int32_t reps, void* hip_stream, int32_t* slices,
                          float* kernel_ms);

/* ---- matrix-core attention probe ------------------------------------------ */

/* One causal flash attention of the prompt path alone, in the launch
 * kie_prefill uses (the prompt is part of the work the pages put on the GPU:
 * revietech.ru page, section "Chto takoye monokernel"): query row m = 0 .. M-1
 * at position p0 + m attends to cache rows 0 .. p0 + m.
 *   qkv_dev: fp32 [M][ldq], ldq = n_heads*head_dim + 2*n_kv_heads*head_dim
 *     (the prompt path's QKV rows, q already rotated; only the first
 *     n_heads*head_dim columns are read).
 *   k_cache_dev, v_cache_dev: [n_kv_heads][max_seq][head_dim] of dtype, rows
 *     0 .. p0+M-1 filled.
 *   out_dev: [M][n_heads*head_dim]: fp16 for KIE_F16, fp32 for KIE_BF16.
 * head_dim 64 or 128; n_heads / n_kv_heads in {1, 2, 4, 8}; 1 <= M <= 65536;
 * p0 + M <= max_seq; pointers 16-byte aligned.  Scores and the weighted sum run
 * on the matrix cores: queries (scaled by 1/sqrt(head_dim)) and softmax
 * weights as fp16 operands (bf16 models: two bf16 terms each), fp32
 * accumulation, softmax in base 2.  reps and *kernel_ms as for
 * kie_gemm_probe.  KIE_ERR_ARG for anything out of range. */
kie_status kie_attn_probe(int32_t dtype, const float* qkv_dev, int32_t M, int32_t n_heads, int32_t n_kv_heads,
                          int32_t head_dim, int32_t p0, int32_t max_seq, const void* k_cache_dev,
                          const void* v_cache_dev, void* out_dev, int32_t reps, void* hip_stream,
                          float* kernel_ms);

/* ---- hand-off latency probe ---------------------------------------------- */

/* The cost of one exchange between work-groups, which the persistent kernel
 * pays at every stage boundary in place of a kernel launch (revietech.ru page,
 * section "Chto takoye monokernel": the work stays resident and work-groups
 * synchronise through memory).  ONE cooperative launch of one work-group of
 * 512 threads per compute unit uses the decode kernel's exchange form: 8-byte
 * agent-scope stores polled with agent-scope loads, s_sleep 1 between polls.
 *   KIE_PROBE_PING: work-groups wg_a and wg_b (distinct, < grid) trade
 *     `rounds` round trips, one thread each: a stores round r, b answers once
 *     it sees r.  exchange_us = mean round trip.
 *   KIE_PROBE_ALL_TO_ALL: every work-group publishes round r in its own word
 *     and waits until all grid words hold r (wave 0; each lane polls grid/64
 *     words together).  The words lie slot_stride 8-byte words apart (1, 2,
 *     4, 8 or 16: 16 producers share a 128-byte line at 1, none at 16).
 *     exchange_us = mean over work-groups of the mean round,
 *     exchange_max_us = the slowest work-group's.  wg_a, wg_b are ignored.
 * Two untimed rounds come first.  stream_where adds non-temporal dwordx4
 * streaming of buf_dev (stream_depth = 1, 2, 3, 4 or 8 loads in flight per
 * thread) by KIE_PROBE_STREAM_OTHERS (all threads of the work-groups that do
 * not exchange; ping only) and/or KIE_PROBE_STREAM_OWN (waves 1..7 of the
 * exchanging work-groups), until the exchange ends; stream_gbps = their read
 * rate over their common window.  buf_dev: 16-byte aligned, at least
 * grid * 512 * 16 * 33 * stream_depth bytes (KIE_ERR_CAPACITY below), unused
 * with KIE_PROBE_STREAM_NONE.  scratch_dev: device memory of at least
 * KIE_HANDOFF_PROBE_SCRATCH_BYTES (enough for any grid and stride), cleared
 * by the call.  Each wait gives up after 10 ms (completed = 0 then).  xcc_a, xcc_b: the accelerator die (XCD)
 * work-groups a and b (all-to-all: 0 and 1) ran on.  Runs on hip_stream and
 * synchronises it.  KIE_ERR_ARG for arguments out of range. */
enum {
  KIE_PROBE_PING = 0,
  KIE_PROBE_ALL_TO_ALL = 1,
  KIE_PROBE_STREAM_NONE = 0,
  KIE_PROBE_STREAM_OTHERS = 1,
  KIE_PROBE_STREAM_OWN = 2
};
#define KIE_HANDOFF_PROBE_SCRATCH_BYTES (192u * 1024u)
typedef struct {
  double exchange_us;
  double exchange_max_us;
  double stream_gbps;
  int32_t xcc_a, xcc_b;
  int32_t completed;
  int32_t grid;
} kie_handoff_probe_result;

kie_status kie_handoff_probe(int32_t kind, int32_t wg_a, int32_t wg_b, int32_t rounds,
                             int32_t slot_stride, int32_t stream_depth, int32_t stream_where, const void* buf_dev,
                             size_t bytes, uint64_t* scratch_dev, size_t scratch_bytes,
                             void* hip_stream, kie_handoff_probe_result* out);

#ifdef __cplusplus
}
#endif

#endif /* KIE_H */
