// Host interface of the matrix-core prompt path (kie_prefill.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kie.h"

namespace kie {

constexpr int kPfChunk = 8192;  // prompt positions per chunk (bounds the activation buffers)

// Device buffers and weights of one engine for the prompt path.
struct PrefillCtx {
  kie_config cfg;
  hipStream_t stream;
  const uint16_t* tok_emb;
  const uint16_t* const* wtab;  // host table [L][W_PER_LAYER] of device pointers
  const float* rope;            // [max_seq][hd/2][cos, sin]
  uint16_t* kc;                 // KV cache [L][Hkv][max_seq][hd]
  uint16_t* vc;
  float* X;                     // [chunk][d] residual
  void* Xn;                     // [chunk][d] normalised input      (activations: fp16 for
  float* QKV;                   // [chunk][qd + 2 kvd] (q rotated in place)     fp16 models,
  void* A;                      // [chunk][qd] attention output                 fp32 for
  void* H;                      // [chunk][F] SwiGLU output                     bf16 models)
  float* P;                     // split-K partial products (prefill_part_floats)
};

// Shapes the prompt path handles (fp16 or bf16 weights, head_dim 64 or 128;
// projection widths multiples of 128, reduction widths multiples of 64).
bool prefill_supported(const kie_config& c);

// Bytes of one activation element between the prompt-path kernels.
size_t prefill_act_bytes(const kie_config& c);

// fp32 elements of the split-K partial-product buffer for chunks of `chunk`.
size_t prefill_part_floats(const kie_config& c, int chunk);

// Positions p0 .. p0+M-1 (tokens tok_dev[0 .. M-1], device) through every
// layer: KV cache rows written, residual left in ctx.X.  M <= kPfChunk.
hipError_t prefill_chunk(const PrefillCtx& ctx, const int* tok_dev, int p0, int M);

}  // namespace kie
