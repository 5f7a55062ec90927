// Instantiations of the persistent decode kernel: bf16, 4 query heads per KV head,
// every (d_model, d_ffn) GEMV width-class pair the runtime accepts.
#include "kie_monokernel.hpp"

namespace kie {
const void* monokernel_fn_bf16_g4(int vd, int vf) {
  if (vd == 0 && vf == 1) return reinterpret_cast<const void*>(&monokernel<KIE_BF16, 4, 0, 1, false>);
  if (vd == 0 && vf == 2) return reinterpret_cast<const void*>(&monokernel<KIE_BF16, 4, 0, 2, false>);
  if (vd == 0 && vf == 4) return reinterpret_cast<const void*>(&monokernel<KIE_BF16, 4, 0, 4, false>);
  if (vd == 1 && vf == 1) return reinterpret_cast<const void*>(&monokernel<KIE_BF16, 4, 1, 1, false>);
  if (vd == 1 && vf == 2) return reinterpret_cast<const void*>(&monokernel<KIE_BF16, 4, 1, 2, false>);
  if (vd == 1 && vf == 4) return reinterpret_cast<const void*>(&monokernel<KIE_BF16, 4, 1, 4, false>);
  if (vd == 2 && vf == 2) return reinterpret_cast<const void*>(&monokernel<KIE_BF16, 4, 2, 2, false>);
  if (vd == 2 && vf == 4) return reinterpret_cast<const void*>(&monokernel<KIE_BF16, 4, 2, 4, false>);
  if (vd == 4 && vf == 4) return reinterpret_cast<const void*>(&monokernel<KIE_BF16, 4, 4, 4, false>);
  return nullptr;
}

// The same instances as one launch per stage (the launch-tax comparison).
const void* stage_kernel_fn_bf16_g4(int vd, int vf) {
  if (vd == 0 && vf == 1) return reinterpret_cast<const void*>(&stage_kernel<KIE_BF16, 4, 0, 1>);
  if (vd == 0 && vf == 2) return reinterpret_cast<const void*>(&stage_kernel<KIE_BF16, 4, 0, 2>);
  if (vd == 0 && vf == 4) return reinterpret_cast<const void*>(&stage_kernel<KIE_BF16, 4, 0, 4>);
  if (vd == 1 && vf == 1) return reinterpret_cast<const void*>(&stage_kernel<KIE_BF16, 4, 1, 1>);
  if (vd == 1 && vf == 2) return reinterpret_cast<const void*>(&stage_kernel<KIE_BF16, 4, 1, 2>);
  if (vd == 1 && vf == 4) return reinterpret_cast<const void*>(&stage_kernel<KIE_BF16, 4, 1, 4>);
  if (vd == 2 && vf == 2) return reinterpret_cast<const void*>(&stage_kernel<KIE_BF16, 4, 2, 2>);
  if (vd == 2 && vf == 4) return reinterpret_cast<const void*>(&stage_kernel<KIE_BF16, 4, 2, 4>);
  if (vd == 4 && vf == 4) return reinterpret_cast<const void*>(&stage_kernel<KIE_BF16, 4, 4, 4>);
  return nullptr;
}

// The arrival-counter comparison instance, for the shapes it is measured on
// (4 query heads per KV head, both widths in the 4-vectors-per-lane class).
const void* monokernel_counters_fn_bf16_g4(int vd, int vf) {
  if (vd == 4 && vf == 4) return reinterpret_cast<const void*>(&monokernel<KIE_BF16, 4, 4, 4, true>);
  return nullptr;
}

}  // namespace kie
