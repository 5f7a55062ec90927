// Instantiations of the persistent decode kernel: bf16, 8 query heads per KV head,
// every (d_model, d_ffn) GEMV width-class pair the runtime accepts.
#include "kie_monokernel.hpp"

namespace kie {
const void* monokernel_fn_bf16_g8(int vd, int vf) {
  if (vd == 0 && vf == 1) return reinterpret_cast<const void*>(&monokernel<KIE_BF16, 8, 0, 1, false>);
  if (vd == 0 && vf == 2) return reinterpret_cast<const void*>(&monokernel<KIE_BF16, 8, 0, 2, false>);
  if (vd == 0 && vf == 4) return reinterpret_cast<const void*>(&monokernel<KIE_BF16, 8, 0, 4, false>);
  if (vd == 1 && vf == 1) return reinterpret_cast<const void*>(&monokernel<KIE_BF16, 8, 1, 1, false>);
  if (vd == 1 && vf == 2) return reinterpret_cast<const void*>(&monokernel<KIE_BF16, 8, 1, 2, false>);
  if (vd == 1 && vf == 4) return reinterpret_cast<const void*>(&monokernel<KIE_BF16, 8, 1, 4, false>);
  if (vd == 2 && vf == 2) return reinterpret_cast<const void*>(&monokernel<KIE_BF16, 8, 2, 2, false>);
  if (vd == 2 && vf == 4) return reinterpret_cast<const void*>(&monokernel<KIE_BF16, 8, 2, 4, false>);
  if (vd == 4 && vf == 4) return reinterpret_cast<const void*>(&monokernel<KIE_BF16, 8, 4, 4, false>);
  return nullptr;
}

// The same instances as one launch per stage (the launch-tax comparison).
const void* stage_kernel_fn_bf16_g8(int vd, int vf) {
  if (vd == 0 && vf == 1) return reinterpret_cast<const void*>(&stage_kernel<KIE_BF16, 8, 0, 1>);
  if (vd == 0 && vf == 2) return reinterpret_cast<const void*>(&stage_kernel<KIE_BF16, 8, 0, 2>);
  if (vd == 0 && vf == 4) return reinterpret_cast<const void*>(&stage_kernel<KIE_BF16, 8, 0, 4>);
  if (vd == 1 && vf == 1) return reinterpret_cast<const void*>(&stage_kernel<KIE_BF16, 8, 1, 1>);
  if (vd == 1 && vf == 2) return reinterpret_cast<const void*>(&stage_kernel<KIE_BF16, 8, 1, 2>);
  if (vd == 1 && vf == 4) return reinterpret_cast<const void*>(&stage_kernel<KIE_BF16, 8, 1, 4>);
  if (vd == 2 && vf == 2) return reinterpret_cast<const void*>(&stage_kernel<KIE_BF16, 8, 2, 2>);
  if (vd == 2 && vf == 4) return reinterpret_cast<const void*>(&stage_kernel<KIE_BF16, 8, 2, 4>);
  if (vd == 4 && vf == 4) return reinterpret_cast<const void*>(&stage_kernel<KIE_BF16, 8, 4, 4>);
  return nullptr;
}
}  // namespace kie
