// Instantiations of the persistent decode kernel: bf16, 2 query heads per KV head,
// every (d_model, d_ffn) GEMV width-class pair the runtime accepts.
#include "kie_monokernel.hpp"

namespace kie {
const void* monokernel_fn_bf16_g2(int vd, int vf) {
  if (vd == 0 && vf == 1) return reinterpret_cast<const void*>(&monokernel<KIE_BF16, 2, 0, 1>);
  if (vd == 0 && vf == 2) return reinterpret_cast<const void*>(&monokernel<KIE_BF16, 2, 0, 2>);
  if (vd == 0 && vf == 4) return reinterpret_cast<const void*>(&monokernel<KIE_BF16, 2, 0, 4>);
  if (vd == 1 && vf == 1) return reinterpret_cast<const void*>(&monokernel<KIE_BF16, 2, 1, 1>);
  if (vd == 1 && vf == 2) return reinterpret_cast<const void*>(&monokernel<KIE_BF16, 2, 1, 2>);
  if (vd == 1 && vf == 4) return reinterpret_cast<const void*>(&monokernel<KIE_BF16, 2, 1, 4>);
  if (vd == 2 && vf == 2) return reinterpret_cast<const void*>(&monokernel<KIE_BF16, 2, 2, 2>);
  if (vd == 2 && vf == 4) return reinterpret_cast<const void*>(&monokernel<KIE_BF16, 2, 2, 4>);
  if (vd == 4 && vf == 4) return reinterpret_cast<const void*>(&monokernel<KIE_BF16, 2, 4, 4>);
  return nullptr;
}
}  // namespace kie
