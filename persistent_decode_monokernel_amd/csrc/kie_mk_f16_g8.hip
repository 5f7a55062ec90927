// Instantiations of the persistent decode kernel: f16, 8 query heads per KV head.
#include "kie_monokernel.hpp"

namespace kie {
const void* monokernel_fn_f16_g8(int vd, int vf) {
  if (vd == 0 && vf == 1) return reinterpret_cast<const void*>(&monokernel<KIE_F16, 8, 0, 1>);
  if (vd == 1 && vf == 1) return reinterpret_cast<const void*>(&monokernel<KIE_F16, 8, 1, 1>);
  if (vd == 1 && vf == 2) return reinterpret_cast<const void*>(&monokernel<KIE_F16, 8, 1, 2>);
  if (vd == 1 && vf == 4) return reinterpret_cast<const void*>(&monokernel<KIE_F16, 8, 1, 4>);
  return nullptr;
}
}  // namespace kie
