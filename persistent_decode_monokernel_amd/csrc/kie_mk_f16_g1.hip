// Instantiations of the persistent decode kernel: f16, 1 query head per KV head,
// every (d_model, d_ffn) GEMV width-class pair the runtime accepts.
#include "kie_monokernel.hpp"

namespace kie {
const void* monokernel_fn_f16_g1(int vd, int vf) {
  if (vd == 0 && vf == 1) return reinterpret_cast<const void*>(&monokernel<KIE_F16, 1, 0, 1>);
  if (vd == 0 && vf == 2) return reinterpret_cast<const void*>(&monokernel<KIE_F16, 1, 0, 2>);
  if (vd == 0 && vf == 4) return reinterpret_cast<const void*>(&monokernel<KIE_F16, 1, 0, 4>);
  if (vd == 1 && vf == 1) return reinterpret_cast<const void*>(&monokernel<KIE_F16, 1, 1, 1>);
  if (vd == 1 && vf == 2) return reinterpret_cast<const void*>(&monokernel<KIE_F16, 1, 1, 2>);
  if (vd == 1 && vf == 4) return reinterpret_cast<const void*>(&monokernel<KIE_F16, 1, 1, 4>);
  if (vd == 2 && vf == 2) return reinterpret_cast<const void*>(&monokernel<KIE_F16, 1, 2, 2>);
  if (vd == 2 && vf == 4) return reinterpret_cast<const void*>(&monokernel<KIE_F16, 1, 2, 4>);
  if (vd == 4 && vf == 4) return reinterpret_cast<const void*>(&monokernel<KIE_F16, 1, 4, 4>);
  return nullptr;
}
}  // namespace kie
