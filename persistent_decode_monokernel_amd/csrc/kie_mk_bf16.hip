// bf16 instantiations of the persistent decode kernel.
#include "kie_monokernel.hpp"

namespace kie {
const void* monokernel_fn_bf16(int group) {
  switch (group) {
    case 1: return reinterpret_cast<const void*>(&monokernel<KIE_BF16, 1>);
    case 2: return reinterpret_cast<const void*>(&monokernel<KIE_BF16, 2>);
    case 4: return reinterpret_cast<const void*>(&monokernel<KIE_BF16, 4>);
    case 8: return reinterpret_cast<const void*>(&monokernel<KIE_BF16, 8>);
  }
  return nullptr;
}
}  // namespace kie
