// Isolated GEMV probe kernel and the fill kernel.
#include "kie_monokernel.hpp"

namespace kie {

__global__ void fill_u32(uint32_t* p, uint64_t n, uint32_t v) {
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (uint64_t)gridDim.x * blockDim.x)
    p[i] = v;
}


const void* gemv_probe_fn(int dtype) {
  return dtype == KIE_F16 ? reinterpret_cast<const void*>(&gemv_probe<KIE_F16>)
                          : reinterpret_cast<const void*>(&gemv_probe<KIE_BF16>);
}

hipError_t launch_fill(uint32_t* p, uint64_t n, uint32_t v, hipStream_t st) {
  if (n == 0) return hipSuccess;
  uint64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_u32, dim3((unsigned)blocks), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

}  // namespace kie
