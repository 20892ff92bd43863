// Zero fill of a device buffer by a kernel (not hipMemsetAsync), so that it
// can sit inside a captured HIP graph: clears the zero row of the static
// scratch before a forward that uses it.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

__global__ __launch_bounds__(256) void k_zero16(u32x4* __restrict__ p, size_t n16) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n16) p[i] = u32x4{0u, 0u, 0u, 0u};
}

// bytes: a multiple of 16; p: 16-byte aligned.
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  hipLaunchKernelGGL(k_zero16, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, s,
                     static_cast<u32x4*>(p), n16);
  return hipGetLastError();
}

}  // namespace moe
