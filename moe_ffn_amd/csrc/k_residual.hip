// Residual add between the layers of an fp32 FFN stack: h_next = h + ffn(h).
//
// The ZONOS2 backbone stacks 28 layers (digest item 5: the first three and
// the last one dense, the middle ones MoE); each layer's FFN output is added
// to the residual stream it read.  fp32 stacks add in fp32 here, after each
// layer.  bf16 layers add their output to the residual stream in their last
// kernel instead (out = bf16(h + bf16(ffn)): the layer output's rounding,
// then one round-to-nearest-even of the fp32 sum), which saves a launch per
// layer.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

__global__ __launch_bounds__(256) void k_residual_f32(const float* __restrict__ h,
                                                      const float* __restrict__ y,
                                                      float* __restrict__ out, size_t n4) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;  // 4 elements per thread
  if (i >= n4) return;
  const f32x4 a = *reinterpret_cast<const f32x4*>(h + i * 4);
  const f32x4 b = *reinterpret_cast<const f32x4*>(y + i * 4);
  *reinterpret_cast<f32x4*>(out + i * 4) = a + b;
}

// n: elements (a multiple of 4: d_model is).
hipError_t launch_residual_f32(const float* h, const float* y, float* out, size_t n,
                               hipStream_t s) {
  const size_t n4 = n / 4;
  hipLaunchKernelGGL(k_residual_f32, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, h, y,
                     out, n4);
  return hipGetLastError();
}

}  // namespace moe
