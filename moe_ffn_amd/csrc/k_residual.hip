// Residual add between the layers of an FFN stack: h_next = h + ffn(h)
// (fp32 stacks; bf16 layers add their output to the residual stream in their
// last kernel, with the same roundings as k_residual_bf16).
//
// The ZONOS2 backbone stacks 28 layers (digest item 5: the first three and
// the last one dense, the middle ones MoE); each layer's FFN output is added
// to the residual stream it read.  Stored in the activations' type: bf16
// rounds the fp32 sum of the two bf16 values once (round to nearest even);
// fp32 adds in fp32.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

__global__ __launch_bounds__(256) void k_residual_bf16(const uint16_t* __restrict__ h,
                                                       const uint16_t* __restrict__ y,
                                                       uint16_t* __restrict__ out, size_t n8) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;  // 8 elements per thread
  if (i >= n8) return;
  const u32x4 a = ldg16(h + i * 8), b = ldg16(y + i * 8);
  u32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    o[q] = pack_bf16x2(bf16_lo(a[q]) + bf16_lo(b[q]), bf16_hi(a[q]) + bf16_hi(b[q]));
  stg16(out + i * 8, o);
}

__global__ __launch_bounds__(256) void k_residual_f32(const float* __restrict__ h,
                                                      const float* __restrict__ y,
                                                      float* __restrict__ out, size_t n4) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;  // 4 elements per thread
  if (i >= n4) return;
  const f32x4 a = *reinterpret_cast<const f32x4*>(h + i * 4);
  const f32x4 b = *reinterpret_cast<const f32x4*>(y + i * 4);
  *reinterpret_cast<f32x4*>(out + i * 4) = a + b;
}

// n: elements (a multiple of 8 for bf16, of 4 for fp32: d_model is).
hipError_t launch_residual(const void* h, const void* y, void* out, size_t n, int dtype,
                           hipStream_t s) {
  if (dtype == 1) {
    const size_t n8 = n / 8;
    hipLaunchKernelGGL(k_residual_bf16, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s,
                       (const uint16_t*)h, (const uint16_t*)y, (uint16_t*)out, n8);
  } else {
    const size_t n4 = n / 4;
    hipLaunchKernelGGL(k_residual_f32, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s,
                       (const float*)h, (const float*)y, (float*)out, n4);
  }
  return hipGetLastError();
}

}  // namespace moe
