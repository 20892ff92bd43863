// Measurement probe, not part of the layer: the sustained rate of
// v_mfma_f32_32x32x16_bf16 on this part with register-resident operands and
// four independent accumulator chains per wave (no memory traffic in the
// loop).  bench.py reports it beside the layer's own MFMA rate, as the
// practical ceiling of the matrix cores under full load (the clock drops
// below the 2.4 GHz of the published peak).  Built into libmoe_probe.so,
// separate from libmoe_layer.so.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kChains = 4;

__global__ __launch_bounds__(256) void k_mfma_rate(int iters, float* __restrict__ sink) {
  const int l = threadIdx.x;
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1e-3f * (float)(l + i));
    b[i] = (__bf16)(2e-3f * (float)(l - i));
  }
  f32x16 acc[kChains];
  for (int j = 0; j < kChains; ++j)
    for (int i = 0; i < 16; ++i) acc[j][i] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kChains; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
  for (int j = 0; j < kChains; ++j)
    for (int i = 0; i < 16; ++i) s += acc[j][i];
  sink[(size_t)blockIdx.x * 256 + l] = s;  // keeps the chains live
}
}  // namespace

extern "C" {

// Flops one launch performs: blocks * 4 waves * iters * kChains MFMAs of
// 2 * 32 * 32 * 16 flops.
double moe_probe_mfma_flops(int32_t blocks, int32_t iters) {
  return (double)blocks * 4.0 * iters * kChains * 2.0 * 32 * 32 * 16;
}

// Enqueue one launch of `blocks` workgroups of 256 threads on `stream`
// (hipStream_t as void*); `sink` is DEVICE memory of blocks * 256 floats.
// Returns 0, or the hipError_t of the launch.
int32_t moe_probe_mfma(int32_t blocks, int32_t iters, float* sink, void* stream) {
  if (blocks <= 0 || iters <= 0 || sink == nullptr) return (int32_t)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_mfma_rate, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, sink);
  return (int32_t)hipGetLastError();
}

}  // extern "C"
