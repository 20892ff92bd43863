// K3 (fp32 layers): SwiGLU experts in fp32 on the vector ALUs.
//
// Same computation as the bf16 grouped GEMM (SwiGLU expert, GLU variants paper
// on the ZONOS2 report's "Builds on" list) for layers stored in fp32, where
// bf16 matrix cores would not hold the fp32 result.  One thread per output
// element, rows taken through the expert-ordered slot list.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

__global__ __launch_bounds__(256) void k_gateup_f32(const float* __restrict__ wg,
                                                    const float* __restrict__ wu,
                                                    const float* __restrict__ xn,
                                                    const int* __restrict__ gather,
                                                    const int* __restrict__ slot_expert,
                                                    const float* __restrict__ inv, int n,
                                                    int d, int F, float* __restrict__ act) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)n * F) return;
  const int p = (int)(idx / F), f = (int)(idx % F);
  const int e = slot_expert[p];
  const float* x = xn + (size_t)gather[p] * d;
  const float* g = wg + ((size_t)e * F + f) * d;
  const float* u = wu + ((size_t)e * F + f) * d;
  float sg = 0.f, su = 0.f;
  for (int i = 0; i < d; i += 4) {
    const f32x4 xv = *reinterpret_cast<const f32x4*>(x + i);
    const f32x4 gv = *reinterpret_cast<const f32x4*>(g + i);
    const f32x4 uv = *reinterpret_cast<const f32x4*>(u + i);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      sg = fmaf(gv[q], xv[q], sg);
      su = fmaf(uv[q], xv[q], su);
    }
  }
  const float s = inv[gather[p]];  // RMSNorm scale of this token
  sg *= s;
  su *= s;
  act[(size_t)p * F + f] = sg / (1.0f + expf(-sg)) * su;
}

__global__ __launch_bounds__(256) void k_down_f32(const float* __restrict__ wd,
                                                  const float* __restrict__ act,
                                                  const int* __restrict__ gather,
                                                  const int* __restrict__ slot_expert,
                                                  const float* __restrict__ gate, int n, int d,
                                                  int F, int k, float* __restrict__ out,
                                                  float* __restrict__ ybuf) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)n * d) return;
  const int p = (int)(idx / d), m = (int)(idx % d);
  const int e = slot_expert[p];
  const float* a = act + (size_t)p * F;
  const float* w = wd + ((size_t)e * d + m) * F;
  float s = 0.f;
  for (int f = 0; f < F; f += 4) {
    const f32x4 av = *reinterpret_cast<const f32x4*>(a + f);
    const f32x4 wv = *reinterpret_cast<const f32x4*>(w + f);
#pragma unroll
    for (int q = 0; q < 4; ++q) s = fmaf(wv[q], av[q], s);
  }
  if (k == 1) {
    const int tok = gather[p];
    out[(size_t)tok * d + m] = gate[tok] * s;
  } else {
    ybuf[(size_t)p * d + m] = s;
  }
}

hipError_t launch_experts_f32(const FwdArgs& a) {
  const int d = a.dim.d, F = a.dim.F, n = a.n;
  const size_t g1 = ((size_t)n * F + 255) / 256;
  hipError_t err = launch(k_gateup_f32, dim3((unsigned)g1), dim3(256), a.stream,
                          a.ev[kSlotExpertsA], (const float*)a.wgu, (const float*)a.wup,
                          (const float*)a.xn, (const int*)a.gather, (const int*)a.slot_expert,
                          (const float*)a.inv, n, d, F, (float*)a.act);
  if (err != hipSuccess) return err;
  const size_t g2 = ((size_t)n * d + 255) / 256;
  return launch(k_down_f32, dim3((unsigned)g2), dim3(256), a.stream, a.ev[kSlotExpertsB],
                (const float*)a.wd, (const float*)a.act, (const int*)a.gather,
                (const int*)a.slot_expert, (const float*)a.gate, n, d, F, a.dim.k, (float*)a.out,
                a.ybuf);
}

}  // namespace moe
