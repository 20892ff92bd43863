// K4: gate-weighted combine of a token's k expert outputs (k >= 2).
//
// out_t = sum_j gate[t, j] * y[scatter[t*k + j]], the weighted sum of the
// selected experts' outputs (telknet.cc article, section 2.1; ZONOS2 digest
// item 5: the last MoE layer routes each token to two experts).  Summation is
// in fp32 in j order, so the result does not depend on scheduling.  For k = 1
// this step is folded into the down-projection epilogue.  In a stack of bf16
// layers the residual add follows: out_t = bf16(res_t + bf16(sum)).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

template <bool BF16>
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ ybuf,
                                                 const float* __restrict__ gate,
                                                 const int* __restrict__ scatter, int T, int k,
                                                 int d, const uint16_t* __restrict__ res,
                                                 void* __restrict__ out) {
  const int groups = d / 4;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)T * groups) return;
  const int t = (int)(idx / groups), g4 = (int)(idx % groups);
  u32x2 hv = {0u, 0u};  // in a stack (bf16 res): the residual stream's four values
  if (BF16 && res != nullptr) hv = *reinterpret_cast<const u32x2*>(res + (size_t)t * d + g4 * 4);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const int slot = scatter[(size_t)t * k + j];
    const float w = gate[(size_t)t * k + j];
    const f32x4 y = *reinterpret_cast<const f32x4*>(ybuf + (size_t)slot * d + g4 * 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = fmaf(w, y[q], acc[q]);
  }
  if constexpr (BF16) {
    u32x2 v;
    v[0] = pack_bf16x2(acc[0], acc[1]);
    v[1] = pack_bf16x2(acc[2], acc[3]);
    if (res != nullptr) {  // bf16(res + bf16(sum))
#pragma unroll
      for (int q = 0; q < 2; ++q)
        v[q] = pack_bf16x2(bf16_lo(hv[q]) + bf16_lo(v[q]), bf16_hi(hv[q]) + bf16_hi(v[q]));
    }
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(out) + (size_t)t * d + g4 * 4) = v;
  } else {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + (size_t)t * d + g4 * 4) = acc;
  }
}

hipError_t launch_combine(const FwdArgs& a) {
  const size_t total = (size_t)a.T * (a.dim.d / 4);
  const unsigned grid = (unsigned)((total + 255) / 256);
  const KEv& ev = a.ev[kSlotCombine];
  if (a.dim.dtype == 1)
    return launch(k_combine<true>, dim3(grid), dim3(256), a.stream, ev, (const float*)a.ybuf,
                  (const float*)a.gate, (const int*)a.scatter, a.T, a.dim.k, a.dim.d,
                  (const uint16_t*)a.res, a.out);
  return launch(k_combine<false>, dim3(grid), dim3(256), a.stream, ev, (const float*)a.ybuf,
                (const float*)a.gate, (const int*)a.scatter, a.T, a.dim.k, a.dim.d, nullptr,
                a.out);
}

}  // namespace moe
