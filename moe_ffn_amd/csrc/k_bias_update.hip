// Auxiliary-loss-free balancing step on the router bias.
//
// The ZONOS2 report keeps a per-expert bias b_l that steers routing toward
// uniform expert usage (digest item 6) and builds on the auxiliary-loss-free
// load-balancing paper (index page, "Builds on"), whose step moves every bias
// by a fixed rate toward balance:
//   b_e <- b_e + rate * sign(mean load - c_e)
// with c_e the expert's assignment count in the last batch.  The sign is that
// of the integer sum(c) - E * c_e, so no division or rounding decides it; the
// float32 add rounds the exact b_e + rate * s_e once.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

__global__ __launch_bounds__(64) void k_bias_update(const int* __restrict__ counts, int E,
                                                    float rate, float* __restrict__ bias) {
  const int e = threadIdx.x;
  long long total = 0;
  for (int i = 0; i < E; ++i) total += counts[i];
  if (e >= E) return;
  const long long diff = total - (long long)E * counts[e];
  const float s = diff > 0 ? 1.f : (diff < 0 ? -1.f : 0.f);
  bias[e] = bias[e] + rate * s;
}

hipError_t launch_bias_update(const int* counts, int E, float rate, float* bias, hipStream_t s) {
  hipLaunchKernelGGL(k_bias_update, dim3(1), dim3(64), 0, s, counts, E, rate, bias);
  return hipGetLastError();
}

}  // namespace moe
