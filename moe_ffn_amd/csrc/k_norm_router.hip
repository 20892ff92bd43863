// K1 (fp32 layers): fused RMSNorm + linear router + bias-steered top-k + gates.
//
// ZONOS2 Technical Report (audio-paper-digest page, "Method overview and
// architecture"): item 5 normalises the backbone input with RMSNorm and routes
// every token to 1 of 16 experts (2 in the last MoE layer); item 6 keeps a
// per-expert bias vector b_l for load balancing.  The bias only moves the
// choice (s = z + b); gates come from the unbiased logits z.
//
// One workgroup (256 threads) handles TOK consecutive tokens.  Each thread owns
// 16-byte chunks of the d_model axis and accumulates, in one pass over h, the
// sum of squares and the E dot products with the gain-folded router rows
// (W_r[e][i] * g[i], each product rounded once to fp32):  z_e = inv_rms * sum_i
// (W_r g)_{e,i} h_i.  The TOK x E partial sums are reduced by a butterfly that
// spreads the totals over the lanes, then across the four waves through LDS.
// A second pass writes x' = g * h for the experts and inv_rms per token; the
// experts apply inv_rms to their fp32 accumulators.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

template <int EP, int TOK>
__global__ __launch_bounds__(256) void k_norm_router(const void* __restrict__ hidden, int T, int d,
                                                     const float* __restrict__ wrg,
                                                     const float* __restrict__ gain,
                                                     const float* __restrict__ bias, int E, int k,
                                                     float eps, void* __restrict__ xn,
                                                     float* __restrict__ inv_out,
                                                     int* __restrict__ sel, float* __restrict__ gate) {
  constexpr int VEC = 4;  // fp32 elements per 16-byte chunk
  constexpr int NV = TOK * EP;
  constexpr int R = NV >= 64 ? NV / 64 : 1;
  __shared__ float red[4][NV];
  __shared__ float ssr[4][TOK];
  __shared__ float zs[NV];
  __shared__ float inv_s[TOK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * TOK;
  const int nch = d / VEC;
  const char* hb = reinterpret_cast<const char*>(hidden);
  const size_t row_bytes = (size_t)d * 4;

  float acc[NV];
  float ss[TOK];
#pragma unroll
  for (int i = 0; i < NV; ++i) acc[i] = 0.f;
#pragma unroll
  for (int t = 0; t < TOK; ++t) ss[t] = 0.f;

  for (int c = tid; c < nch; c += 256) {
    float h[TOK][VEC];
#pragma unroll
    for (int t = 0; t < TOK; ++t) {
      if (t0 + t < T) {
        const u32x4 v = ldg16(hb + (size_t)(t0 + t) * row_bytes + (size_t)c * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) h[t][i] = __uint_as_float(v[i]);
      } else {
#pragma unroll
        for (int i = 0; i < VEC; ++i) h[t][i] = 0.f;
      }
#pragma unroll
      for (int i = 0; i < VEC; ++i) ss[t] = fmaf(h[t][i], h[t][i], ss[t]);
    }
#pragma unroll
    for (int e = 0; e < EP; ++e) {
      float w[VEC];
      const float* wp = wrg + (size_t)e * d + (size_t)c * VEC;
#pragma unroll
      for (int q = 0; q < VEC / 4; ++q) {
        const u32x4 v = ldg16(wp + 4 * q);
#pragma unroll
        for (int i = 0; i < 4; ++i) w[4 * q + i] = __uint_as_float(v[i]);
      }
#pragma unroll
      for (int t = 0; t < TOK; ++t) {
        float s = acc[t * EP + e];
#pragma unroll
        for (int i = 0; i < VEC; ++i) s = fmaf(w[i], h[t][i], s);
        acc[t * EP + e] = s;
      }
    }
  }

  WaveSpread<NV, 32>::run(acc, lane);
  WaveSpread<TOK, 32>::run(ss, lane);
  if (spread_owner<NV>(lane)) {
#pragma unroll
    for (int i = 0; i < R; ++i) red[wave][spread_index<NV>(lane, i)] = acc[i];
  }
  if (spread_owner<TOK>(lane)) ssr[wave][spread_index<TOK>(lane, 0)] = ss[0];
  __syncthreads();
  for (int i = tid; i < NV; i += 256) zs[i] = ((red[0][i] + red[1][i]) + red[2][i]) + red[3][i];
  if (tid < TOK) {
    const float s = ((ssr[0][tid] + ssr[1][tid]) + ssr[2][tid]) + ssr[3][tid];
    inv_s[tid] = 1.0f / sqrtf(s / (float)d + eps);
  }
  __syncthreads();

  if (tid < TOK && t0 + tid < T) {
    const int t = t0 + tid;
    const float inv = inv_s[tid];
    float z[EP], s[EP];
#pragma unroll
    for (int e = 0; e < EP; ++e) {
      z[e] = zs[tid * EP + e] * inv;
      s[e] = e < E ? z[e] + bias[e] : 0.f;
    }
    // top-k by descending s; an exact tie keeps the lower index (strict >).
    // A NaN score never wins a comparison, so `best` always lands on a valid
    // expert that is not taken yet.
    uint64_t taken = 0;
    int chosen[8];
    float zc[8];
    for (int j = 0; j < k; ++j) {
      int best = -1;
      float bs = 0.f, bz = 0.f;
#pragma unroll
      for (int e = 0; e < EP; ++e) {
        if (e < E && !((taken >> e) & 1)) {
          if (best < 0 || s[e] > bs) {
            best = e;
            bs = s[e];
            bz = z[e];
          }
        }
      }
      chosen[j] = best;
      zc[j] = bz;
      taken |= 1ull << best;
    }
    // gates from the unbiased logits
    float zmax = -INFINITY, den = 0.f;
    if (k == 1) {
#pragma unroll
      for (int e = 0; e < EP; ++e)
        if (e < E) zmax = fmaxf(zmax, z[e]);
#pragma unroll
      for (int e = 0; e < EP; ++e)
        if (e < E) den += expf(z[e] - zmax);
    } else {
      for (int j = 0; j < k; ++j) zmax = fmaxf(zmax, zc[j]);
      for (int j = 0; j < k; ++j) den += expf(zc[j] - zmax);
    }
    for (int j = 0; j < k; ++j) {
      sel[(size_t)t * k + j] = chosen[j];
      gate[(size_t)t * k + j] = expf(zc[j] - zmax) / den;
    }
    inv_out[t] = inv;
  }

  // second pass: x' = g * h for the experts
  for (int c = tid; c < nch; c += 256) {
    float g[VEC];
#pragma unroll
    for (int q = 0; q < VEC / 4; ++q) {
      const u32x4 v = ldg16(gain + (size_t)c * VEC + 4 * q);
#pragma unroll
      for (int i = 0; i < 4; ++i) g[4 * q + i] = __uint_as_float(v[i]);
    }
#pragma unroll
    for (int t = 0; t < TOK; ++t) {
      if (t0 + t >= T) break;
      const u32x4 v = ldg16(hb + (size_t)(t0 + t) * row_bytes + (size_t)c * 16);
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = __float_as_uint(__uint_as_float(v[i]) * g[i]);
      stg16(reinterpret_cast<char*>(xn) + (size_t)(t0 + t) * row_bytes + (size_t)c * 16, o);
    }
  }
}

namespace {
constexpr int tok_big(int ep) { return ep >= 64 ? 2 : (128 / ep > 16 ? 16 : 128 / ep); }

template <int EP>
hipError_t launch_ep(const FwdArgs& a) {
  constexpr int TB = tok_big(EP);
  constexpr int TS = TB < 2 ? TB : 2;
  const int T = a.T;
  const bool small = (T + TB - 1) / TB < 256;
  const KEv& ev = a.ev[kSlotNormRouter];
  if (small)
    return launch(k_norm_router<EP, TS>, dim3((T + TS - 1) / TS), dim3(256), a.stream, ev,
                  a.hidden, T, a.dim.d, a.wrg, a.gain, a.bias, a.dim.E, a.dim.k, a.dim.eps, a.xn,
                  a.inv, a.sel, a.gate);
  return launch(k_norm_router<EP, TB>, dim3((T + TB - 1) / TB), dim3(256), a.stream, ev,
                a.hidden, T, a.dim.d, a.wrg, a.gain, a.bias, a.dim.E, a.dim.k, a.dim.eps, a.xn,
                a.inv, a.sel, a.gate);
}

hipError_t launch_by_experts(const FwdArgs& a) {
  switch (a.dim.EP) {
    case 1: return launch_ep<1>(a);
    case 2: return launch_ep<2>(a);
    case 4: return launch_ep<4>(a);
    case 8: return launch_ep<8>(a);
    case 16: return launch_ep<16>(a);
    case 32: return launch_ep<32>(a);
    case 64: return launch_ep<64>(a);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace

hipError_t launch_norm_router(const FwdArgs& a) { return launch_by_experts(a); }

}  // namespace moe
