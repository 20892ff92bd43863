// K1 (bf16 layers, decode-sized batches): RMSNorm statistics + linear router +
// bias-steered top-k + gates, one workgroup per token.
//
// Same computation as the prefill router (ZONOS2 Technical Report,
// audio-paper-digest page, "Method overview and architecture", items 5 and 6:
// RMSNorm-normalised input, top-1/top-2 over 16 experts, a per-expert bias that
// moves the choice but not the gate).  At decode sizes a batch of T <= 64
// tokens would leave a single workgroup pulling the whole router and every
// hidden row through one CU, so each token gets its own workgroup: 256 threads
// own 8-element chunks of the token's row and accumulate, in one pass,
//   sum h^2,  x' = g * h (stored as bf16 for the experts),
//   z_raw[e] = sum_i W_r[e][i] * x'_i     (every product exact in fp32).
// The E partial sums are reduced by a spreading butterfly inside each wave and
// across the four waves in LDS (fixed order); then the lanes of wave 0, one per
// expert, apply inv_rms = 1/sqrt(mean(h^2) + eps) (and, when a stack passes
// its depth-averaging state eda, replace the logits z by z~ = alpha * z~_prev
// + (1 - alpha) * z; the first MoE layer only writes the state), add the
// bias, pick the top-k by wave-wide maximum reductions and write the gates.
// The dispatch of decode batches happens in the expert kernels.
//
// Layers with fp8 activations (xs != null) get the quantised expert input
// instead of x': the row's scale a = max_i |u_i| / 448 of u = bf16(inv_rms *
// x') is bf16(inv_rms * max_i |x'_i|) / 448 (both roundings are monotone), so
// the first pass also tracks max |x'|; a second pass over the row (its first
// 2048 values from registers, the rest from cache) writes the E4M3 values of
// u (quant4_e4m3, exact in bf16) and xs[t] = a.  The weight streams then
// multiply exact code values and scale the sums by a.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

template <int EP>
__global__ __launch_bounds__(256) void k_router_token(
    const uint16_t* __restrict__ hidden, int d, const uint16_t* __restrict__ wr,
    const uint16_t* __restrict__ gain, const float* __restrict__ bias, int E, int k, float eps,
    const uint16_t* __restrict__ zrow, uint16_t* __restrict__ xg, float* __restrict__ inv_out,
    int* __restrict__ sel, float* __restrict__ gate, float* __restrict__ eda, float eda_alpha,
    int eda_first, float* __restrict__ xs) {
  constexpr int NV = EP;
  constexpr int R = NV >= 64 ? NV / 64 : 1;
  __shared__ float red[4][NV];
  __shared__ float ssr[4], mxr[4];
  __shared__ float s_inv, s_r;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = blockIdx.x;
  const uint16_t* hrow = hidden + (size_t)t * d;
  uint16_t* xrow = xg + (size_t)t * d;
  const uint16_t* wrow[EP];
#pragma unroll
  for (int e = 0; e < EP; ++e) wrow[e] = e < E ? wr + (size_t)e * d : zrow;

  // wave 0's lane e finishes expert e: its bias and (depth averaging) the
  // previous MoE layer's logit are loaded now, under the main loop's loads
  float bias_e = 0.f, eda_prev = 0.f;
  if (wave == 0) {
    bias_e = bias[lane];  // bias is zero-padded to 64 entries
    if (eda != nullptr && !eda_first && lane < E) eda_prev = eda[(size_t)t * 64 + lane];
  }

  float acc[NV];
#pragma unroll
  for (int e = 0; e < NV; ++e) acc[e] = 0.f;
  float ss = 0.f, mx = 0.f;
  constexpr int G = EP < 16 ? EP : 16;  // router rows loaded together
  u32x4 hv0 = {0u, 0u, 0u, 0u}, gv0 = {0u, 0u, 0u, 0u};  // this thread's first chunk
  for (int c = tid * 8; c < d; c += 256 * 8) {
    u32x4 wv[G];
#pragma unroll
    for (int e = 0; e < G; ++e) wv[e] = ldg16(wrow[e] + c);
    float h[8], g[8], x[8];
    const u32x4 hv = ldg16(hrow + c), gv = ldg16(gain + c);
    if (c == tid * 8) {
      hv0 = hv;
      gv0 = gv;
    }
    unpack8(hv, h);
    unpack8(gv, g);
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ss = fmaf(h[i], h[i], ss);
      x[i] = g[i] * h[i];
      mx = fmaxf(mx, fabsf(x[i]));
    }
    if (xs == nullptr) {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
      stg16(xrow + c, o);
    }
#pragma unroll
    for (int e0 = 0; e0 < EP; e0 += G) {
      if (e0 > 0) {
#pragma unroll
        for (int e = 0; e < G; ++e) wv[e] = ldg16(wrow[e0 + e] + c);
      }
#pragma unroll
      for (int e = 0; e < G; ++e) {
        float w[8];
        unpack8(wv[e], w);
        float s = acc[e0 + e];
#pragma unroll
        for (int i = 0; i < 8; ++i) s = fmaf(w[i], x[i], s);
        acc[e0 + e] = s;
      }
    }
  }
  WaveSpread<NV, 32>::run(acc, lane);
#pragma unroll
  for (int dlt = 32; dlt >= 1; dlt >>= 1) {
    ss += __shfl_xor(ss, dlt, kWave);
    mx = fmaxf(mx, __shfl_xor(mx, dlt, kWave));
  }
  if (spread_owner<NV>(lane)) {
#pragma unroll
    for (int i = 0; i < R; ++i) red[wave][spread_index<NV>(lane, i)] = acc[i];
  }
  if (lane == 0) {
    ssr[wave] = ss;
    mxr[wave] = mx;
  }
  __syncthreads();

  if (wave == 0) {
    // lane e < E owns expert e: logit, score, then the top-k and the gates by
    // wave-wide reductions (EP <= 64 experts, one per lane)
    const float sq = ((ssr[0] + ssr[1]) + ssr[2]) + ssr[3];
    const float inv = 1.0f / sqrtf(sq / (float)d + eps);
    const bool live = lane < E;
    const int el = lane < EP ? lane : 0;
    float z = live ? (((red[0][el] + red[1][el]) + red[2][el]) + red[3][el]) * inv : 0.f;
    if (eda != nullptr && live) {  // depth-averaged logits across the stack's MoE layers
      if (!eda_first) z = eda_alpha * eda_prev + (1.0f - eda_alpha) * z;
      eda[(size_t)t * 64 + lane] = z;
    }
    const float sc = z + bias_e;
    // top-k by descending score, exact ties to the lower index: each round
    // takes the wave maximum of a 64-bit key (available flag, the score's
    // order-preserving bits with NaN lowest, 63 - lane), unique per lane, so
    // exactly one lane wins every round and only experts < E can
    const uint32_t u = sc == 0.f ? 0u : __float_as_uint(sc);  // -0 ranks as +0
    const uint32_t ord = sc != sc ? 0u : (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    bool avail = live;
    int chosen = -1;  // this lane's rank j if chosen
    for (int j = 0; j < k; ++j) {
      uint64_t key = ((avail ? 1ull : 0ull) << 62) | ((uint64_t)ord << 6) | (uint64_t)(63 - lane);
#pragma unroll
      for (int dl = 1; dl < 64; dl <<= 1) {
        const uint64_t o = (uint64_t)__shfl_xor((unsigned long long)key, dl, kWave);
        key = o > key ? o : key;
      }
      if (lane == 63 - (int)(key & 63ull)) {
        chosen = j;
        avail = false;
      }
    }
    // gates: k = 1 softmax over all E logits at the chosen expert; k >= 2
    // softmax over the chosen logits
    const bool in_set = k == 1 ? live : chosen >= 0;
    float zm = in_set ? z : -INFINITY;
#pragma unroll
    for (int dl = 1; dl < 64; dl <<= 1) zm = fmaxf(zm, __shfl_xor(zm, dl, kWave));
    float ex = in_set ? expf(z - zm) : 0.f;
    float den = ex;
#pragma unroll
    for (int dl = 1; dl < 64; dl <<= 1) den += __shfl_xor(den, dl, kWave);
    if (chosen >= 0) {
      sel[(size_t)t * k + chosen] = lane;
      gate[(size_t)t * k + chosen] = ex / den;
    }
    if (lane == 0) inv_out[t] = inv;
    if (xs != nullptr && lane == 0) {
      const float m = fmaxf(fmaxf(mxr[0], mxr[1]), fmaxf(mxr[2], mxr[3]));
      const float a = bf16_lo(f32_to_bf16(inv * m)) / 448.f;
      xs[t] = a;
      s_inv = inv;
      s_r = e4m3_recip(a);
    }
  }
  if (xs != nullptr) {  // second pass: the E4M3 values of u = bf16(inv * x')
    __syncthreads();
    const float inv = s_inv, r = s_r;
    // the first chunk comes from registers (at d_model <= 2048 the whole row)
    for (int c = tid * 8; c < d; c += 256 * 8) {
      float h[8], g[8];
      const bool first = c == tid * 8;
      unpack8(first ? hv0 : ldg16(hrow + c), h);
      unpack8(first ? gv0 : ldg16(gain + c), g);
      uint32_t uw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        uw[i] = pack_bf16x2(inv * (g[2 * i] * h[2 * i]), inv * (g[2 * i + 1] * h[2 * i + 1]));
      const uint32_t c0 = quant4_e4m3(uw[0], uw[1], r), c1 = quant4_e4m3(uw[2], uw[3], r);
      u32x4 o;
      o[0] = e4m3_pair_to_bf16x2<false>(c0);
      o[1] = e4m3_pair_to_bf16x2<true>(c0);
      o[2] = e4m3_pair_to_bf16x2<false>(c1);
      o[3] = e4m3_pair_to_bf16x2<true>(c1);
      stg16(xrow + c, o);
    }
  }
}

namespace {
template <int EP>
hipError_t go(const FwdArgs& a) {
  return launch(k_router_token<EP>, dim3(a.T), dim3(256), a.stream, a.ev[kSlotNormRouter],
                (const uint16_t*)a.hidden, a.dim.d, (const uint16_t*)a.wr16,
                (const uint16_t*)a.gain16, (const float*)a.bias, a.dim.E, a.dim.k, a.dim.eps,
                (const uint16_t*)a.zrow, (uint16_t*)a.xn, a.inv, a.sel, a.gate, a.eda, a.eda_alpha,
                a.eda_first, a.dim.act8 ? a.xs_tok : nullptr);
}
}  // namespace

hipError_t launch_router_token(const FwdArgs& a) {
  switch (a.dim.EP) {
    case 1: return go<1>(a);
    case 2: return go<2>(a);
    case 4: return go<4>(a);
    case 8: return go<8>(a);
    case 16: return go<16>(a);
    case 32: return go<32>(a);
    case 64: return go<64>(a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
