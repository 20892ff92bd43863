// K1 (bf16 layers, prefill-sized batches): fused RMSNorm statistics + linear
// router on bf16 MFMA + bias-steered top-k + gates.
//
// ZONOS2 Technical Report (audio-paper-digest page, "Method overview and
// architecture"): item 5 normalises the backbone input with RMSNorm and routes
// each token to 1 of 16 experts (2 in the last MoE layer); item 6 keeps a
// per-expert bias b_l for load balancing, which here only moves the choice
// (s = z + b) while gates come from the unbiased logits z.
//
// Exact router on bf16 matrix cores: with x' = g * h (the gain times the bf16
// input) every product is exact in fp32 because both factors are bf16, and
// x' carries at most 16 significant bits, so x' = hi + lo with hi = bf16(x')
// and lo = bf16(x' - hi) both exact.  z_raw = W_r x' = W_r hi + W_r lo is
// therefore two bf16 MFMAs with fp32 accumulation: fp32-router precision at
// matrix-core speed.  z = inv_rms * z_raw with inv_rms = 1/sqrt(mean(h^2)+eps).
//
// Outputs: inv_rms[T], sel[T,k], gate[T,k]; with fp8 activations also each
// token's quantisation scale xs[T] = max_i |bf16(inv_rms * x'_i)| / 448, which
// is bf16(inv_rms * max_i |x'_i|) / 448 because both roundings are monotone,
// so the gather can write E4M3 rows in one pass.  In a stack that depth-averages
// the router state (the digest's item 5 names exponential depth averaging
// after ZAYA1 without defining it; read as z~ = alpha * z~_prev + (1 - alpha)
// * z on the logits), eda holds each token's averaged logits of the previous
// MoE layer, which selection and gates then use in place of z.  The normalised expert inputs
// are formed by the gather kernel from the hidden rows it copies (with this
// kernel's inv_rms), which saves writing and re-reading T*d*2 bytes here.
//
// The kernel reads T*d*2 bytes, so it is sized for memory-level
// parallelism: a workgroup owns 16*TT tokens (TT = 1; MFMA 16x16x32:
// A = 16 router rows per tile, NA tiles; B = 16 tokens per tile, TT tiles),
// its NW waves split the reduction axis into NW slices, and each wave issues
// the loads of up to kRBatch k-steps at once.  One wave-wide token load reads
// 64 contiguous bytes from each of 16 rows.  Partial logits of the waves meet
// in LDS and are summed in a fixed order, one (token, expert) pair per thread;
// with 16 experts the top-k and gates run on 16 lanes per token.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {
constexpr int kRK = 32;     // k per MFMA 16x16x32 step
constexpr int kRBatch = 8;  // k-steps whose loads are issued together

// D = A * B + C on a 16x16 tile with K = 32, bf16 inputs, fp32 accumulation.
// Operands: lane l carries row (l % 16) of A (column (l % 16) of B) and 8
// consecutive k of k-group (l / 16).  Output: lane l holds column (l % 16),
// rows 4*(l/16) + i for accumulator element i.
__device__ __forceinline__ f32x4 mfma_16x16x32(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
}  // namespace

template <int NA, int TT, int NW>
__global__ __launch_bounds__(NW * 64) void k_router_mfma(
    const uint16_t* __restrict__ hidden, int T, int d, const uint16_t* __restrict__ wr,
    const uint16_t* __restrict__ gain, const float* __restrict__ bias, int E, int k, float eps,
    const uint16_t* __restrict__ zrow, float* __restrict__ inv_out, int* __restrict__ sel,
    float* __restrict__ gate, float* __restrict__ eda, float eda_alpha, int eda_first,
    float* __restrict__ xs_out) {
  constexpr int NTOK = 16 * TT;
  constexpr int EPAD = 16 * NA;
  static_assert(EPAD != 16 || NTOK != 16 || NW * 64 >= 16 * NTOK,
                "the 16-expert finish takes 16 lanes per token");
  __shared__ float red[NW][TT][NA][4][64];
  __shared__ float ssr[NW][TT][64];
  __shared__ float mxr[NW][TT][64];
  __shared__ float zs[NTOK][EPAD + 1];
  // each wave's gain for its current batch of k-steps (kRBatch x 4 k-groups of
  // 8 values): loaded once per batch and read back by the 16 lanes sharing a
  // k-group, instead of one copy per lane from memory
  __shared__ u32x4 gsh[NW][kRBatch * 4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * NTOK;
  const int kgrp = (lane >> 4) * 8;
  const int kper = d / (kRK * NW);  // k-steps per wave
  const int k0 = wave * kper * kRK;

  const uint16_t* ap[NA];
#pragma unroll
  for (int a = 0; a < NA; ++a) {
    const int e = a * 16 + (lane & 15);
    ap[a] = (e < E ? wr + (size_t)e * d : zrow) + kgrp + k0;
  }
  const uint16_t* hp[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    const int t = t0 + tt * 16 + (lane & 15);
    hp[tt] = (t < T ? hidden + (size_t)t * d : zrow) + kgrp + k0;
  }
  const uint16_t* gp = gain + kgrp + k0;

  // the 16-expert finish (16 lanes per token, lane e % 16 owns expert e):
  // its bias and (depth averaging) the previous MoE layer's logit are loaded
  // now, under the main loop's loads
  float bias_e = 0.f, eda_prev = 0.f;
  if (EPAD == 16 && NTOK == 16 && tid < 16 * NTOK) {
    const int e = tid & 15, t = t0 + (tid >> 4);
    bias_e = bias[e];  // bias is padded with zeros to 64 entries
    if (eda != nullptr && !eda_first && e < E && t < T) eda_prev = eda[(size_t)t * 64 + e];
  }

  f32x4 acc[TT][NA];
  float ss[TT], mx[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    ss[tt] = 0.f;
    mx[tt] = 0.f;
#pragma unroll
    for (int a = 0; a < NA; ++a) acc[tt][a] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // one k-step: x' = g*h split into exact bf16 hi + lo, two MFMAs per tile pair
  auto step = [&](const u32x4& gv, const u32x4 (&av)[NA], const u32x4 (&hv)[TT]) {
    float g[8];
    unpack8(gv, g);
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      float h[8];
      unpack8(hv[tt], h);
      u32x4 bhi, blo;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x0 = g[2 * i] * h[2 * i], x1 = g[2 * i + 1] * h[2 * i + 1];
        ss[tt] = fmaf(h[2 * i], h[2 * i], ss[tt]);
        ss[tt] = fmaf(h[2 * i + 1], h[2 * i + 1], ss[tt]);
        mx[tt] = fmaxf(mx[tt], fmaxf(fabsf(x0), fabsf(x1)));
        const uint32_t hi = pack_bf16x2(x0, x1);
        bhi[i] = hi;
        blo[i] = pack_bf16x2(x0 - bf16_lo(hi), x1 - bf16_hi(hi));
      }
#pragma unroll
      for (int a = 0; a < NA; ++a) {
        acc[tt][a] = mfma_16x16x32(av[a], bhi, acc[tt][a]);
        acc[tt][a] = mfma_16x16x32(av[a], blo, acc[tt][a]);
      }
    }
  };

  int s = 0;
  const uint16_t* gw = gain + k0 + lane * 8;  // lanes 0 .. 4 kRBatch - 1: a batch's gain
  for (; s + kRBatch <= kper; s += kRBatch) {
    u32x4 av[kRBatch][NA], hv[kRBatch][TT];
    u32x4 gb = {0u, 0u, 0u, 0u};
    if (lane < kRBatch * 4) gb = ldg16(gw + s * kRK);
#pragma unroll
    for (int b = 0; b < kRBatch; ++b) {
      const int ko = (s + b) * kRK;
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) hv[b][tt] = ldg16(hp[tt] + ko);
#pragma unroll
      for (int a = 0; a < NA; ++a) av[b][a] = ldg16(ap[a] + ko);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the whole batch of loads in flight together
    if (lane < kRBatch * 4) gsh[wave][lane] = gb;  // one wave's LDS operations run in order
#pragma unroll
    for (int b = 0; b < kRBatch; ++b) step(gsh[wave][b * 4 + (lane >> 4)], av[b], hv[b]);
  }
  for (; s < kper; ++s) {
    const int ko = s * kRK;
    u32x4 av[NA], hv[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) hv[tt] = ldg16(hp[tt] + ko);
#pragma unroll
    for (int a = 0; a < NA; ++a) av[a] = ldg16(ap[a] + ko);
    step(ldg16(gp + ko), av, hv);
  }

#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    ssr[wave][tt][lane] = ss[tt];
    mxr[wave][tt][lane] = mx[tt];
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][tt][a][i][lane] = acc[tt][a][i];
  }
  __syncthreads();

  // cross-wave sums in a fixed order, one (token, expert) pair per thread:
  // C[row r][column c] of a 16x16 tile sits in lane c + 16*(r/4), element r%4.
  for (int p = tid; p < NTOK * EPAD; p += NW * 64) {
    const int t = p % NTOK, e = p / NTOK;
    const int tt = t >> 4, c = t & 15, a = e >> 4, r = e & 15;
    const int l = c + 16 * (r >> 2), i = r & 3;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) v += red[w][tt][a][i][l];
    zs[t][e] = v;
  }
  __syncthreads();

  if constexpr (EPAD == 16 && NTOK == 16) {
    // 16 experts: 16 lanes per token (lane e owns expert e), top-k as k maxima
    // of a unique key over the lane group (availability, the score's
    // order-preserving bits with NaN lowest, 63 - e): the same choice as the
    // one-thread loop below, ties to the lower index, one winner per round
    if (tid < 16 * NTOK) {
      const int tl = tid >> 4, e = tid & 15;
      const int t = t0 + tl;
      float sq = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w)
        sq += (ssr[w][0][tl] + ssr[w][0][tl + 16]) + (ssr[w][0][tl + 32] + ssr[w][0][tl + 48]);
      const float inv = 1.0f / sqrtf(sq / (float)d + eps);
      const bool live = e < E;
      float z = zs[tl][e] * inv;
      if (eda != nullptr && live && t < T) {  // depth-averaged logits across MoE layers
        if (!eda_first) z = eda_alpha * eda_prev + (1.0f - eda_alpha) * z;
        eda[(size_t)t * 64 + e] = z;
      }
      const float sc = z + bias_e;
      const uint32_t u = sc == 0.f ? 0u : __float_as_uint(sc);  // -0 ranks as +0
      const uint32_t ord = sc != sc ? 0u : (u & 0x80000000u) ? ~u : (u | 0x80000000u);
      bool avail = live;
      int chosen = -1;
      for (int j = 0; j < k; ++j) {
        uint64_t key = ((avail ? 1ull : 0ull) << 62) | ((uint64_t)ord << 6) | (uint64_t)(63 - e);
#pragma unroll
        for (int dl = 1; dl < 16; dl <<= 1) {
          const uint64_t o = (uint64_t)__shfl_xor((unsigned long long)key, dl, 16);
          key = o > key ? o : key;
        }
        if (e == 63 - (int)(key & 63ull)) {
          chosen = j;
          avail = false;
        }
      }
      const bool in_set = k == 1 ? live : chosen >= 0;
      float zm = in_set ? z : -INFINITY;
#pragma unroll
      for (int dl = 1; dl < 16; dl <<= 1) zm = fmaxf(zm, __shfl_xor(zm, dl, 16));
      const float ex = in_set ? expf(z - zm) : 0.f;
      float den = ex;
#pragma unroll
      for (int dl = 1; dl < 16; dl <<= 1) den += __shfl_xor(den, dl, 16);
      if (t < T) {
        if (chosen >= 0) {
          sel[(size_t)t * k + chosen] = e;
          gate[(size_t)t * k + chosen] = ex / den;
        }
        if (e == 0) inv_out[t] = inv;
        if (e == 1 && xs_out != nullptr) {
          float m = 0.f;
#pragma unroll
          for (int w = 0; w < NW; ++w)
            m = fmaxf(m, fmaxf(fmaxf(mxr[w][0][tl], mxr[w][0][tl + 16]),
                               fmaxf(mxr[w][0][tl + 32], mxr[w][0][tl + 48])));
          xs_out[t] = bf16_lo(f32_to_bf16(inv * m)) / 448.f;
        }
      }
    }
  } else if (tid < NTOK) {
    const int tt = tid >> 4, c = tid & 15;
    const int t = t0 + tid;
    float sq = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w)
      sq += (ssr[w][tt][c] + ssr[w][tt][c + 16]) + (ssr[w][tt][c + 32] + ssr[w][tt][c + 48]);
    const float inv = 1.0f / sqrtf(sq / (float)d + eps);
    float z[EPAD], sc[EPAD];
#pragma unroll
    for (int e = 0; e < EPAD; ++e) {
      z[e] = zs[tid][e] * inv;
      if (eda != nullptr && e < E && t < T) {  // depth-averaged logits across MoE layers
        float* st = eda + (size_t)t * 64 + e;
        if (!eda_first) z[e] = eda_alpha * *st + (1.0f - eda_alpha) * z[e];
        *st = z[e];
      }
      sc[e] = z[e] + bias[e];  // bias is padded with zeros to 64 entries
    }
    if (t < T) {
      // top-k by descending score, exact ties to the lower index; NaN never wins
      uint64_t taken = 0;
      int chosen[8];
      float zc[8];
      for (int j = 0; j < k; ++j) {
        int best = -1;
        float bs = 0.f, bz = 0.f;
#pragma unroll
        for (int e = 0; e < EPAD; ++e) {
          const bool ok = e < E && !((taken >> e) & 1) && (best < 0 || sc[e] > bs);
          best = ok ? e : best;
          bs = ok ? sc[e] : bs;
          bz = ok ? z[e] : bz;
        }
        chosen[j] = best;
        zc[j] = bz;
        taken |= 1ull << best;
      }
      float zmax = -INFINITY, den = 0.f;
      if (k == 1) {
#pragma unroll
        for (int e = 0; e < EPAD; ++e) zmax = e < E ? fmaxf(zmax, z[e]) : zmax;
#pragma unroll
        for (int e = 0; e < EPAD; ++e) den += e < E ? expf(z[e] - zmax) : 0.f;
      } else {
        for (int j = 0; j < k; ++j) zmax = fmaxf(zmax, zc[j]);
        for (int j = 0; j < k; ++j) den += expf(zc[j] - zmax);
      }
      for (int j = 0; j < k; ++j) {
        sel[(size_t)t * k + j] = chosen[j];
        gate[(size_t)t * k + j] = expf(zc[j] - zmax) / den;
      }
      inv_out[t] = inv;
      if (xs_out != nullptr) {
        float m = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w)
          m = fmaxf(m, fmaxf(fmaxf(mxr[w][tt][c], mxr[w][tt][c + 16]),
                             fmaxf(mxr[w][tt][c + 32], mxr[w][tt][c + 48])));
        xs_out[t] = bf16_lo(f32_to_bf16(inv * m)) / 448.f;
      }
    }
  }
}

namespace {
// Four waves, one per SIMD, each owning a quarter of d_model: at 16384 tokens
// eight waves (each with one batch of loads) took 28.3 us and four 22.6 us,
// the same at 4096 tokens.
template <int NA, int TT>
hipError_t go(const FwdArgs& a) {
  constexpr int NW = 4;
  if (a.dim.d % (kRK * NW) != 0) return hipErrorInvalidValue;
  const int grid = (a.T + 16 * TT - 1) / (16 * TT);
  return launch(k_router_mfma<NA, TT, NW>, dim3(grid), dim3(NW * 64), a.stream,
                a.ev[kSlotNormRouter], (const uint16_t*)a.hidden, a.T, a.dim.d,
                (const uint16_t*)a.wr16, (const uint16_t*)a.gain16, (const float*)a.bias, a.dim.E,
                a.dim.k, a.dim.eps, (const uint16_t*)a.zrow, a.inv, a.sel, a.gate, a.eda,
                a.eda_alpha, a.eda_first, a.dim.act8 ? a.xs_tok : nullptr);
}
}  // namespace

// One 16-token tile per workgroup: at 16384 tokens two tiles per workgroup
// (half the workgroups, each reading the router rows once for 32 tokens)
// measured 6% slower, and again with the gain staged in LDS: 25.0 against
// 21.8 us.
hipError_t launch_router_mfma(const FwdArgs& a) {
  const int E = a.dim.E;
  return E > 32 ? go<4, 1>(a) : E > 16 ? go<2, 1>(a) : go<1, 1>(a);
}

}  // namespace moe
