// K3 (decode shapes): grouped SwiGLU experts with the weights streamed from HBM
// straight into MFMA operands.
//
// Expert FFN y = W_down (SiLU(W_gate x) * (W_up x)) (SwiGLU, from the GLU
// variants paper on the ZONOS2 report's "Builds on" list; 16 such experts per
// MoE layer, digest item 5).  At decode sizes an expert sees a handful of
// tokens, so every weight element is used once per forward: the kernel is a
// weight stream.  The packed bank is laid out in MFMA operand order, so each
// wave-wide 16-byte-per-lane load reads 1 KiB of contiguous HBM; tokens (up to
// 32 per pass) fill the B operand of v_mfma_f32_32x32x16_bf16.  Experts that
// received no token exit before reading any weight.
//
// Each workgroup owns one 32-row weight tile of one expert; its four waves
// split the reduction axis into quarters and combine partial sums through LDS
// in a fixed order (deterministic).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {
constexpr int kSplit = 4;   // waves per weight tile (split of the reduction axis)
constexpr int kBatch = 8;   // k-steps whose loads are issued together

// Partial sums of waves 1..3 -> wave 0, fixed order.
template <int NACC>
__device__ __forceinline__ void reduce_split(f32x16 (&acc)[NACC], float* red, int wave, int lane) {
  if (wave > 0) {
#pragma unroll
    for (int q = 0; q < NACC; ++q)
#pragma unroll
      for (int i = 0; i < 16; ++i) red[(((wave - 1) * NACC + q) * 16 + i) * 64 + lane] = acc[q][i];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int w = 1; w < kSplit; ++w)
#pragma unroll
      for (int q = 0; q < NACC; ++q)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[q][i] += red[(((w - 1) * NACC + q) * 16 + i) * 64 + lane];
  }
  __syncthreads();
}
}  // namespace

// Gate/up projections and the SiLU(gate) * up epilogue for one 32-column F tile.
__global__ __launch_bounds__(256) void k_gateup_stream(const uint16_t* __restrict__ wgu,
                                                       const uint16_t* __restrict__ xn,
                                                       const int* __restrict__ counts,
                                                       const int* __restrict__ offsets,
                                                       const int* __restrict__ gather,
                                                       uint16_t* __restrict__ act, int d, int F) {
  __shared__ float red[(kSplit - 1) * 2 * 16 * 64];
  const int e = blockIdx.y;
  const int cnt = counts[e];
  if (cnt == 0) return;
  const int off = offsets[e];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ft = blockIdx.x;
  const int ksteps = d / kKStep;
  const int kper = ksteps / kSplit;
  const int ks0 = wave * kper;
  const size_t tile_elems = (size_t)ksteps * kBlockElems;
  const uint16_t* wg = wgu + (((size_t)e * (F / kTileRows) + ft) * 2) * tile_elems + lane * 8;
  const uint16_t* wu = wg + tile_elems;
  const int col = lane & 31;

  for (int c0 = 0; c0 < cnt; c0 += 32) {
    const int ntok = min(32, cnt - c0);
    const bool valid = col < ntok;
    const uint16_t* xrow = xn + (size_t)(valid ? gather[off + c0 + col] : 0) * d + (lane >> 5) * 8;
    f32x16 acc[2];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[q][i] = 0.f;

    int s = ks0;
    for (; s + kBatch <= ks0 + kper; s += kBatch) {
      u32x4 ag[kBatch], au[kBatch], b[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        ag[u] = ldg16_stream(wg + (size_t)(s + u) * kBlockElems);
        au[u] = ldg16_stream(wu + (size_t)(s + u) * kBlockElems);
        b[u] = valid ? ldg16(xrow + (s + u) * kKStep) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        acc[0] = mfma_32x32x16(ag[u], b[u], acc[0]);
        acc[1] = mfma_32x32x16(au[u], b[u], acc[1]);
      }
    }
    for (; s < ks0 + kper; ++s) {
      const u32x4 ag = ldg16_stream(wg + (size_t)s * kBlockElems);
      const u32x4 au = ldg16_stream(wu + (size_t)s * kBlockElems);
      const u32x4 b = valid ? ldg16(xrow + s * kKStep) : u32x4{0, 0, 0, 0};
      acc[0] = mfma_32x32x16(ag, b, acc[0]);
      acc[1] = mfma_32x32x16(au, b, acc[1]);
    }
    reduce_split<2>(acc, red, wave, lane);

    if (wave == 0 && valid) {
      uint16_t* dst = act + (size_t)(off + c0 + col) * F + ft * kTileRows;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r = c32_row(4 * g, lane);
        u32x2 v;
        v[0] = pack_bf16x2(silu(acc[0][4 * g]) * acc[1][4 * g],
                           silu(acc[0][4 * g + 1]) * acc[1][4 * g + 1]);
        v[1] = pack_bf16x2(silu(acc[0][4 * g + 2]) * acc[1][4 * g + 2],
                           silu(acc[0][4 * g + 3]) * acc[1][4 * g + 3]);
        *reinterpret_cast<u32x2*>(dst + r) = v;
      }
    }
  }
}

// Down projection for one 32-row d_model tile; k = 1 writes gate * y into the
// output row of the token, k > 1 writes y (fp32) for the combine kernel.
__global__ __launch_bounds__(256) void k_down_stream(
    const uint16_t* __restrict__ wd, const uint16_t* __restrict__ act,
    const int* __restrict__ counts, const int* __restrict__ offsets,
    const int* __restrict__ gather, const float* __restrict__ gate, int k,
    uint16_t* __restrict__ out, float* __restrict__ ybuf, int d, int F) {
  __shared__ float red[(kSplit - 1) * 16 * 64];
  const int e = blockIdx.y;
  const int cnt = counts[e];
  if (cnt == 0) return;
  const int off = offsets[e];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int mt = blockIdx.x;
  const int ksteps = F / kKStep;
  const int kper = ksteps / kSplit;
  const int ks0 = wave * kper;
  const uint16_t* wrow =
      wd + ((size_t)e * (d / kTileRows) + mt) * (size_t)ksteps * kBlockElems + lane * 8;
  const int col = lane & 31;

  for (int c0 = 0; c0 < cnt; c0 += 32) {
    const int ntok = min(32, cnt - c0);
    const bool valid = col < ntok;
    const int slot = off + c0 + (valid ? col : 0);
    const uint16_t* arow = act + (size_t)slot * F + (lane >> 5) * 8;
    f32x16 acc[1];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[0][i] = 0.f;

    int s = ks0;
    for (; s + kBatch <= ks0 + kper; s += kBatch) {
      u32x4 aw[kBatch], b[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        aw[u] = ldg16_stream(wrow + (size_t)(s + u) * kBlockElems);
        b[u] = valid ? ldg16(arow + (s + u) * kKStep) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) acc[0] = mfma_32x32x16(aw[u], b[u], acc[0]);
    }
    for (; s < ks0 + kper; ++s) {
      const u32x4 aw = ldg16_stream(wrow + (size_t)s * kBlockElems);
      const u32x4 b = valid ? ldg16(arow + s * kKStep) : u32x4{0, 0, 0, 0};
      acc[0] = mfma_32x32x16(aw, b, acc[0]);
    }
    reduce_split<1>(acc, red, wave, lane);

    if (wave == 0 && valid) {
      const int m0 = mt * kTileRows;
      if (k == 1) {
        const int tok = gather[slot];
        const float g = gate[tok];
        uint16_t* dst = out + (size_t)tok * d + m0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = c32_row(4 * q, lane);
          u32x2 v;
          v[0] = pack_bf16x2(g * acc[0][4 * q], g * acc[0][4 * q + 1]);
          v[1] = pack_bf16x2(g * acc[0][4 * q + 2], g * acc[0][4 * q + 3]);
          *reinterpret_cast<u32x2*>(dst + r) = v;
        }
      } else {
        float* dst = ybuf + (size_t)slot * d + m0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = c32_row(4 * q, lane);
          f32x4 v = {acc[0][4 * q], acc[0][4 * q + 1], acc[0][4 * q + 2], acc[0][4 * q + 3]};
          *reinterpret_cast<f32x4*>(dst + r) = v;
        }
      }
    }
  }
}

hipError_t launch_experts_stream(const FwdArgs& a) {
  const int d = a.dim.d, F = a.dim.F, E = a.dim.E;
  hipLaunchKernelGGL(k_gateup_stream, dim3(F / kTileRows, E), dim3(256), 0, a.stream,
                     (const uint16_t*)a.wgu, (const uint16_t*)a.xn, a.counts, a.offsets, a.gather,
                     (uint16_t*)a.act, d, F);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (a.ev_mid != nullptr && (err = hipEventRecord(a.ev_mid, a.stream)) != hipSuccess) return err;
  hipLaunchKernelGGL(k_down_stream, dim3(d / kTileRows, E), dim3(256), 0, a.stream,
                     (const uint16_t*)a.wd, (const uint16_t*)a.act, a.counts, a.offsets, a.gather,
                     a.gate, a.dim.k, (uint16_t*)a.out, a.ybuf, d, F);
  return hipGetLastError();
}

}  // namespace moe
