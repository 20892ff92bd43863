// K2b (prefill shapes): gather of the routed token rows into expert-ordered
// MFMA operand tiles.
//
// The dispatch step (telknet.cc article, section 2.1: each token's row goes to
// the experts TopK chose for it) made explicit as a copy: slot p of expert e
// holds the normalised row x = bf16(inv_rms * (g * h)) of token gather[p]:
// RMSNorm is applied here, on the way from the hidden row to the tile (g * h
// is exact in fp32, times the router's inv_rms of the token, rounded once to
// fp32 and once to bf16), so the grouped GEMM's epilogue has no per-row
// scale.  Rows are stored in
// 32-slot subtiles, each expert's slots padded to a whole number of subtiles
// (the expert owning ceil(count / 32) subtiles from psub[e], the running sum
// of those numbers), and every subtile in the B-operand order of
// v_mfma_f32_32x32x16_bf16:
//   xt[P][s][lane][8],  lane = row + 32 * (k-group),  k = 16 s + 8 * (k-group) + 0..7
// so that the grouped GEMM reads its token operands as contiguous 1 KiB
// blocks, like its weights.  Padding rows are zero.
//
// One wave per (subtile, 64-wide k group): four wave-wide loads, each reading
// 8 rows x 128 contiguous bytes, and four non-temporal stores, each writing 8
// runs of 128 contiguous bytes.
//
// Layers with fp8 activations (Q8) store E4M3 codes instead: the router has
// left each token's quantisation scale a (its row's largest |x| / 448), so
// the row's codes RNE_E4M3(x * fl32(1 / a)) (quant4_e4m3) go straight into
// E4M3 operand tiles in the order of the layer's fp8 weight banks
// (block b of 32 k, lane l: row l % 32, bytes 0-7 k = 32 b + 8 (l / 32) + 0..7,
// bytes 8-15 the same + 16), with a in xs[slot] (0 for padding rows).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

template <bool Q8>
__global__ __launch_bounds__(256) void k_gather_tiles(const uint16_t* __restrict__ hidden,
                                                      const uint16_t* __restrict__ gain,
                                                      const float* __restrict__ inv,
                                                      const int* __restrict__ counts,
                                                      const int* __restrict__ gather, int E, int d,
                                                      uint16_t* __restrict__ xt,
                                                      const float* __restrict__ xs_tok,
                                                      uint8_t* __restrict__ xq,
                                                      float* __restrict__ xs) {
  const int groups = d / 64;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);  // wave of the grid
  const int P = gw / groups, g = gw - (gw / groups) * groups;
  // the subtile's expert: the experts' counts eight at a time (all eight
  // scalar loads in flight together), with running sums of their subtiles and
  // of their slots (the expert's first slot, so offsets is not read)
  int e = -1, base = 0, off = 0, cnt = 0;
  for (int e0 = 0; e0 < E && e < 0; e0 += 8) {
    int c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = counts[min(e0 + j, E - 1)];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (e < 0 && e0 + j < E) {
        const int ns = (c[j] + 31) >> 5;
        if (P < base + ns) {
          e = e0 + j;
          cnt = c[j];
        } else {
          base += ns;
          off += c[j];
        }
      }
    }
  }
  if (e < 0) return;  // past the last subtile (no barrier in this kernel)
  const int r0 = (P - base) * 32;
  const int lane = threadIdx.x & 63;
  uint16_t* dst = Q8 ? nullptr : xt + (size_t)P * (d / kKStep) * kBlockElems;
  u32x4 v[4];
  float s[4], qa[4];  // inv_rms and (Q8) the quantisation scale of each lane's row
  const u32x4 gv = ldg16(gain + g * 64 + (lane & 7) * 8);  // chunk c = lane & 7 in every q
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int idx = q * 64 + lane;
    const int rr = idx >> 3, c = idx & 7;  // row of the subtile, 16-byte chunk of the 128 bytes
    v[q] = u32x4{0u, 0u, 0u, 0u};
    s[q] = 0.f;
    qa[q] = 0.f;
    if (r0 + rr < cnt) {
      const int tok = gather[off + r0 + rr];
      v[q] = ldg16(hidden + (size_t)tok * d + g * 64 + c * 8);
      s[q] = inv[tok];
      if constexpr (Q8) qa[q] = xs_tok[tok];
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {  // x = bf16(inv * (g * h)); padding rows stay +0
    const bool ok = r0 + ((q * 64 + lane) >> 3) < cnt;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t x = pack_bf16x2(s[q] * (bf16_lo(gv[i]) * bf16_lo(v[q][i])),
                                     s[q] * (bf16_hi(gv[i]) * bf16_hi(v[q][i])));
      v[q][i] = ok ? x : 0u;
    }
  }
  if constexpr (Q8) {
    // chunk c of the group holds k = 64 g + 8 c .. +7: block 2g + c/4, lane
    // slot rr + 32 (c % 2), bytes 8 ((c / 2) % 2) ..; one store of the wave
    // fills two 128-byte runs of each of two blocks
    uint8_t* dq = xq + (size_t)P * (d / 32) * 1024;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = q * 64 + lane;
      const int rr = idx >> 3, c = idx & 7;
      const float r = e4m3_recip(qa[q]);
      u32x2 o;
      o[0] = quant4_e4m3(v[q][0], v[q][1], r);
      o[1] = quant4_e4m3(v[q][2], v[q][3], r);
      *reinterpret_cast<u32x2*>(dq + ((size_t)(2 * g + (c >> 2)) * 64 + rr + 32 * (c & 1)) * 16 +
                                8 * ((c >> 1) & 1)) = o;
      if (g == 0 && c == 0) xs[(size_t)P * 32 + rr] = qa[q];
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = q * 64 + lane;
      const int rr = idx >> 3, c = idx & 7;
      const int s = g * 4 + (c >> 1), li = (c & 1) * 32 + rr;
      stg16_stream(dst + ((size_t)s * 64 + li) * 8, v[q]);
    }
  }
}

// Subtiles of all experts for n assignments: at most floor((n + 31 E) / 32).
int max_subtiles(int n, int E) { return (n + 31 * E) / 32; }

hipError_t launch_gather_tiles(const FwdArgs& a) {
  const int waves = max_subtiles(a.n, a.dim.E) * (a.dim.d / 64);
  return launch(a.dim.act8 ? k_gather_tiles<true> : k_gather_tiles<false>, dim3((waves + 3) / 4),
                dim3(256), a.stream, a.ev[kSlotGather], (const uint16_t*)a.hidden,
                (const uint16_t*)a.gain16, (const float*)a.inv, (const int*)a.counts,
                (const int*)a.gather, a.dim.E, a.dim.d, (uint16_t*)a.xt,
                (const float*)a.xs_tok, (uint8_t*)a.xq, a.sx);
}

}  // namespace moe
