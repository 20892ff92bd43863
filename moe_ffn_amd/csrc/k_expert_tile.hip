// K3 (prefill shapes): grouped SwiGLU GEMMs over the experts, LDS-staged tiles.
//
// Expert FFN y = W_down (SiLU(W_gate x) * (W_up x)) per routed assignment
// (SwiGLU: GLU variants paper on the ZONOS2 report's "Builds on" list; 16
// experts per layer, digest item 5).  Two launches:
//   MODE 0  act[slot, f] = bf16( SiLU(x W_gate^T) * (x W_up^T) )   K = d_model
//   MODE 1  y[slot, m]   = act[slot] W_down^T                       K = d_ff
//           k = 1: out[token] = bf16(gate * y); k > 1: y kept in fp32.
// A workgroup computes a 256-weight-row x 128-token tile (32 weight rows of an
// MFMA tile per row of a wave's grid, 2x2 waves, each 128 rows x 64 tokens)
// over k-tiles of 64.  Weights come from the packed bank (MFMA operand order,
// 1 KiB blocks) and tokens are gathered on load from the expert-ordered slot
// list, so no permuted copy of the activations is made.  The next k-tile is
// fetched into registers while the current one is multiplied from LDS (two
// LDS buffers, one barrier per k-tile).  Token tiles come from the tile map:
// (expert, 128-slot block) entries, one per block, unused grid rows exit.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {
constexpr int kWRowTiles = 8;                 // 8 x 32 = 256 weight rows per workgroup
constexpr int kTokTiles = kTileTokens / 32;   // 4 x 32 = 128 tokens
constexpr int kKT = 64;                       // k per LDS stage
constexpr int kSteps = kKT / kKStep;          // 4 MFMA k-steps per stage
constexpr int kWChunks = kWRowTiles * kSteps * 64;  // 16-byte chunks of a weight stage (2048)
constexpr int kXChunks = kTokTiles * kSteps * 64;   // 16-byte chunks of a token stage (1024)
}  // namespace

template <int MODE>
__global__ __launch_bounds__(256) void k_expert_tile(
    const uint16_t* __restrict__ wpk, const uint16_t* __restrict__ src,
    const int* __restrict__ tilemap, const int* __restrict__ counts,
    const int* __restrict__ offsets, const int* __restrict__ gather,
    const float* __restrict__ gate, const float* __restrict__ inv, int k,
    uint16_t* __restrict__ dst16,
    float* __restrict__ ybuf, int d, int F) {
  __shared__ u32x4 lds_w[2][kWChunks];
  __shared__ u32x4 lds_x[2][kXChunks];

  const int ntiles = tilemap[0];
  if ((int)blockIdx.x >= ntiles) return;
  const int ent = tilemap[1 + blockIdx.x];
  const int e = ent >> 16, mtile = ent & 0xffff;
  const int cnt = counts[e], off = offsets[e];
  const int row0 = mtile * kTileTokens;          // first expert-local slot of the tile
  const int nvalid = min(kTileTokens, cnt - row0);
  const int K = MODE == 0 ? d : F;
  const int ksteps = K / kKStep;
  const int nkt = K / kKT;
  const size_t tile_elems = (size_t)ksteps * kBlockElems;
  const int wb = blockIdx.y;
  // The workgroup's 8 packed row tiles are consecutive in the bank.
  const uint16_t* wbase =
      wpk + (MODE == 0 ? ((size_t)e * (F / kTileRows) + (size_t)wb * 4) * 2
                       : (size_t)e * (d / kTileRows) + (size_t)wb * kWRowTiles) *
                tile_elems;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wt = wave & 1;

  // per-thread token-row sources (fixed over k)
  const uint16_t* xptr[kXChunks / 256];
  int xdst[kXChunks / 256];
  bool xval[kXChunks / 256];
#pragma unroll
  for (int j = 0; j < kXChunks / 256; ++j) {
    const int idx = tid + 256 * j;
    const int r = idx >> 3, kc = idx & 7;
    xval[j] = r < nvalid;
    const int slot = off + row0 + (xval[j] ? r : 0);
    const int row = MODE == 0 ? gather[slot] : slot;
    xptr[j] = src + (size_t)row * K + kc * 8;
    xdst[j] = ((r >> 5) * kSteps + (kc >> 1)) * 64 + (kc & 1) * 32 + (r & 31);
  }

  u32x4 pw[kWChunks / 256], px[kXChunks / 256];
  auto fetch = [&](int kt) {
#pragma unroll
    for (int j = 0; j < kWChunks / 256; ++j) {
      const int idx = tid + 256 * j;
      const int rt = idx >> 8, w = idx & 255;
      pw[j] = ldg16(wbase + rt * tile_elems + (size_t)kt * (kSteps * kBlockElems) + w * 8);
    }
#pragma unroll
    for (int j = 0; j < kXChunks / 256; ++j)
      px[j] = xval[j] ? ldg16(xptr[j] + kt * kKT) : u32x4{0, 0, 0, 0};
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int j = 0; j < kWChunks / 256; ++j) lds_w[buf][tid + 256 * j] = pw[j];
#pragma unroll
    for (int j = 0; j < kXChunks / 256; ++j) lds_x[buf][xdst[j]] = px[j];
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  fetch(0);
  stash(0);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nkt) fetch(kt + 1);
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      u32x4 av[4], bv[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = lds_w[buf][((wr * 4 + i) * kSteps + s) * 64 + lane];
#pragma unroll
      for (int j = 0; j < 2; ++j) bv[j] = lds_x[buf][((wt * 2 + j) * kSteps + s) * 64 + lane];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma_32x32x16(av[i], bv[j], acc[i][j]);
    }
    if (kt + 1 < nkt) stash(buf ^ 1);
    __syncthreads();
  }

  // epilogue
  const int col = lane & 31;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = (wt * 2 + j) * 32 + col;  // tile-local token row
    if (r >= nvalid) continue;
    const int slot = off + row0 + r;
    if constexpr (MODE == 0) {
      const float sc = inv[gather[slot]];  // RMSNorm scale of this token
      uint16_t* dst = dst16 + (size_t)slot * F;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        // row tiles (2p, 2p+1) of this wave are the gate and up halves of one F tile
        const int ft = wb * 4 + wr * 2 + p;
        const f32x16& g = acc[2 * p][j];
        const f32x16& u = acc[2 * p + 1][j];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int f = ft * kTileRows + c32_row(4 * q, lane);
          float v4[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) v4[c] = silu(sc * g[4 * q + c]) * (sc * u[4 * q + c]);
          u32x2 v;
          v[0] = pack_bf16x2(v4[0], v4[1]);
          v[1] = pack_bf16x2(v4[2], v4[3]);
          *reinterpret_cast<u32x2*>(dst + f) = v;
        }
      }
    } else {
      const int tok = k == 1 ? gather[slot] : 0;
      const float gw = k == 1 ? gate[tok] : 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int mbase = (wb * kWRowTiles + wr * 4 + i) * kTileRows;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int m = mbase + c32_row(4 * q, lane);
          if (k == 1) {
            u32x2 v;
            v[0] = pack_bf16x2(gw * acc[i][j][4 * q], gw * acc[i][j][4 * q + 1]);
            v[1] = pack_bf16x2(gw * acc[i][j][4 * q + 2], gw * acc[i][j][4 * q + 3]);
            *reinterpret_cast<u32x2*>(dst16 + (size_t)tok * d + m) = v;
          } else {
            f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                       acc[i][j][4 * q + 3]};
            *reinterpret_cast<f32x4*>(ybuf + (size_t)slot * d + m) = v;
          }
        }
      }
    }
  }
}

hipError_t launch_experts_tile(const FwdArgs& a) {
  const int d = a.dim.d, F = a.dim.F;
  hipError_t err = launch(k_expert_tile<0>, dim3(a.max_tiles, F / 128), dim3(256), a.stream,
                          a.ev[kSlotExpertsA], (const uint16_t*)a.wgu, (const uint16_t*)a.xn,
                          (const int*)a.tilemap, (const int*)a.counts, (const int*)a.offsets,
                          (const int*)a.gather, (const float*)a.gate, (const float*)a.inv,
                          a.dim.k, (uint16_t*)a.act, a.ybuf, d, F);
  if (err != hipSuccess) return err;
  return launch(k_expert_tile<1>, dim3(a.max_tiles, d / 256), dim3(256), a.stream,
                a.ev[kSlotExpertsB], (const uint16_t*)a.wd, (const uint16_t*)a.act,
                (const int*)a.tilemap, (const int*)a.counts, (const int*)a.offsets,
                (const int*)a.gather, (const float*)a.gate, (const float*)a.inv, a.dim.k,
                (uint16_t*)a.out, a.ybuf, d, F);
}

}  // namespace moe
