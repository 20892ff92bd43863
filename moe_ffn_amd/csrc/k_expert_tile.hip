// K3 (prefill shapes): grouped SwiGLU GEMMs over the experts, LDS-staged tiles.
//
// Expert FFN y = W_down (SiLU(W_gate x) * (W_up x)) per routed assignment
// (SwiGLU: GLU variants paper on the ZONOS2 report's "Builds on" list; 16
// experts per layer, digest item 5).  Two launches:
//   MODE 0  act[slot, f] = bf16( SiLU(x W_gate^T) * (x W_up^T) )   K = d_model
//   MODE 1  y[slot, m]   = act[slot] W_down^T                       K = d_ff
//           k = 1: out[token] = bf16(gate * y); k > 1: y kept in fp32.
// A workgroup computes a 256-weight-row x 128-token tile: four waves stacked
// along the weight rows, each owning two 32-row MFMA tiles against all four
// 32-token tiles (8 accumulators of 32x32).  Weights are read straight from
// the packed bank (MFMA operand order, 1 KiB per wave-wide load) into
// registers, four k-steps ahead, so they never pass through LDS.  Only the
// token tile is shared: rows gathered on load through the expert-ordered slot
// list (8 rows x 128 contiguous bytes per wave-wide load) are written to LDS in
// operand order (conflict-free 1 KiB reads), three 64-wide k-tiles in flight
// (two in registers, one in LDS) and one barrier per k-tile.  Two workgroups
// per CU, so one's barrier and load waits overlap the other's MFMAs.  Partial
// token tiles (the tail of each expert) run a variant that skips the empty
// 32-token tiles.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {
constexpr int kTT = kTileTokens / 32;      // 32-token MFMA tiles per workgroup (4)
constexpr int kWaves = 4;                  // waves per workgroup, stacked along weight rows
constexpr int kWR = 2;                     // 32-row weight tiles per wave
constexpr int kRowsWG = kWaves * kWR * 32; // 256 weight rows per workgroup
constexpr int kPre = 4;                    // k-steps of weight loads in flight per wave
constexpr int kKT = 64;                    // k per LDS stage of the token tile
constexpr int kBlk = kTT * (kKT / kKStep); // 1 KiB operand blocks per token stage (16)
constexpr int kBW = kBlk / kWaves;         // blocks staged by each wave per stage
constexpr int kTPW = kTT / kWaves;         // token tiles staged by each wave

struct TileCtx {
  const uint16_t* wa;     // this wave's first weight tile (lane offset applied)
  size_t tile_elems;      // elements of one packed 32-row tile
  int ksteps;             // K / 16
  const uint16_t* brow[kBW];  // this thread's source for each staged chunk (k offset applied)
  int bdst;                   // LDS index (16-byte units) of chunk 0; chunk j adds j * kBlk*64/kBW
  int wave, lane;
};

__device__ __forceinline__ void load_a(const TileCtx& c, int s, u32x4 (&q)[kWR]) {
  const int sc = s < c.ksteps ? s : c.ksteps - 1;  // clamp: surplus loads stay in bounds
#pragma unroll
  for (int r = 0; r < kWR; ++r) q[r] = ldg16(c.wa + r * c.tile_elems + (size_t)sc * kBlockElems);
}

// Token staging: the workgroup's 256 threads copy a kTileTokens x 64 slice of
// gathered rows per k-tile, each wave-wide load reading 8 rows x 128 contiguous
// bytes (8 full cache lines): thread t, chunk j covers row r = (j*256 + t) / 8
// and 16-byte k-chunk kc = t % 8.  The LDS write scatters each chunk to its
// place in MFMA operand order: block (r/32)*4 + kc/2, lane (kc%2)*32 + r%32.
__device__ __forceinline__ void load_b(const TileCtx& c, int kt, int nkt, u32x4 (&p)[kBW]) {
  const int kc = kt < nkt ? kt : nkt - 1;
#pragma unroll
  for (int j = 0; j < kBW; ++j) p[j] = ldg16(c.brow[j] + kc * kKT);
}
__device__ __forceinline__ void store_b(u32x4* buf, const TileCtx& c, const u32x4 (&p)[kBW]) {
#pragma unroll
  for (int j = 0; j < kBW; ++j) buf[c.bdst + j * (kBlk * 64 / kBW)] = p[j];
}

template <int NT>
__device__ __forceinline__ void read_b(const u32x4* buf, int s16, int lane, u32x4 (&bv)[NT]) {
#pragma unroll
  for (int j = 0; j < NT; ++j) bv[j] = buf[(j * 4 + s16) * 64 + lane];
}

template <int NT>
__device__ __forceinline__ void mac(const u32x4 (&a)[kWR], const u32x4 (&bv)[NT],
                                    f32x16 (&acc)[kWR][kTT]) {
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int r = 0; r < kWR; ++r) acc[r][j] = mfma_32x32x16(a[r], bv[j], acc[r][j]);
}

// Scheduling pattern of one k-step: each LDS read of the next k-step's token
// operands is paired with the two MFMAs of one token tile of this k-step, and
// the weight loads follow (masks: 0x100 DS read, 0x008 MFMA, 0x020 VMEM read).
template <int NT>
__device__ __forceinline__ void step_schedule() {
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, kWR, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x020, kWR, 0);
}

// Main loop over K for a tile whose first NT 32-token tiles hold tokens.
// Software pipeline, per k-step: the token operands of the next k-step are
// read from LDS into a second register set while this k-step's 2*NT MFMAs run;
// the weight queue runs kPre k-steps ahead.  Per 64-wide k-tile the staged
// token slice of the next k-tile is written to the other LDS buffer and the
// barrier placed before the last k-step, so even the first operands of a
// k-tile are read under MFMA work; the token loads of the k-tile after that
// are already in flight.  Two k-tiles per iteration keep every queue slot and
// buffer static; loads are unconditional (clamped), so nothing in the loop
// branches.
template <int NT>
__device__ __forceinline__ void tile_mainloop(const TileCtx& c, u32x4 (*lds)[kBlk * 64],
                                              f32x16 (&acc)[kWR][kTT]) {
  const int nkt = c.ksteps / (kKT / kKStep);
  u32x4 qa[kPre][kWR], bc[NT], bn[NT];
  // The prologue issues its loads in the loop's own order (stage k+1, stage
  // k+2, then the weight queue), so the wait counts the compiler derives at the
  // loop head are the steady-state ones rather than a tighter prologue bound.
  u32x4 pbs[2][kBW];  // token stages k2+1 and k2+2 in flight
  load_b(c, 0, nkt, pbs[0]);
  store_b(lds[0], c, pbs[0]);
  load_b(c, 1, nkt, pbs[1]);
  load_b(c, 2, nkt, pbs[0]);
#pragma unroll
  for (int i = 0; i < kPre; ++i) load_a(c, i, qa[i]);
  __syncthreads();
  read_b<NT>(lds[0], 0, c.lane, bc);
  for (int kt = 0; kt < nkt; kt += 2) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int k2 = kt + half;
      const u32x4* buf = lds[half];
      u32x4* nbuf = lds[half ^ 1];
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        const int q = (half * 4 + i) % kPre;
        read_b<NT>(buf, i + 1, c.lane, bn);
        mac<NT>(qa[q], bc, acc);
        load_a(c, k2 * 4 + i + kPre, qa[q]);
        step_schedule<NT>();
#pragma unroll
        for (int j = 0; j < NT; ++j) bc[j] = bn[j];
      }
      store_b(nbuf, c, pbs[half ^ 1]);
      __syncthreads();
      load_b(c, k2 + 3, nkt, pbs[half ^ 1]);
      const int q = (half * 4 + 3) % kPre;
      read_b<NT>(nbuf, 0, c.lane, bn);
      mac<NT>(qa[q], bc, acc);
      load_a(c, k2 * 4 + 3 + kPre, qa[q]);
      step_schedule<NT>();
#pragma unroll
      for (int j = 0; j < NT; ++j) bc[j] = bn[j];
    }
  }
}
}  // namespace

// Grid: a 1-D list of (expert, weight block, token tile) work units, ordered
// expert-major, then weight block, then token tile, and dealt to the 8 XCDs in
// contiguous ranges (workgroup b runs on XCD b % 8), so the token tiles that
// share a weight block run at the same time on one XCD and share its L2.
template <int MODE>
__global__ __launch_bounds__(256, 2) void k_expert_tile(
    const uint16_t* __restrict__ wpk, const uint16_t* __restrict__ src,
    const int* __restrict__ tilemap, int max_tiles, const int* __restrict__ counts,
    const int* __restrict__ offsets, const int* __restrict__ gather,
    const float* __restrict__ gate, const float* __restrict__ inv, int k, int E,
    const uint16_t* __restrict__ zrow, uint16_t* __restrict__ dst16, float* __restrict__ ybuf,
    int d, int F) {
  __shared__ u32x4 lds[2][kBlk * 64];

  const int K = MODE == 0 ? d : F;
  const int nwb = MODE == 0 ? 2 * F / kRowsWG : d / kRowsWG;
  const int G = gridDim.x, b = blockIdx.x;
  const int L = (b & 7) * (G >> 3) + (b >> 3);
  const int ntiles = tilemap[0];
  if (L >= ntiles * nwb) return;
  const int* tstart = tilemap + 1 + max_tiles;
  int e = 0;
  while (e + 1 < E && tstart[e + 1] * nwb <= L) ++e;
  const int r = L - tstart[e] * nwb, nt = tstart[e + 1] - tstart[e];
  const int wb = r / nt, mtile = r - (r / nt) * nt;  // token tiles of one weight block adjacent
  const int cnt = counts[e], off = offsets[e];
  const int row0 = mtile * kTileTokens;
  const int nvalid = min(kTileTokens, cnt - row0);
  const int ntt = (nvalid + 31) >> 5;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  TileCtx c;
  c.wave = wave;
  c.lane = lane;
  c.ksteps = K / kKStep;
  c.tile_elems = (size_t)c.ksteps * kBlockElems;
  // this wave's weight tiles: gate and up of F tile (4*wb + wave), or
  // d_model tiles (8*wb + 2*wave, +1)
  const size_t blk = MODE == 0 ? ((size_t)e * (F / kTileRows) + (size_t)wb * 4 + wave) * 2
                               : (size_t)e * (d / kTileRows) + (size_t)wb * 8 + wave * 2;
  c.wa = wpk + blk * c.tile_elems + lane * 8;
  {
    const int kc = tid & 7;
#pragma unroll
    for (int j = 0; j < kBW; ++j) {
      const int rr = (j * 256 + tid) >> 3;  // token row of this chunk (tile-local)
      const bool valid = rr < nvalid;
      const int slot = off + row0 + rr;
      const uint16_t* row = valid ? src + (size_t)(MODE == 0 ? gather[slot] : slot) * K : zrow;
      c.brow[j] = row + kc * 8;
    }
    const int r0 = tid >> 3;  // row of chunk 0; chunk j is row r0 + 32 j (same lane, next tile)
    c.bdst = ((r0 >> 5) * 4 + (kc >> 1)) * 64 + (kc & 1) * 32 + (r0 & 31);
  }

  f32x16 acc[kWR][kTT];
#pragma unroll
  for (int i = 0; i < kWR; ++i)
#pragma unroll
    for (int j = 0; j < kTT; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  switch (ntt) {
    case 4: tile_mainloop<4>(c, lds, acc); break;
    case 3: tile_mainloop<3>(c, lds, acc); break;
    case 2: tile_mainloop<2>(c, lds, acc); break;
    default: tile_mainloop<1>(c, lds, acc); break;
  }

  // epilogue
  const int col = lane & 31;
#pragma unroll
  for (int j = 0; j < kTT; ++j) {
    const int rr = j * 32 + col;  // tile-local token row
    if (rr >= nvalid) continue;
    const int slot = off + row0 + rr;
    if constexpr (MODE == 0) {
      const float sc = inv[gather[slot]];  // RMSNorm scale of this token
      const int ft = wb * 4 + wave;
      uint16_t* dst = dst16 + (size_t)slot * F + ft * kTileRows;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float v4[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
          v4[t] = silu(sc * acc[0][j][4 * q + t]) * (sc * acc[1][j][4 * q + t]);
        u32x2 v;
        v[0] = pack_bf16x2(v4[0], v4[1]);
        v[1] = pack_bf16x2(v4[2], v4[3]);
        *reinterpret_cast<u32x2*>(dst + c32_row(4 * q, lane)) = v;
      }
    } else {
      const int tok = k == 1 ? gather[slot] : 0;
      const float gw = k == 1 ? gate[tok] : 0.f;
#pragma unroll
      for (int i = 0; i < kWR; ++i) {
        const int mbase = (wb * 8 + wave * 2 + i) * kTileRows;
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
  const int g0 = ((2 * F / kRowsWG) * a.max_tiles + 7) / 8 * 8;
  const int g1 = ((d / kRowsWG) * a.max_tiles + 7) / 8 * 8;
  hipError_t err = launch(k_expert_tile<0>, dim3(g0), dim3(256), a.stream, a.ev[kSlotExpertsA],
                          (const uint16_t*)a.wgu, (const uint16_t*)a.xn, (const int*)a.tilemap,
                          a.max_tiles, (const int*)a.counts, (const int*)a.offsets,
                          (const int*)a.gather, (const float*)a.gate, (const float*)a.inv,
                          a.dim.k, a.dim.E, (const uint16_t*)a.zrow, (uint16_t*)a.act, a.ybuf, d,
                          F);
  if (err != hipSuccess) return err;
  return launch(k_expert_tile<1>, dim3(g1), dim3(256), a.stream, a.ev[kSlotExpertsB],
                (const uint16_t*)a.wd, (const uint16_t*)a.act, (const int*)a.tilemap, a.max_tiles,
                (const int*)a.counts, (const int*)a.offsets, (const int*)a.gather,
                (const float*)a.gate, (const float*)a.inv, a.dim.k, a.dim.E,
                (const uint16_t*)a.zrow, (uint16_t*)a.out, a.ybuf, d, F);
}

}  // namespace moe
