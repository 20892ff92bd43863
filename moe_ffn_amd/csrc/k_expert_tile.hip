// K3 (prefill shapes): grouped SwiGLU GEMMs over the experts, LDS-staged tiles.
//
// Expert FFN y = W_down (SiLU(W_gate x) * (W_up x)) per routed assignment
// (SwiGLU: GLU variants paper on the ZONOS2 report's "Builds on" list; 16
// experts per layer, digest item 5).  Two launches:
//   MODE 0  act[slot, f] = bf16( SiLU(x W_gate^T) * (x W_up^T) )   K = d_model
//   MODE 1  y[slot, m]   = act[slot] W_down^T                       K = d_ff
//           k = 1: out[token] = bf16(gate * y); k > 1: y kept in fp32.
// A workgroup computes a (NR*64)-weight-row x 128-token tile: NR waves (8, or
// 4 where the rows do not divide by 512) stacked along the weight rows, each
// owning two 32-row MFMA tiles against all four 32-token tiles (8
// accumulators of 32x32).  Weights are read straight from the packed bank
// (MFMA operand order, 1 KiB per wave-wide load) into registers, four k-steps
// ahead, so they never pass through LDS.  Only the token tile is shared: rows
// gathered on load through the expert-ordered slot list (8 rows x 128
// contiguous bytes per wave-wide load) are written to LDS in operand order
// (swizzled, conflict-free both ways), three 64-wide k-tiles in flight (two
// in registers, one in LDS) and one barrier per k-tile.  The operand bytes a
// CU pulls from L2 per flop fall as its resident tile grows (per 16-wide
// k-step: 16 KiB of weights + 4 KiB of tokens for 2 MFLOP with eight waves,
// against 24 KiB for two four-wave workgroups), and that L2-to-CU stream is
// what bounds this kernel.  Partial token tiles (the tail of each expert) run
// a variant that skips the empty 32-token tiles.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {
constexpr int kTT = kTileTokens / 32;      // 32-token MFMA tiles per workgroup (4)
constexpr int kWR = 2;                     // 32-row weight tiles per wave
constexpr int kPre = 4;                    // k-steps of weight loads in flight per wave
constexpr int kKT = 64;                    // k per LDS stage of the token tile
constexpr int kBlk = kTT * (kKT / kKStep); // 1 KiB operand blocks per token stage (16)

// Workgroup shape: NR x NTG waves, NR stacked along the weight rows (NR*64
// rows), NTG along the tokens (NTG*128 tokens).  Waves of one row group load
// the same weight tiles (the second load hits the CU's L1).
template <int NR_, int NTG_>
struct Geo {
  static constexpr int NR = NR_, NTG = NTG_;
  static constexpr int kWaves = NR * NTG;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kRowsWG = NR * kWR * 32;
  static constexpr int kTokWG = NTG * kTileTokens;
  static constexpr int kStage = NTG * kBlk;                // operand blocks per token stage
  static constexpr int kBW = kStage * 64 / kThreads;       // chunks staged per thread per stage
};

template <class GEO>
struct TileCtx {
  const uint16_t* wa;     // this wave's first weight tile (lane offset applied)
  size_t tile_elems;      // elements of one packed 32-row tile
  int ksteps;             // K / 16
  const uint16_t* brow[GEO::kBW];  // source of each staged chunk (k offset applied)
  int bdst;  // LDS slot (16-byte units) of chunk 0; chunk j is kThreads/8 rows = kThreads slots on
  int bofs;  // LDS slot of this wave's token group (kBlk blocks per group)
  int wave, lane;
};

template <class GEO>
__device__ __forceinline__ void load_a(const TileCtx<GEO>& c, int s, u32x4 (&q)[kWR]) {
  const int sc = s < c.ksteps ? s : c.ksteps - 1;  // clamp: surplus loads stay in bounds
#pragma unroll
  for (int r = 0; r < kWR; ++r) q[r] = ldg16(c.wa + r * c.tile_elems + (size_t)sc * kBlockElems);
}

// Token staging: the workgroup's threads copy a kTokWG x 64 slice of gathered
// rows per k-tile, each wave-wide load reading 8 rows x 128 contiguous bytes
// (8 full cache lines): thread t, chunk j covers row r = (j*kThreads + t) / 8
// and 16-byte k-chunk kc = t % 8.  The LDS write scatters each chunk to its
// place in MFMA operand order: block (r/32)*4 + kc/2, operand lane
// li = (kc%2)*32 + r%32, stored at 16-byte slot swz(block, li) of the block.
//
// swz(block, li) = li ^ ((4*(block%4) + 2*(li/32)) & 15) permutes the slots
// inside each group of 16: the 16 lanes an MFMA operand read serves together
// still cover 16 consecutive slots (all 64 banks), while the 8 k-chunks of one
// token row, which the staging write issues together, now land in 8
// different bank groups instead of the same one (block stride 1 KiB and
// k-group stride 512 B are multiples of the 256-byte bank cycle).
__device__ __forceinline__ int swz(int block, int li) {
  return li ^ ((4 * (block & 3) + 2 * (li >> 5)) & 15);
}
template <class GEO>
__device__ __forceinline__ void load_b(const TileCtx<GEO>& c, int kt, int nkt,
                                       u32x4 (&p)[GEO::kBW]) {
  const int kc = kt < nkt ? kt : nkt - 1;
#pragma unroll
  for (int j = 0; j < GEO::kBW; ++j) p[j] = ldg16(c.brow[j] + kc * kKT);
}
template <class GEO>
__device__ __forceinline__ void store_b(u32x4* buf, const TileCtx<GEO>& c,
                                        const u32x4 (&p)[GEO::kBW]) {
#pragma unroll
  for (int j = 0; j < GEO::kBW; ++j) buf[c.bdst + j * GEO::kThreads] = p[j];
}

template <int NT>
__device__ __forceinline__ void read_b(const u32x4* buf, int s16, int lane, u32x4 (&bv)[NT]) {
#pragma unroll
  for (int j = 0; j < NT; ++j) bv[j] = buf[(j * 4 + s16) * 64 + swz(s16, lane)];
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
template <int NT, class GEO>
__device__ __forceinline__ void tile_mainloop(const TileCtx<GEO>& c,
                                              u32x4 (*lds)[GEO::kStage * 64],
                                              f32x16 (&acc)[kWR][kTT]) {
  const int nkt = c.ksteps / (kKT / kKStep);
  u32x4 qa[kPre][kWR], bc[NT], bn[NT];
  // The prologue issues its loads in the loop's own order (stage k+1, stage
  // k+2, then the weight queue), so the wait counts the compiler derives at the
  // loop head are the steady-state ones rather than a tighter prologue bound.
  u32x4 pbs[2][GEO::kBW];  // token stages k2+1 and k2+2 in flight
  load_b(c, 0, nkt, pbs[0]);
  store_b(lds[0], c, pbs[0]);
  load_b(c, 1, nkt, pbs[1]);
  load_b(c, 2, nkt, pbs[0]);
#pragma unroll
  for (int i = 0; i < kPre; ++i) load_a(c, i, qa[i]);
  __syncthreads();
  read_b<NT>(lds[0] + c.bofs, 0, c.lane, bc);
  for (int kt = 0; kt < nkt; kt += 2) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int k2 = kt + half;
      const u32x4* buf = lds[half] + c.bofs;
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
      read_b<NT>(nbuf + c.bofs, 0, c.lane, bn);
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
template <int MODE, class GEO>
__global__ __launch_bounds__(GEO::kThreads, 8 / GEO::kWaves) void k_expert_tile(
    const uint16_t* __restrict__ wpk, const uint16_t* __restrict__ src,
    const int* __restrict__ tilemap, int max_tiles, const int* __restrict__ counts,
    const int* __restrict__ offsets, const int* __restrict__ gather,
    const float* __restrict__ gate, const float* __restrict__ inv, int k, int E,
    const uint16_t* __restrict__ zrow, uint16_t* __restrict__ dst16, float* __restrict__ ybuf,
    int d, int F) {
  constexpr int NR = GEO::NR, NTG = GEO::NTG;
  __shared__ u32x4 lds[2][GEO::kStage * 64];

  const int K = MODE == 0 ? d : F;
  const int nwb = MODE == 0 ? 2 * F / GEO::kRowsWG : d / GEO::kRowsWG;
  const int G = gridDim.x, b = blockIdx.x;
  const int L = (b & 7) * (G >> 3) + (b >> 3);
  // work units: per expert, nwb weight blocks x ceil(tiles / NTG) token spans
  const int* tstart = tilemap + 1 + max_tiles;
  int e = 0, base = 0, nsp = 0;
  for (; e < E; ++e) {
    nsp = (tstart[e + 1] - tstart[e] + NTG - 1) / NTG;
    if (L < base + nsp * nwb) break;
    base += nsp * nwb;
  }
  if (e >= E) return;
  const int r = L - base;
  const int wb = r / nsp, span = r - (r / nsp) * nsp;  // token spans of one weight block adjacent
  const int cnt = counts[e], off = offsets[e];
  const int row0 = span * GEO::kTokWG;
  const int nvalid = min(GEO::kTokWG, cnt - row0);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rg = wave % NR, tg = wave / NR;  // row group, token group of this wave
  const int nvw = nvalid - tg * kTileTokens;  // tokens of this wave's group (may be <= 0)
  const int ntt = nvw <= 0 ? 1 : (nvw + 31) >> 5;
  TileCtx<GEO> c;
  c.wave = wave;
  c.lane = lane;
  c.ksteps = K / kKStep;
  c.tile_elems = (size_t)c.ksteps * kBlockElems;
  c.bofs = tg * kBlk * 64;
  // this wave's weight tiles: gate and up of F tile (NR*wb + rg), or
  // d_model tiles (2*NR*wb + 2*rg, +1)
  const size_t blk = MODE == 0
      ? ((size_t)e * (F / kTileRows) + (size_t)wb * NR + rg) * 2
      : (size_t)e * (d / kTileRows) + (size_t)wb * 2 * NR + rg * 2;
  c.wa = wpk + blk * c.tile_elems + lane * 8;
  {
    const int kc = tid & 7;
#pragma unroll
    for (int j = 0; j < GEO::kBW; ++j) {
      const int rr = (j * GEO::kThreads + tid) >> 3;  // token row of this chunk (tile-local)
      const bool valid = rr < nvalid;
      const int slot = off + row0 + rr;
      const uint16_t* row = valid ? src + (size_t)(MODE == 0 ? gather[slot] : slot) * K : zrow;
      c.brow[j] = row + kc * 8;
    }
    const int r0 = tid >> 3;  // row of chunk 0; chunk j is row r0 + j*kThreads/8
    c.bdst = ((r0 >> 5) * 4 + (kc >> 1)) * 64 + swz(kc >> 1, (kc & 1) * 32 + (r0 & 31));
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
    const int rr = tg * kTileTokens + j * 32 + col;  // tile-local token row
    if (rr >= nvalid) continue;
    const int slot = off + row0 + rr;
    if constexpr (MODE == 0) {
      const float sc = inv[gather[slot]];  // RMSNorm scale of this token
      const int ft = wb * NR + rg;
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
        const int mbase = (wb * 2 * NR + rg * 2 + i) * kTileRows;
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

namespace {
template <int MODE, class GEO>
hipError_t launch_mode(const FwdArgs& a) {
  const int d = a.dim.d, F = a.dim.F;
  const int rows = MODE == 0 ? 2 * F : d;
  const int grid = ((rows / GEO::kRowsWG) * a.max_tiles + 7) / 8 * 8;
  return launch(k_expert_tile<MODE, GEO>, dim3(grid), dim3(GEO::kThreads), a.stream,
                a.ev[MODE == 0 ? kSlotExpertsA : kSlotExpertsB],
                (const uint16_t*)(MODE == 0 ? a.wgu : a.wd),
                (const uint16_t*)(MODE == 0 ? a.xn : a.act), (const int*)a.tilemap, a.max_tiles,
                (const int*)a.counts, (const int*)a.offsets, (const int*)a.gather,
                (const float*)a.gate, (const float*)a.inv, a.dim.k, a.dim.E,
                (const uint16_t*)a.zrow, (uint16_t*)(MODE == 0 ? a.act : a.out), a.ybuf, d, F);
}
// 512 weight rows x 128 tokens, one workgroup per CU.  (A 256 x 256 shape,
// Geo<4, 2>, pulls fewer bytes per flop but its two row groups fetch the same
// weight lines back to back, and the second fetch stalls the CU's L1 on the
// pending line instead of sharing it: measured 1.5-1.9x slower.)
using GBig = Geo<8, 1>;
constexpr int kBigRows = GBig::kRowsWG;
using G4x1 = Geo<4, 1>;  // 256 weight rows x 128 tokens, two workgroups per CU
}  // namespace

// Eight waves (one workgroup per CU) where the rows divide into them, else
// four (two workgroups per CU).  The down projection of top-k > 1 layers
// keeps four waves: its fp32 epilogue is twice as large and is hidden only
// behind a second resident workgroup.
hipError_t launch_experts_tile(const FwdArgs& a) {
  const bool big_gu = (2 * a.dim.F) % kBigRows == 0;
  const bool big_d = a.dim.d % kBigRows == 0 && a.dim.k == 1;
  hipError_t err = big_gu ? launch_mode<0, GBig>(a) : launch_mode<0, G4x1>(a);
  if (err != hipSuccess) return err;
  return big_d ? launch_mode<1, GBig>(a) : launch_mode<1, G4x1>(a);
}

}  // namespace moe
