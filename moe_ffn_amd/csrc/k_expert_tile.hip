// K3 (prefill shapes): grouped SwiGLU GEMMs over the experts, LDS-staged tiles.
//
// Expert FFN y = W_down (SiLU(W_gate x) * (W_up x)) per routed assignment
// (SwiGLU: GLU variants paper on the ZONOS2 report's "Builds on" list; 16
// experts per layer, digest item 5).  Two launches:
//   MODE 0  act[slot, f] = bf16( SiLU(x W_gate^T) * (x W_up^T) )   K = d_model
//   MODE 1  y[slot, m]   = act[slot] W_down^T                       K = d_ff
//           k = 1: out[token] = bf16(gate * y); k > 1: y kept in fp32.
// A workgroup computes a 256-weight-row x 256-token tile: four waves stacked
// along the weight rows, each owning two 32-row MFMA tiles against all eight
// 32-token tiles (16 accumulators of 32x32 = 256 registers).  Weights are read
// straight from the packed bank (MFMA operand order, 1 KiB per wave-wide load)
// into registers, eight k-steps ahead, so they never pass through LDS.  Only
// the token tile is shared, staged in LDS in operand order (conflict-free
// 1 KiB reads) from rows gathered on load through the expert-ordered slot
// list; it is fetched two k-tiles ahead and double-buffered, one barrier per
// 64-wide k-tile.  One workgroup per CU (the register file holds the deep
// queues).  Partial token tiles (the tail of each expert) run a variant that
// skips the empty 32-token tiles.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {
constexpr int kTT = kTileTokens / 32;      // 32-token MFMA tiles per workgroup (4)
constexpr int kCons = 4;                   // consumer waves (MFMA), stacked along weight rows
constexpr int kProd = 4;                   // producer waves (token staging)
constexpr int kThreads = (kCons + kProd) * 64;
constexpr int kWR = 2;                     // 32-row weight tiles per consumer wave
constexpr int kRowsWG = kCons * kWR * 32;  // 256 weight rows per workgroup
constexpr int kPre = 8;                    // k-steps of weight loads in flight per consumer
constexpr int kKT = 64;                    // k per LDS stage of the token tile
constexpr int kBlk = kTT * (kKT / kKStep); // 1 KiB operand blocks per token stage (16)
constexpr int kStages = 3;                 // LDS ring of token stages
constexpr int kPC = kBlk * 64 / (kProd * 64);  // 16-byte chunks per producer thread per stage (4)

struct TileCtx {
  const uint16_t* wa;        // consumer: first weight tile of this wave (lane offset applied)
  size_t tile_elems;         // elements of one packed 32-row tile
  int ksteps;                // K / 16
  const uint16_t* brow[kPC]; // producer: source of each staged chunk (k offset applied)
  int bdst;                  // producer: LDS index (16-byte units) of chunk 0
  int lane;
};

__device__ __forceinline__ void load_a(const TileCtx& c, int s, u32x4 (&q)[kWR]) {
  const int sc = s < c.ksteps ? s : c.ksteps - 1;  // clamp: surplus loads stay in bounds
#pragma unroll
  for (int r = 0; r < kWR; ++r) q[r] = ldg16(c.wa + r * c.tile_elems + (size_t)sc * kBlockElems);
}

// Producer thread pt copies 16-byte chunks j = 0..kPC-1 of the stage: row
// (j*256 + pt)/8 of the token tile, k-chunk pt%8 -- each wave-wide load reads
// 8 rows x 128 contiguous bytes.  The LDS write scatters each chunk to its
// place in MFMA operand order: block (row/32)*4 + kc/2, lane (kc%2)*32 + row%32.
__device__ __forceinline__ void load_b(const TileCtx& c, int kt, int nkt, u32x4 (&p)[kPC]) {
  const int kc = kt < nkt ? kt : nkt - 1;
#pragma unroll
  for (int j = 0; j < kPC; ++j) p[j] = ldg16(c.brow[j] + kc * kKT);
}
__device__ __forceinline__ void store_b(u32x4* buf, const TileCtx& c, const u32x4 (&p)[kPC]) {
#pragma unroll
  for (int j = 0; j < kPC; ++j) buf[c.bdst + j * 256] = p[j];
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

// Consumer waves: multiply k-tile kt from stage kt % 3.  Per k-step the token
// operands of the next k-step are read into a second register set while this
// k-step's MFMAs run; at the last k-step of a k-tile the next stage (written
// two k-tiles ago, published by the previous barrier) is already readable.
// The weight queue runs kPre k-steps ahead; these waves issue no other global
// load, so nothing slow can sit ahead of a weight load in the in-order return
// queue.  Two k-tiles per iteration keep the queue slots static.
template <int NT>
__device__ __forceinline__ void consumer_loop(const TileCtx& c, u32x4 (*lds)[kBlk * 64],
                                              f32x16 (&acc)[kWR][kTT]) {
  const int nkt = c.ksteps / (kKT / kKStep);
  u32x4 qa[kPre][kWR], bc[NT], bn[NT];
#pragma unroll
  for (int i = 0; i < kPre; ++i) load_a(c, i, qa[i]);
  __syncthreads();  // stages 0 and 1 published
  read_b<NT>(lds[0], 0, c.lane, bc);
  int st = 0;  // stage of the current k-tile
  for (int kt = 0; kt < nkt; kt += 2) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int k2 = kt + half;
      const int nst = st == kStages - 1 ? 0 : st + 1;
      const u32x4* buf = lds[st];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int q = half * 4 + i;
        read_b<NT>(i < 3 ? buf : lds[nst], i < 3 ? i + 1 : 0, c.lane, bn);
        mac<NT>(qa[q], bc, acc);
        load_a(c, k2 * 4 + i + kPre, qa[q]);
        step_schedule<NT>();
#pragma unroll
        for (int j = 0; j < NT; ++j) bc[j] = bn[j];
      }
      __syncthreads();
      st = nst;
    }
  }
}

// Producer waves: at k-tile kt write stage (kt+2) % 3 with the token slice of
// k-tile kt+2 (its loads were issued during k-tile kt-1) and issue the loads of
// k-tile kt+3; the stage being written was last read before the previous
// barrier.  Same number of barriers as the consumers.
__device__ __forceinline__ void producer_loop(const TileCtx& c, u32x4 (*lds)[kBlk * 64]) {
  const int nkt = c.ksteps / (kKT / kKStep);
  u32x4 pb[2][kPC];
  load_b(c, 0, nkt, pb[0]);
  load_b(c, 1, nkt, pb[1]);
  store_b(lds[0], c, pb[0]);
  store_b(lds[1], c, pb[1]);
  load_b(c, 2, nkt, pb[0]);
  __syncthreads();  // stages 0 and 1 published
  int st = 2;       // stage receiving k-tile kt + 2
  for (int kt = 0; kt < nkt; kt += 2) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int k2 = kt + half;
      load_b(c, k2 + 3, nkt, pb[half ^ 1]);
      store_b(lds[st], c, pb[half]);
      __syncthreads();
      st = st == kStages - 1 ? 0 : st + 1;
    }
  }
}
}  // namespace

// Grid: a 1-D list of (expert, weight block, token tile) work units, ordered
// expert-major, then weight block, then token tile, and dealt to the 8 XCDs in
// contiguous ranges (workgroup b runs on XCD b % 8), so the token tiles that
// share a weight block run at the same time on one XCD and share its L2.
template <int MODE>
__global__ __launch_bounds__(kThreads, 1) void k_expert_tile(
    const uint16_t* __restrict__ wpk, const uint16_t* __restrict__ src,
    const int* __restrict__ tilemap, int max_tiles, const int* __restrict__ counts,
    const int* __restrict__ offsets, const int* __restrict__ gather,
    const float* __restrict__ gate, const float* __restrict__ inv, int k, int E,
    const uint16_t* __restrict__ zrow, uint16_t* __restrict__ dst16, float* __restrict__ ybuf,
    int d, int F) {
  __shared__ u32x4 lds[kStages][kBlk * 64];

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
#if MOE_TILE_ORDER == 1
  const int mtile = r / nwb, wb = r - mtile * nwb;  // weight blocks of one token tile adjacent
#elif MOE_TILE_ORDER == 2
  // groups of up to 8 token tiles: within a group, the token tiles of one
  // weight block are adjacent, and consecutive weight blocks follow
  const int gsz = 8 * nwb, g = r / gsz, rem = r - g * gsz;
  const int gm = min(8, nt - g * 8);
  const int wb = rem / gm, mtile = g * 8 + (rem - (rem / gm) * gm);
#else
  const int wb = r / nt, mtile = r - (r / nt) * nt;  // token tiles of one weight block adjacent
#endif
  const int cnt = counts[e], off = offsets[e];
  const int row0 = mtile * kTileTokens;
  const int nvalid = min(kTileTokens, cnt - row0);
  const int ntt = (nvalid + 31) >> 5;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  TileCtx c;
  c.lane = lane;
  c.ksteps = K / kKStep;
  c.tile_elems = (size_t)c.ksteps * kBlockElems;

  f32x16 acc[kWR][kTT];
#pragma unroll
  for (int i = 0; i < kWR; ++i)
#pragma unroll
    for (int j = 0; j < kTT; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  if (wave >= kCons) {
    // producer: gathered token rows, coalesced 8 rows x 128 B per wave-wide load
    const int pt = tid - kCons * 64;
    const int kc = pt & 7;
#pragma unroll
    for (int j = 0; j < kPC; ++j) {
      const int rr = (j * 256 + pt) >> 3;  // token row of this chunk (tile-local)
      const bool valid = rr < nvalid;
      const int slot = off + row0 + rr;
      const uint16_t* row = valid ? src + (size_t)(MODE == 0 ? gather[slot] : slot) * K : zrow;
      c.brow[j] = row + kc * 8;
    }
    const int r0 = pt >> 3;  // chunk j is row r0 + 32 j: next token tile, same lane
    c.bdst = (kc >> 1) * 64 + (kc & 1) * 32 + r0;
    producer_loop(c, lds);
    return;
  }
  // consumer: gate and up of F tile (4*wb + wave), or d_model tiles (8*wb + 2*wave, +1)
  const size_t blk = MODE == 0 ? ((size_t)e * (F / kTileRows) + (size_t)wb * 4 + wave) * 2
                               : (size_t)e * (d / kTileRows) + (size_t)wb * 8 + wave * 2;
  c.wa = wpk + blk * c.tile_elems + lane * 8;
  switch (ntt) {
#if MOE_TILE_TOK > 128
    case 8: consumer_loop<8>(c, lds, acc); break;
    case 7: consumer_loop<7>(c, lds, acc); break;
    case 6: consumer_loop<6>(c, lds, acc); break;
    case 5: consumer_loop<5>(c, lds, acc); break;
#endif
    case 4: consumer_loop<4>(c, lds, acc); break;
    case 3: consumer_loop<3>(c, lds, acc); break;
    case 2: consumer_loop<2>(c, lds, acc); break;
    default: consumer_loop<1>(c, lds, acc); break;
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
  hipError_t err = launch(k_expert_tile<0>, dim3(g0), dim3(kThreads), a.stream, a.ev[kSlotExpertsA],
                          (const uint16_t*)a.wgu, (const uint16_t*)a.xn, (const int*)a.tilemap,
                          a.max_tiles, (const int*)a.counts, (const int*)a.offsets,
                          (const int*)a.gather, (const float*)a.gate, (const float*)a.inv,
                          a.dim.k, a.dim.E, (const uint16_t*)a.zrow, (uint16_t*)a.act, a.ybuf, d,
                          F);
  if (err != hipSuccess) return err;
  return launch(k_expert_tile<1>, dim3(g1), dim3(kThreads), a.stream, a.ev[kSlotExpertsB],
                (const uint16_t*)a.wd, (const uint16_t*)a.act, (const int*)a.tilemap, a.max_tiles,
                (const int*)a.counts, (const int*)a.offsets, (const int*)a.gather,
                (const float*)a.gate, (const float*)a.inv, a.dim.k, a.dim.E,
                (const uint16_t*)a.zrow, (uint16_t*)a.out, a.ybuf, d, F);
}

}  // namespace moe
