// K2: expert histogram, prefix scan and stable token permutation.
//
// Dispatch step implied by sparse routing (telknet.cc article, section 2.1:
// TopK restricts each token's compute to a few experts): the T*k assignments
// a = t*k + j are counting-sorted by expert so that every expert sees its rows
// contiguously, with slots inside an expert in increasing a.
//
// One workgroup of 16 waves.  The assignment array is cut into 16 contiguous
// segments (one per wave) of 64-wide chunks.  Ranks never come from atomics:
// within a chunk, a lane's rank among lanes of the same expert is the popcount
// of that expert's ballot below the lane; across chunks a per-expert running
// base (held by lane e) advances by the ballot's popcount; across waves the
// bases start from an exclusive scan of the per-wave counts of a first pass.
// The result is deterministic and identical to a stable sort by expert.
// The same workgroup then writes the tile map of the grouped GEMM.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

template <int EP>
__global__ __launch_bounds__(1024) void k_route_permute(
    const int* __restrict__ sel, int n, int k, int E, int* __restrict__ counts,
    int* __restrict__ offsets, int* __restrict__ gather, int* __restrict__ scatter,
    int* __restrict__ slot_expert, int* __restrict__ tilemap, int tile_rows, int max_tiles) {
  __shared__ int wc[16][EP];
  __shared__ int cnt_s[EP];
  __shared__ int off_s[EP + 1];
  __shared__ int tstart[EP + 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nchunks = (n + 63) / 64;
  const int cpw = (nchunks + 15) / 16;
  const int c_begin = wave * cpw;
  const int c_end = min(nchunks, c_begin + cpw);

  // pass 1: per-wave counts; lane e keeps expert e's count
  int cnt = 0;
  for (int c = c_begin; c < c_end; ++c) {
    const int a = c * 64 + lane;
    int my = a < n ? sel[a] : -1;
    my = (my >= 0 && my < E) ? my : (a < n ? 0 : -1);
    for (int e = 0; e < E; ++e) {
      const uint64_t m = __ballot(my == e);
      if (lane == e) cnt += __popcll(m);
    }
  }
  if (lane < EP) wc[wave][lane] = lane < E ? cnt : 0;
  __syncthreads();

  // exclusive scan over waves (per expert), then over experts
  if (tid < E) {
    int run = 0;
    for (int w = 0; w < 16; ++w) {
      const int v = wc[w][tid];
      wc[w][tid] = run;
      run += v;
    }
    cnt_s[tid] = run;
  }
  __syncthreads();
  if (tid == 0) {
    int o = 0, ts = 0;
    for (int e = 0; e < E; ++e) {
      off_s[e] = o;
      tstart[e] = ts;
      o += cnt_s[e];
      ts += (cnt_s[e] + tile_rows - 1) / tile_rows;
    }
    off_s[E] = o;
    tstart[E] = ts;
  }
  __syncthreads();
  if (tid < E) {
    counts[tid] = cnt_s[tid];
    offsets[tid] = off_s[tid];
  }
  if (tid == 0) offsets[E] = off_s[E];

  // pass 2: slots
  int base = lane < E ? off_s[lane] + wc[wave][lane] : 0;
  for (int c = c_begin; c < c_end; ++c) {
    const int a = c * 64 + lane;
    int my = a < n ? sel[a] : -1;
    my = (my >= 0 && my < E) ? my : (a < n ? 0 : -1);
    uint64_t mine = 0;
    int add = 0;
    for (int e = 0; e < E; ++e) {
      const uint64_t m = __ballot(my == e);
      if (my == e) mine = m;
      if (lane == e) add = __popcll(m);
    }
    const int b = __shfl(base, my < 0 ? 0 : my, kWave);
    if (my >= 0) {
      const uint64_t below = (1ull << lane) - 1ull;
      const int pos = b + __popcll(mine & below);
      gather[pos] = a / k;
      scatter[a] = pos;
      slot_expert[pos] = my;
    }
    base += add;
  }

  // tile map for the grouped GEMM: count, entries (expert << 16 | m-tile),
  // then the first tile of each expert (E + 1 values)
  if (tilemap != nullptr) {
    const int total = min(tstart[E], max_tiles);
    if (tid == 0) tilemap[0] = total;
    if (tid <= E) tilemap[1 + max_tiles + tid] = min(tstart[tid], max_tiles);
    for (int e = 0; e < E; ++e) {
      const int s0 = tstart[e], nt = tstart[e + 1] - tstart[e];
      for (int i = tid; i < nt; i += 1024)
        if (s0 + i < max_tiles) tilemap[1 + s0 + i] = (e << 16) | i;
    }
  }
}

namespace {
template <int EP>
hipError_t launch_ep(const FwdArgs& a) {
  return launch(k_route_permute<EP>, dim3(1), dim3(1024), a.stream, a.ev[kSlotPermute], a.sel, a.n,
                a.dim.k, a.dim.E, a.counts, a.offsets, a.gather, a.scatter, a.slot_expert,
                a.tilemap, kTileTokens, a.max_tiles);
}
}  // namespace

hipError_t launch_route_permute(const FwdArgs& a) {
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

}  // namespace moe
