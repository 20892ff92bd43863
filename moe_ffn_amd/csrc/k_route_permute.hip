// K2: expert histogram, prefix scan and stable token permutation.
//
// Dispatch step implied by sparse routing (telknet.cc article, section 2.1:
// TopK restricts each token's compute to a few experts): the T*k assignments
// a = t*k + j are counting-sorted by expert so that every expert sees its rows
// contiguously, with slots inside an expert in increasing a.
//
// Ranks never come from the order of atomics: within a chunk of 64
// assignments, the lanes holding the same expert are found with log2(E)
// ballots (one per bit of the expert id), and a lane's rank is the number of
// such peers below it.  Up to 8192 assignments one launch does it all
// (k_route_fused: every workgroup counts all chunks itself and places four;
// at 4096 assignments 5.0 us of event time against 10.0 for two launches, the
// step 1.5-1.8 us shorter).  Larger batches take two launches over P groups of
// consecutive chunks (P at most kPermuteMaxGroups, each group one workgroup of
// four waves, each wave a contiguous run of the group's chunks): the first
// counts each group's assignments per expert; the second gives every group
// its bases: the expert's offset (from the totals of all groups) plus the
// counts of the groups before it, then of the waves before it in the group,
// then a running base per wave across its chunks.  Either way the result is
// deterministic and identical to a stable sort by expert.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {
constexpr int kPB = 16;  // 64-wide chunks whose expert ids are loaded together
// one-launch form: waves per workgroup, chunks placed per workgroup, and the
// most chunks it takes (8192 assignments: each wave counts at most 8 chunks;
// at 16384 assignments the redundant counting made the step no faster than
// the two launches)
constexpr int kFusedWaves = 16, kFusedCpg = 4, kFusedMaxChunks = 128;

// Expert ids of chunks cb .. cb+kPB-1 for this lane; indexes past the end are
// clamped (their values are ignored), so every load stays in bounds.
__device__ __forceinline__ void load_batch(const int* __restrict__ sel, int n, int cb, int lane,
                                           int (&v)[kPB]) {
#pragma unroll
  for (int j = 0; j < kPB; ++j) v[j] = sel[min((cb + j) * 64 + lane, n - 1)];
}

// Expert of assignment (chunk c, lane): -1 past the end; an id outside [0, E)
// (which the router never writes) is counted as expert 0 so every slot is filled.
__device__ __forceinline__ int expert_of(int v, int c, int lane, int n, int E) {
  const int a = c * 64 + lane;
  if (a >= n) return -1;
  return (v >= 0 && v < E) ? v : 0;
}

// Lanes of the wave whose expert equals this lane's (valid lanes only).
template <int NB>
__device__ __forceinline__ uint64_t peers_of(int my) {
  uint64_t p = __ballot(my >= 0);
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const bool bit = (my >> b) & 1;
    const uint64_t m = __ballot(bit);
    p &= bit ? m : ~m;
  }
  return p;
}
}  // namespace

// The chunks of group g and wave w of it: [c0, c1).
struct Part {
  int c0, c1;
};
__device__ __forceinline__ Part wave_part(int nchunks, int cpg, int g, int w) {
  const int cpw = (cpg + 3) / 4;
  const int c0 = min(nchunks, g * cpg + w * cpw);
  const int c1 = min(min(nchunks, (g + 1) * cpg), c0 + cpw);
  return {c0, max(c0, c1)};
}

// This wave's counts per expert over its chunks, added into cnt[EP] (LDS) by
// the lowest lane of each peer group.
template <int EP>
__device__ __forceinline__ void count_part(const int* __restrict__ sel, int n, int E, Part pt,
                                           int lane, int* cnt) {
  constexpr int NB = ilog2(EP);
  const uint64_t below = (1ull << lane) - 1ull;
  for (int cb = pt.c0; cb < pt.c1; cb += kPB) {
    int v[kPB];
    load_batch(sel, n, cb, lane, v);
#pragma unroll
    for (int j = 0; j < kPB; ++j) {
      if (cb + j >= pt.c1) break;
      const int my = expert_of(v[j], cb + j, lane, n, E);
      const uint64_t peers = peers_of<NB>(my);
      if (my >= 0 && (peers & below) == 0) atomicAdd(&cnt[my], __popcll(peers));
    }
  }
}

// Slots of this wave's chunks from its running bases base[EP] (LDS).  All
// lanes read their expert's base before the peer group's lowest lane advances
// it (the write depends on the value read; one wave's LDS operations complete
// in order).
template <int EP>
__device__ __forceinline__ void place_part(const int* __restrict__ sel, int n, int k, int E,
                                           Part pt, int lane, int* base,
                                           int* __restrict__ gather, int* __restrict__ scatter,
                                           int* __restrict__ slot_expert) {
  constexpr int NB = ilog2(EP);
  const uint64_t below = (1ull << lane) - 1ull;
  for (int cb = pt.c0; cb < pt.c1; cb += kPB) {
    int v[kPB];
    load_batch(sel, n, cb, lane, v);
#pragma unroll
    for (int j = 0; j < kPB; ++j) {
      if (cb + j >= pt.c1) break;
      const int a = (cb + j) * 64 + lane;
      const int my = expert_of(v[j], cb + j, lane, n, E);
      const uint64_t peers = peers_of<NB>(my);
      if (my >= 0) {
        const int b = base[my];
        const int pos = b + __popcll(peers & below);
        gather[pos] = a / k;
        scatter[a] = pos;
        slot_expert[pos] = my;
        if ((peers & below) == 0) base[my] = b + __popcll(peers);
      }
    }
  }
}

// Launch 1: hist[g][e] = assignments of group g routed to expert e.
template <int EP>
__global__ __launch_bounds__(256) void k_route_hist(const int* __restrict__ sel, int n, int E,
                                                    int cpg, int* __restrict__ hist) {
  __shared__ int wc[4][EP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nchunks = (n + 63) / 64;
  for (int i = tid; i < 4 * EP; i += 256) wc[i / EP][i % EP] = 0;
  __syncthreads();
  count_part<EP>(sel, n, E, wave_part(nchunks, cpg, blockIdx.x, wave), lane, wc[wave]);
  __syncthreads();
  if (tid < EP) hist[blockIdx.x * EP + tid] = wc[0][tid] + wc[1][tid] + wc[2][tid] + wc[3][tid];
}

// Launch 2: counts, offsets (group 0 writes them) and every assignment's slot.
template <int EP>
__global__ __launch_bounds__(256) void k_route_place(
    const int* __restrict__ sel, int n, int k, int E, int cpg, const int* __restrict__ hist,
    int* __restrict__ counts, int* __restrict__ offsets, int* __restrict__ gather,
    int* __restrict__ scatter, int* __restrict__ slot_expert) {
  constexpr int G = 256 / EP;  // thread groups that split the group axis
  __shared__ int part_tot[G][EP], part_pre[G][EP];
  __shared__ int wc[4][EP];    // per-wave counts, then per-wave running bases
  __shared__ int off_s[EP + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nchunks = (n + 63) / 64;
  const int P = gridDim.x, g = blockIdx.x;

  {  // totals over all groups and over the groups before this one
    const int e = tid % EP, gi = tid / EP;
    int tot = 0, pre = 0;
    for (int q = gi; q < P; q += G) {
      const int v = hist[q * EP + e];
      tot += v;
      pre += q < g ? v : 0;
    }
    part_tot[gi][e] = tot;
    part_pre[gi][e] = pre;
  }
  for (int i = tid; i < 4 * EP; i += 256) wc[i / EP][i % EP] = 0;
  __syncthreads();
  const Part pt = wave_part(nchunks, cpg, g, wave);
  count_part<EP>(sel, n, E, pt, lane, wc[wave]);
  if (wave == 0) {  // offsets: exclusive scan of the totals over the experts (EP <= 64)
    int tot = 0;
    if (lane < EP)
      for (int gi = 0; gi < G; ++gi) tot += part_tot[gi][lane];
    int inc = tot;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(inc, o, 64);
      if (lane >= o) inc += t;
    }
    if (lane < EP) off_s[lane] = inc - tot;
    if (lane == EP - 1) off_s[EP] = inc;
    if (g == 0 && lane < E) {
      counts[lane] = tot;
      offsets[lane] = inc - tot;
    }
    if (g == 0 && lane == E - 1) offsets[E] = inc;
  }
  __syncthreads();
  if (tid < EP) {  // this group's first slot of each expert, then each wave's
    int base = off_s[tid];
    for (int gi = 0; gi < G; ++gi) base += part_pre[gi][tid];
    for (int w = 0; w < 4; ++w) {
      const int v = wc[w][tid];
      wc[w][tid] = base;
      base += v;
    }
  }
  __syncthreads();
  place_part<EP>(sel, n, k, E, pt, lane, wc[wave], gather, scatter, slot_expert);
}

// One launch for up to kFusedMaxChunks chunks: workgroup g places chunks
// 4g .. 4g+3 (one per wave), and first counts every chunk itself, its 16
// waves taking the chunks in turn: per wave the totals per expert, the counts
// of the chunks before its group, and each own chunk's counts, so no
// histogram of the other groups is needed.  (One workgroup placing every
// chunk took 8.2 us at 4096 assignments and 18.9 us at 16384: its scattered
// stores all go through one CU; here they spread over the groups.)
template <int EP>
__global__ __launch_bounds__(kFusedWaves * 64) void k_route_fused(
    const int* __restrict__ sel, int n, int k, int E, int* __restrict__ counts,
    int* __restrict__ offsets, int* __restrict__ gather, int* __restrict__ scatter,
    int* __restrict__ slot_expert) {
  constexpr int NB = ilog2(EP);
  __shared__ int tot[kFusedWaves][EP], pre[kFusedWaves][EP];
  __shared__ int own[kFusedCpg][EP];  // own chunks' counts, then their running bases
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nchunks = (n + 63) / 64;
  const int c0 = blockIdx.x * kFusedCpg, c1 = min(nchunks, c0 + kFusedCpg);
  const uint64_t below = (1ull << lane) - 1ull;
  for (int i = tid; i < kFusedWaves * EP; i += kFusedWaves * 64) {
    tot[i / EP][i % EP] = 0;
    pre[i / EP][i % EP] = 0;
  }
  if (tid < kFusedCpg * EP) own[tid / EP][tid % EP] = 0;
  __syncthreads();
  for (int cb = wave; cb < nchunks; cb += kFusedWaves * kPB) {
    int v[kPB];  // chunks cb + 16 j; indexes past the end are clamped and ignored
#pragma unroll
    for (int j = 0; j < kPB; ++j) v[j] = sel[min((cb + kFusedWaves * j) * 64 + lane, n - 1)];
#pragma unroll
    for (int j = 0; j < kPB; ++j) {
      const int c = cb + kFusedWaves * j;
      if (c >= nchunks) break;
      const int my = expert_of(v[j], c, lane, n, E);
      const uint64_t peers = peers_of<NB>(my);
      if (my >= 0 && (peers & below) == 0) {
        const int pc = __popcll(peers);
        atomicAdd(&tot[wave][my], pc);
        if (c < c0) atomicAdd(&pre[wave][my], pc);
        else if (c < c1) atomicAdd(&own[c - c0][my], pc);
      }
    }
  }
  __syncthreads();
  if (wave == 0) {  // offsets: exclusive scan of the totals over the experts (EP <= 64)
    int t = 0, b = 0;
    if (lane < EP)
      for (int w = 0; w < kFusedWaves; ++w) {
        t += tot[w][lane];
        b += pre[w][lane];
      }
    int inc = t;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(inc, o, 64);
      if (lane >= o) inc += u;
    }
    if (blockIdx.x == 0 && lane < E) {
      counts[lane] = t;
      offsets[lane] = inc - t;
    }
    if (blockIdx.x == 0 && lane == E - 1) offsets[E] = inc;
    if (lane < EP) {  // each own chunk's first slot per expert
      int base = inc - t + b;
      for (int j = 0; j < kFusedCpg; ++j) {
        const int v = own[j][lane];
        own[j][lane] = base;
        base += v;
      }
    }
  }
  __syncthreads();
  if (wave < c1 - c0)
    place_part<EP>(sel, n, k, E, Part{c0 + wave, c0 + wave + 1}, lane, own[wave], gather, scatter,
                   slot_expert);
}

namespace {
// One launch up to kFusedMaxChunks chunks; beyond, groups of at least four
// chunks (one per wave), at most kPermuteMaxGroups.
template <int EP>
hipError_t launch_ep(const FwdArgs& a) {
  const int nchunks = (a.n + 63) / 64;
  if (nchunks <= kFusedMaxChunks)
    return launch(k_route_fused<EP>, dim3((nchunks + kFusedCpg - 1) / kFusedCpg),
                  dim3(kFusedWaves * 64), a.stream, a.ev[kSlotPermute], a.sel, a.n, a.dim.k,
                  a.dim.E, a.counts, a.offsets, a.gather, a.scatter, a.slot_expert);
  int cpg = 4;
  if ((nchunks + cpg - 1) / cpg > kPermuteMaxGroups)
    cpg = (nchunks + kPermuteMaxGroups - 1) / kPermuteMaxGroups;
  const int P = (nchunks + cpg - 1) / cpg;
  const KEv& ev = a.ev[kSlotPermute];
  hipError_t he = launch(k_route_hist<EP>, dim3(P), dim3(256), a.stream, KEv{ev.start, nullptr},
                         a.sel, a.n, a.dim.E, cpg, a.hist);
  if (he != hipSuccess) return he;
  return launch(k_route_place<EP>, dim3(P), dim3(256), a.stream, KEv{nullptr, ev.stop}, a.sel,
                a.n, a.dim.k, a.dim.E, cpg, (const int*)a.hist, a.counts, a.offsets, a.gather,
                a.scatter, a.slot_expert);
}
}  // namespace

hipError_t launch_route_permute(const FwdArgs& a) {
  if (a.n <= 0) return hipErrorInvalidValue;
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
