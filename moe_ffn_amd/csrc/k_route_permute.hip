// K2: expert histogram, prefix scan and stable token permutation.
//
// Dispatch step implied by sparse routing (telknet.cc article, section 2.1:
// TopK restricts each token's compute to a few experts): the T*k assignments
// a = t*k + j are counting-sorted by expert so that every expert sees its rows
// contiguously, with slots inside an expert in increasing a.
//
// One workgroup of 16 waves.  The assignment array is cut into 16 contiguous
// segments (one per wave) of 64-wide chunks.  Ranks never come from the order
// of atomics: within a chunk, the lanes holding the same expert are found with
// log2(E) ballots (one per bit of the expert id), and a lane's rank is the
// number of such peers below it; across chunks a per-wave, per-expert running
// base in LDS advances by the peer count; across waves the bases start from an
// exclusive scan of the per-wave counts of a first pass.  The result is
// deterministic and identical to a stable sort by expert.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {
constexpr int kPB = 16;  // 64-wide chunks whose expert ids are loaded together

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

template <int EP>
__global__ __launch_bounds__(1024) void k_route_permute(
    const int* __restrict__ sel, int n, int k, int E, int* __restrict__ counts,
    int* __restrict__ offsets, int* __restrict__ gather, int* __restrict__ scatter,
    int* __restrict__ slot_expert) {
  constexpr int NB = ilog2(EP);
  __shared__ int wc[16][EP];  // per-wave counts, then per-wave running bases
  __shared__ int cnt_s[EP];
  __shared__ int off_s[EP + 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nchunks = (n + 63) / 64;
  const int cpw = (nchunks + 15) / 16;
  const int c_begin = wave * cpw;
  const int c_end = min(nchunks, c_begin + cpw);
  const uint64_t below = (1ull << lane) - 1ull;

  for (int i = tid; i < 16 * EP; i += 1024) wc[i / EP][i % EP] = 0;
  __syncthreads();

  // pass 1: per-wave counts, added by the lowest lane of each peer group.
  // The expert ids of kPB chunks are loaded together.
  for (int cb = c_begin; cb < c_end; cb += kPB) {
    int v[kPB];
    load_batch(sel, n, cb, lane, v);
#pragma unroll
    for (int j = 0; j < kPB; ++j) {
      if (cb + j >= c_end) break;
      const int my = expert_of(v[j], cb + j, lane, n, E);
      const uint64_t peers = peers_of<NB>(my);
      if (my >= 0 && (peers & below) == 0) atomicAdd(&wc[wave][my], __popcll(peers));
    }
  }
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
    int o = 0;
    for (int e = 0; e < E; ++e) {
      off_s[e] = o;
      o += cnt_s[e];
    }
    off_s[E] = o;
  }
  __syncthreads();
  if (tid < E) {
    counts[tid] = cnt_s[tid];
    offsets[tid] = off_s[tid];
  }
  if (tid == 0) offsets[E] = off_s[E];
  if (lane < E) wc[wave][lane] += off_s[lane];  // this wave's first slot of each expert

  // pass 2: slots.  All lanes read their expert's base before the group's
  // lowest lane advances it (the write depends on the value read; one wave's
  // LDS operations complete in order).
  for (int cb = c_begin; cb < c_end; cb += kPB) {
    int v[kPB];
    load_batch(sel, n, cb, lane, v);
#pragma unroll
    for (int j = 0; j < kPB; ++j) {
      if (cb + j >= c_end) break;
      const int a = (cb + j) * 64 + lane;
      const int my = expert_of(v[j], cb + j, lane, n, E);
      const uint64_t peers = peers_of<NB>(my);
      if (my >= 0) {
        const int b = wc[wave][my];
        const int pos = b + __popcll(peers & below);
        gather[pos] = a / k;
        scatter[a] = pos;
        slot_expert[pos] = my;
        if ((peers & below) == 0) wc[wave][my] = b + __popcll(peers);
      }
    }
  }
}

namespace {
template <int EP>
hipError_t launch_ep(const FwdArgs& a) {
  return launch(k_route_permute<EP>, dim3(1), dim3(1024), a.stream, a.ev[kSlotPermute], a.sel, a.n,
                a.dim.k, a.dim.E, a.counts, a.offsets, a.gather, a.scatter, a.slot_expert);
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
