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
// Each workgroup owns one 32-row weight tile of one expert (gate/up: one
// interleaved tile, i.e. 16 columns of d_ff; down: 32 rows of d_model); its
// eight waves split the reduction axis into eighths and combine partial sums
// through LDS in a fixed order (deterministic).  Each wave keeps a rolling
// queue of D k-steps of loads in flight, so the weight stream never drains
// between multiplies.  One tile and eight waves per workgroup put the most
// independent 1 KiB streams in flight at once: measured on the decode
// workload, gate/up 48.0 -> 43.8 us (two tiles, four waves before) and down
// 28.0 -> 22.8 us (four waves before), 6.3 and 6.1 TB/s.
//
// fp8 (E4M3) weights: a second bank holds the codes of two consecutive k-steps
// per lane and 16-byte load (1 KiB per wave-wide load, as in bf16); they are
// widened exactly to bf16 operands in registers and the per-row scales
// multiply the reduced fp32 sums.  With half the bytes per tile, four waves
// per gate/up tile stream faster than eight (decode workload: 33.9 -> 27.7 us
// with per-kernel events; two or eight waves, two tiles or a deeper queue
// were no better); the down projection keeps eight.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {
#ifndef MOE_GU_SPLIT
#define MOE_GU_SPLIT 8
#endif
constexpr int kSplit = MOE_GU_SPLIT;  // waves per gate/up weight tile (split of the reduction axis)
#ifndef MOE_GU_TILES
#define MOE_GU_TILES 1
#endif
constexpr int kGuTiles = MOE_GU_TILES;  // interleaved gate/up tiles (16 columns each) per workgroup
#ifndef MOE_DOWN_SPLIT
#define MOE_DOWN_SPLIT 8
#endif
constexpr int kSplitD = MOE_DOWN_SPLIT;  // waves per down-projection tile
#ifndef MOE_GU_TILES_FP8
#define MOE_GU_TILES_FP8 1
#endif
#ifndef MOE_GU_SPLIT_FP8
#define MOE_GU_SPLIT_FP8 4
#endif
#ifndef MOE_DOWN_SPLIT_FP8
#define MOE_DOWN_SPLIT_FP8 8
#endif
// fp8 weights: tiles and waves per workgroup of the two streams
constexpr int kGuTiles8 = MOE_GU_TILES_FP8, kSplit8 = MOE_GU_SPLIT_FP8;
constexpr int kSplitD8 = MOE_DOWN_SPLIT_FP8;
#ifndef MOE_STREAM_NT
#define MOE_STREAM_NT 1
#endif

__device__ __forceinline__ u32x4 ldw8(const uint8_t* p) {
#if MOE_STREAM_NT
  return ldg16_stream(p);
#else
  return ldg16(p);
#endif
}
__device__ __forceinline__ u32x4 ldw(const uint16_t* p) {
#if MOE_STREAM_NT
  return ldg16_stream(p);
#else
  return ldg16(p);
#endif
}

// Partial sums of waves 1..S-1 -> wave 0, fixed order.
template <int NACC, int S>
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
    for (int w = 1; w < S; ++w)
#pragma unroll
      for (int q = 0; q < NACC; ++q)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[q][i] += red[(((w - 1) * NACC + q) * 16 + i) * 64 + lane];
  }
  __syncthreads();
}

// Dispatch of a decode-sized batch (n = T*k <= 64 assignments) for expert e,
// computed by wave 0 from the routing choice itself: the expert's slot count
// and offset (popcounts of two ballots) and its tokens in slot order (stable:
// increasing assignment index) in `list`.  With `write`, the workgroup also
// stores expert e's part of the routing outputs.  Every workgroup of both
// expert kernels derives the same arrays, so no separate dispatch kernel runs.
struct Route {
  int cnt, off;
};
__device__ __forceinline__ Route small_dispatch(const int* __restrict__ sel, int n, int k, int E,
                                                int e, int lane, int wave, int* list, int* sh,
                                                bool write, int* __restrict__ counts,
                                                int* __restrict__ offsets,
                                                int* __restrict__ gather,
                                                int* __restrict__ scatter) {
  if (wave == 0) {
    const int my = lane < n ? sel[lane] : -1;
    const uint64_t me = __ballot(my == e);
    const uint64_t lt = __ballot(my >= 0 && my < e);
    const int cnt = __popcll(me), off = __popcll(lt);
    if (my == e) {
      const int r = __popcll(me & ((1ull << lane) - 1ull));
      list[r] = lane / k;
      if (write) {
        gather[off + r] = lane / k;
        scatter[lane] = off + r;
      }
    }
    if (lane == 0) {
      sh[0] = cnt;
      sh[1] = off;
      if (write) {
        counts[e] = cnt;
        offsets[e] = off;
        if (e == E - 1) offsets[E] = n;
      }
    }
  }
  __syncthreads();
  return {sh[0], sh[1]};
}

// Rolling prefetch over `kper` k-steps (a multiple of D): D k-steps of
// operands are always in flight while the oldest one is multiplied.
// NW weight streams share one activation operand per k-step.
// Lanes without a token read a row of zeros, so every load is unconditional
// (a branch around a load would make the compiler drain the queue).
template <int D, int NW>
__device__ __forceinline__ void stream_mac(const uint16_t* const (&w)[NW], const uint16_t* xb,
                                           int ks0, int kper, f32x16 (&acc)[NW]) {
  u32x4 qw[NW][D], qx[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
#pragma unroll
    for (int j = 0; j < NW; ++j) qw[j][i] = ldw(w[j] + (size_t)(ks0 + i) * kBlockElems);
    qx[i] = ldg16(xb + (ks0 + i) * kKStep);
  }
  const int rounds = kper / D;
  for (int r = 1; r < rounds; ++r) {
    const int sn = ks0 + r * D;
#pragma unroll
    for (int i = 0; i < D; ++i) {
#pragma unroll
      for (int j = 0; j < NW; ++j) acc[j] = mfma_32x32x16(qw[j][i], qx[i], acc[j]);
#pragma unroll
      for (int j = 0; j < NW; ++j) qw[j][i] = ldw(w[j] + (size_t)(sn + i) * kBlockElems);
      qx[i] = ldg16(xb + (sn + i) * kKStep);
    }
  }
#pragma unroll
  for (int i = 0; i < D; ++i)
#pragma unroll
    for (int j = 0; j < NW; ++j) acc[j] = mfma_32x32x16(qw[j][i], qx[i], acc[j]);
}
// The same stream over an fp8 (E4M3) bank: each 16-byte load of a lane holds
// its codes for two consecutive k-steps (k-step pairs p, 1 KiB per wave-wide
// load), converted exactly to bf16 operands in registers; D2 pairs in flight.
template <int D2, int NW>
__device__ __forceinline__ void stream_mac_fp8(const uint8_t* const (&w)[NW], const uint16_t* xb,
                                               int ks0, int kper, f32x16 (&acc)[NW]) {
  u32x4 qw[NW][D2], qx[D2][2];
  const int p0 = ks0 / 2;
#pragma unroll
  for (int i = 0; i < D2; ++i) {
#pragma unroll
    for (int j = 0; j < NW; ++j) qw[j][i] = ldw8(w[j] + (size_t)(p0 + i) * 1024);
    qx[i][0] = ldg16(xb + (ks0 + 2 * i) * kKStep);
    qx[i][1] = ldg16(xb + (ks0 + 2 * i + 1) * kKStep);
  }
  const int rounds = kper / (2 * D2);
  for (int r = 1; r < rounds; ++r) {
    const int pn = p0 + r * D2;
#pragma unroll
    for (int i = 0; i < D2; ++i) {
#pragma unroll
      for (int j = 0; j < NW; ++j) {
        acc[j] = mfma_32x32x16(e4m3x8_to_bf16x8(qw[j][i][0], qw[j][i][1]), qx[i][0], acc[j]);
        acc[j] = mfma_32x32x16(e4m3x8_to_bf16x8(qw[j][i][2], qw[j][i][3]), qx[i][1], acc[j]);
      }
#pragma unroll
      for (int j = 0; j < NW; ++j) qw[j][i] = ldw8(w[j] + (size_t)(pn + i) * 1024);
      qx[i][0] = ldg16(xb + 2 * (pn + i) * kKStep);
      qx[i][1] = ldg16(xb + (2 * (pn + i) + 1) * kKStep);
    }
  }
#pragma unroll
  for (int i = 0; i < D2; ++i)
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      acc[j] = mfma_32x32x16(e4m3x8_to_bf16x8(qw[j][i][0], qw[j][i][1]), qx[i][0], acc[j]);
      acc[j] = mfma_32x32x16(e4m3x8_to_bf16x8(qw[j][i][2], qw[j][i][3]), qx[i][1], acc[j]);
    }
}

// acc element i of a 32-row tile holds row c32_row(i, lane): multiply each by
// its row's scale (rows 8g + 4*(lane/32) + 0..3 are contiguous, g = 0..3).
__device__ __forceinline__ void scale_rows(f32x16& acc, const float* __restrict__ rs, int lane) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(rs + 8 * g + 4 * (lane >> 5));
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[4 * g + t] *= v[t];
  }
}
}  // namespace

// Gate/up projections and the SiLU(gate) * up epilogue for 16*NT columns of d_ff
// (NT interleaved tiles, S waves splitting the reduction axis).
// The workgroups with ft == 0 also write the routing outputs of their expert.
template <int D, bool FP8, int NT, int S>
__global__ __launch_bounds__(64 * S) void k_gateup_stream(
    const uint16_t* __restrict__ wgu, const uint8_t* __restrict__ wgu8,
    const float* __restrict__ sgu, const uint16_t* __restrict__ xn,
    const int* __restrict__ sel, int n, int k, int E, int* __restrict__ counts,
    int* __restrict__ offsets, int* __restrict__ gather, int* __restrict__ scatter,
    const float* __restrict__ inv, const uint16_t* __restrict__ zrow,
    uint16_t* __restrict__ act, int d, int F) {
  __shared__ float red[(S - 1) * NT * 16 * 64];
  __shared__ int list[64];
  __shared__ int sh[2];
  const int e = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const Route rt = small_dispatch(sel, n, k, E, e, lane, wave, list, sh, blockIdx.x == 0, counts,
                                  offsets, gather, scatter);
  const int cnt = rt.cnt, off = rt.off;
  if (cnt == 0) return;
  const int ft = blockIdx.x;
  const int ksteps = d / kKStep;
  const int kper = ksteps / S;
  const int ks0 = wave * kper;
  const size_t tile_elems = (size_t)ksteps * kBlockElems;
  // the NT interleaved gate/up tiles of columns 16*NT*ft ..
  const uint16_t* wg =
      wgu + ((size_t)e * (2 * F / kTileRows) + NT * ft) * tile_elems + lane * 8;
  const uint16_t* wp[NT];
  const uint8_t* wp8[NT];
#pragma unroll
  for (int q = 0; q < NT; ++q) {
    wp[q] = wg + q * tile_elems;
    // fp8 bank: same tile order, half the bytes per tile
    wp8[q] = FP8 ? wgu8 + (((size_t)e * (2 * F / kTileRows) + NT * ft + q) * tile_elems +
                           lane * 16) : nullptr;
  }
  const int col = lane & 31;

  for (int c0 = 0; c0 < cnt; c0 += 32) {
    const int ntok = min(32, cnt - c0);
    const bool valid = col < ntok;
    const int tok = valid ? list[c0 + col] : 0;
    const uint16_t* xrow = (valid ? xn + (size_t)tok * d : zrow) + (lane >> 5) * 8;
    f32x16 acc[NT];
#pragma unroll
    for (int q = 0; q < NT; ++q)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[q][i] = 0.f;
    if constexpr (FP8) stream_mac_fp8<D, NT>(wp8, xrow, ks0, kper, acc);
    else stream_mac<D, NT>(wp, xrow, ks0, kper, acc);
    reduce_split<NT, S>(acc, red, wave, lane);
    if constexpr (FP8) {
      if (wave == 0) {
#pragma unroll
        for (int q = 0; q < NT; ++q)
          scale_rows(acc[q], sgu + (size_t)e * 2 * F + 32 * (NT * ft + q), lane);
      }
    }

    if (wave == 0 && valid) {
      // tile q covers columns 16*(NT*ft + q) ..: gate(f) in element i, up(f) in i + 8
      const float s = inv[tok];  // RMSNorm scale of this token
      uint16_t* dst = act + (size_t)(off + c0 + col) * F + ft * 16 * NT + 4 * (lane >> 5);
#pragma unroll
      for (int q = 0; q < NT; ++q)
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          float v4[4];
#pragma unroll
          for (int t = 0; t < 4; ++t)
            v4[t] = silu(s * acc[q][4 * g + t]) * (s * acc[q][4 * g + 8 + t]);
          u32x2 v;
          v[0] = pack_bf16x2(v4[0], v4[1]);
          v[1] = pack_bf16x2(v4[2], v4[3]);
          *reinterpret_cast<u32x2*>(dst + 16 * q + 8 * g) = v;
        }
    }
  }
}

// Down projection for one 32-row d_model tile; k = 1 writes gate * y into the
// output row of the token, k > 1 writes y (fp32) for the combine kernel.
// SD waves split the reduction axis.
template <int D, bool FP8, int SD>
__global__ __launch_bounds__(64 * SD) void k_down_stream(
    const uint16_t* __restrict__ wd, const uint8_t* __restrict__ wd8,
    const float* __restrict__ sd, const uint16_t* __restrict__ act,
    const int* __restrict__ sel, int n, int k, int E, const float* __restrict__ gate,
    const uint16_t* __restrict__ zrow, uint16_t* __restrict__ out, float* __restrict__ ybuf, int d,
    int F) {
  __shared__ float red[(SD - 1) * 16 * 64];
  __shared__ int list[64];
  __shared__ int sh[2];
  const int e = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const Route rt = small_dispatch(sel, n, k, E, e, lane, wave, list, sh, false, nullptr, nullptr,
                                  nullptr, nullptr);
  const int cnt = rt.cnt, off = rt.off;
  if (cnt == 0) return;
  const int mt = blockIdx.x;
  const int ksteps = F / kKStep;
  const int kper = ksteps / SD;
  const int ks0 = wave * kper;
  const uint16_t* const wp[1] = {
      wd + ((size_t)e * (d / kTileRows) + mt) * (size_t)ksteps * kBlockElems + lane * 8};
  const uint8_t* const wp8[1] = {
      FP8 ? wd8 + ((size_t)e * (d / kTileRows) + mt) * (size_t)ksteps * kBlockElems + lane * 16
          : nullptr};
  const int col = lane & 31;

  for (int c0 = 0; c0 < cnt; c0 += 32) {
    const int ntok = min(32, cnt - c0);
    const bool valid = col < ntok;
    const int slot = off + c0 + (valid ? col : 0);
    const uint16_t* arow = (valid ? act + (size_t)slot * F : zrow) + (lane >> 5) * 8;
    f32x16 acc[1];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[0][i] = 0.f;
    if constexpr (FP8) stream_mac_fp8<D, 1>(wp8, arow, ks0, kper, acc);
    else stream_mac<D, 1>(wp, arow, ks0, kper, acc);
    reduce_split<1, SD>(acc, red, wave, lane);
    if constexpr (FP8) {
      if (wave == 0) scale_rows(acc[0], sd + (size_t)e * d + mt * kTileRows, lane);
    }

    if (wave == 0 && valid) {
      const int m0 = mt * kTileRows;
      if (k == 1) {
        const int tok = list[c0 + col];
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

namespace {
#ifndef MOE_STREAM_DEPTH
#define MOE_STREAM_DEPTH 4
#endif
#ifndef MOE_STREAM_DEPTH_FP8
#define MOE_STREAM_DEPTH_FP8 4
#endif
// Largest prefetch depth (k-steps, or k-step pairs for fp8) up to dmax that
// divides a wave's share.
int pick_depth(int kper, int dmax) {
  for (int D = dmax; D > 1; D /= 2)
    if (kper % D == 0) return D;
  return 1;
}
}  // namespace

namespace {
template <bool FP8, int NT, int S, int SD>
hipError_t launch_streams(const FwdArgs& a) {
  const int d = a.dim.d, F = a.dim.F, E = a.dim.E;
  // queue depth: k-steps (bf16) or k-step pairs (fp8) in flight per wave
  const int dmax = FP8 ? MOE_STREAM_DEPTH_FP8 : MOE_STREAM_DEPTH;
  const int Da = pick_depth(d / kKStep / S / (FP8 ? 2 : 1), dmax);
  const int Db = pick_depth(F / kKStep / SD / (FP8 ? 2 : 1), dmax);
  auto gu = Da == 8 ? k_gateup_stream<8, FP8, NT, S> : Da == 4 ? k_gateup_stream<4, FP8, NT, S>
          : Da == 2 ? k_gateup_stream<2, FP8, NT, S> : k_gateup_stream<1, FP8, NT, S>;
  auto dn = Db == 8 ? k_down_stream<8, FP8, SD> : Db == 4 ? k_down_stream<4, FP8, SD>
          : Db == 2 ? k_down_stream<2, FP8, SD> : k_down_stream<1, FP8, SD>;
  hipError_t err = launch(gu, dim3(F / (16 * NT), E), dim3(64 * S), a.stream,
                          a.ev[kSlotExpertsA], (const uint16_t*)a.wgu, (const uint8_t*)a.wgu8,
                          a.sgu, (const uint16_t*)a.xn, (const int*)a.sel, a.n, a.dim.k, E,
                          a.counts, a.offsets, a.gather, a.scatter, (const float*)a.inv,
                          (const uint16_t*)a.zrow, (uint16_t*)a.act, d, F);
  if (err != hipSuccess) return err;
  return launch(dn, dim3(d / kTileRows, E), dim3(64 * SD), a.stream, a.ev[kSlotExpertsB],
                (const uint16_t*)a.wd, (const uint8_t*)a.wd8, a.sd, (const uint16_t*)a.act,
                (const int*)a.sel, a.n, a.dim.k, E, (const float*)a.gate,
                (const uint16_t*)a.zrow, (uint16_t*)a.out, a.ybuf, d, F);
}
}  // namespace

hipError_t launch_experts_stream(const FwdArgs& a) {
  return a.wgu8 != nullptr ? launch_streams<true, kGuTiles8, kSplit8, kSplitD8>(a)
                           : launch_streams<false, kGuTiles, kSplit, kSplitD>(a);
}

}  // namespace moe
