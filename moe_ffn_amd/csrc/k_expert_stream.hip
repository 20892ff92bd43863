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
// through LDS in a fixed order (deterministic); the reduction and the
// epilogue are spread over the eight waves (each sums and stores its own
// share of the tile's elements), which took the decode gate/up launch from
// 43.8 to 42.4 us.  Each wave keeps a rolling
// queue of D k-steps of loads in flight, so the weight stream never drains
// between multiplies.  One tile and eight waves per workgroup put the most
// independent 1 KiB streams in flight at once: measured on the decode
// workload, gate/up 48.0 -> 43.8 us (two tiles, four waves before) and down
// 28.0 -> 22.8 us (four waves before), 6.3 and 6.1 TB/s.
//
// fp8 weights and fp8 activations (decode batches of layers made by
// moe_layer_create_w8a8): the router leaves the E4M3 values of the expert
// inputs (exact in bf16) and their row scales, which the gate/up stream takes
// in place of inv_rms; the activation rows are quantised in place between the
// two streams, and the down stream also multiplies its sums by their scales
// (asc), so both streams multiply exact E4M3 values.
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
constexpr int kSplit = 8;     // waves per gate/up weight tile (split of the reduction axis)
constexpr int kGuTiles = 1;   // interleaved gate/up tiles (16 columns each) per workgroup
constexpr int kSplitD = 8;    // waves per down-projection tile
// fp8 weights: tiles and waves per workgroup of the two streams
constexpr int kGuTiles8 = 1, kSplit8 = 4;
constexpr int kSplitD8 = 8;
// prefetch depth of the weight queues (k-steps; k-step pairs for fp8), at most
constexpr int kStreamDepth = 4;
constexpr int kStreamDepth8 = 4;

// A workgroup's weight tiles read as one raw buffer: the base and range in
// scalar registers, the tile and 1 KiB block as the scalar offset and the
// lane's 16 bytes as the one vector offset all loads share (no 64-bit vector
// address per load); non-temporal, as each byte is read once.
struct WTiles {
  __amdgpu_buffer_rsrc_t r;
  int voff, tile_bytes;
  __device__ __forceinline__ u32x4 operator()(int j, int blk) const {
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, j * tile_bytes + blk * 1024, 2);
  }
};
__device__ __forceinline__ WTiles wtiles(const void* base, int ntiles, int tile_bytes, int lane) {
  return {__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, ntiles * tile_bytes,
                                            0x00020000),
          lane * 16, tile_bytes};
}
// The same tiles through plain non-temporal global loads (the lane's 16 bytes
// applied to the pointer): the down streams, which timed no faster through
// the buffer form.
struct WPtr {
  const char* p;
  int tile_bytes;
  __device__ __forceinline__ u32x4 operator()(int j, int blk) const {
    return ldg16_stream(p + (size_t)j * tile_bytes + (size_t)blk * 1024);
  }
};

// Split-K reduction spread over the waves: every wave parks its NACC
// accumulator tiles in LDS; after a barrier, element i of tile q summed over
// the S waves in wave order (so the sum does not depend on which wave reads it)
// is read back by the wave that owns that element's epilogue.
template <int NACC>
__device__ __forceinline__ void stash(const f32x16 (&acc)[NACC], float* red, int wave, int lane) {
#pragma unroll
  for (int q = 0; q < NACC; ++q)
#pragma unroll
    for (int i = 0; i < 16; ++i) red[((wave * NACC + q) * 16 + i) * 64 + lane] = acc[q][i];
}
template <int NACC, int S>
__device__ __forceinline__ float split_sum(const float* red, int q, int i, int lane) {
  float v = red[(q * 16 + i) * 64 + lane];
#pragma unroll
  for (int w = 1; w < S; ++w) v += red[((w * NACC + q) * 16 + i) * 64 + lane];
  return v;
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

// Token operands of the fp8 weight streams: the lane's 16 bytes of k-step ks.
// BGlobal reads them from the token's row in memory (zrow for lanes without a
// token).  BLds reads the wave's LDS copy of its k-range of the pass's token
// rows (stage_b); lanes without a token read the wave's zero piece at stride
// 0, so no branch or select sits between an LDS read and its MFMA.  With half
// the weight bytes per k-step, the fp8 gate/up stream is the one these loads
// slow: a timing copy without any token loads ran it in 24.8 instead of 26.3
// us; staging them in LDS, 25.9 (the fp8 down stream, whose waves stream
// fewer k-steps, and the bf16 streams were no faster with it).
struct BGlobal {
  const uint16_t* xb;  // the lane's row, k-group offset applied
  __device__ __forceinline__ u32x4 operator()(int ks) const { return ldg16(xb + ks * kKStep); }
};
struct BLds {
  const u32x4* b;  // the lane's piece (token, k-step ks0, k-group), or the zero piece
  int ks0, step;   // step: 2 pieces per k-step, 0 for the zero piece
  __device__ __forceinline__ u32x4 operator()(int ks) const { return b[(ks - ks0) * step]; }
};

// LDS pieces a wave can stage for one pass (its slice of the split-K buffer,
// idle during the stream): 256 x 16 bytes per accumulator tile.
constexpr int kStagePieces = 256;

// Copy the wave's k-range [ks0, ks0 + kper) of ntok token rows (row t starts at
// rowp(t)) into bl: piece (t, s, g), the 8 values k = 16 (ks0 + s) + 8 g .. +7,
// at bl[(t * kper + s) * 2 + g]; ntok * 2 * kper <= NP pieces.  Branch-free:
// lanes past the last piece load and store the last piece again (the same
// bytes), so all loads issue together behind the weights in flight.  The same
// wave reads the pieces back (one wave's LDS operations run in order).
template <int NP, class RowP>
__device__ __forceinline__ void stage_b(u32x4* bl, const RowP& rowp, int ntok, int ks0, int kper,
                                        int lane) {
  const int per = 2 * kper, total = ntok * per;
  int c[NP / 64];
  const uint16_t* src[NP / 64];
#pragma unroll
  for (int it = 0; it < NP / 64; ++it) {
    c[it] = min(lane + 64 * it, total - 1);
    src[it] = rowp(c[it] / per) + (size_t)ks0 * kKStep + (c[it] % per) * 8;
  }
  u32x4 v[NP / 64];
#pragma unroll
  for (int it = 0; it < NP / 64; ++it) v[it] = ldg16(src[it]);
#pragma unroll
  for (int it = 0; it < NP / 64; ++it) bl[c[it]] = v[it];
}

// Rolling prefetch over `kper` k-steps (a multiple of D): D k-steps of
// operands are always in flight while the oldest one is multiplied.
// NW weight streams share one activation operand per k-step.
// Lanes without a token read a row of zeros, so every load is unconditional
// (a branch around a load would make the compiler drain the queue).
template <int D, int NW, class W>
__device__ __forceinline__ void stream_mac(const W& w, const uint16_t* xb,
                                           int ks0, int kper, f32x16 (&acc)[NW]) {
  u32x4 qw[NW][D], qx[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
#pragma unroll
    for (int j = 0; j < NW; ++j) qw[j][i] = w(j, ks0 + i);
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
      for (int j = 0; j < NW; ++j) qw[j][i] = w(j, sn + i);
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
template <int D2, int NW, class W, class BS, class Pre>
__device__ __forceinline__ void stream_mac_fp8(const W& w, const BS& xb,
                                               int ks0, int kper, f32x16 (&acc)[NW],
                                               const Pre& pre) {
  u32x4 qw[NW][D2], qx[D2][2];
  const int p0 = ks0 / 2;
#pragma unroll
  for (int i = 0; i < D2; ++i)
#pragma unroll
    for (int j = 0; j < NW; ++j) qw[j][i] = w(j, p0 + i);
  pre();  // with the first weights in flight (the LDS form stages its token rows here)
#pragma unroll
  for (int i = 0; i < D2; ++i) {
    qx[i][0] = xb(ks0 + 2 * i);
    qx[i][1] = xb(ks0 + 2 * i + 1);
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
      for (int j = 0; j < NW; ++j) qw[j][i] = w(j, pn + i);
      qx[i][0] = xb(2 * (pn + i));
      qx[i][1] = xb(2 * (pn + i) + 1);
      __builtin_amdgcn_sched_barrier(0);  // refill each slot right after its multiplies
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

}  // namespace

// Gate/up projections and the SiLU(gate) * up epilogue for 16*NT columns of d_ff
// (NT interleaved tiles, S waves splitting the reduction axis).
// The workgroups with ft == 0 also write the routing outputs of their expert.
template <int D, bool FP8, int NT, int S>
__global__ __launch_bounds__(64 * S, 1) void k_gateup_stream(
    const uint16_t* __restrict__ wgu, const uint8_t* __restrict__ wgu8,
    const float* __restrict__ sgu, const uint16_t* __restrict__ xn,
    const int* __restrict__ sel, int n, int k, int E, int* __restrict__ counts,
    int* __restrict__ offsets, int* __restrict__ gather, int* __restrict__ scatter,
    const float* __restrict__ inv, const uint16_t* __restrict__ zrow,
    uint16_t* __restrict__ act, int d, int F) {
  __shared__ float red[S * NT * 16 * 64];
  __shared__ int list[64];
  __shared__ int sh[2];
  __shared__ u32x4 zp[S];  // fp8: each wave's zero token piece
  const int e = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (FP8 && lane == 0) zp[wave] = u32x4{0u, 0u, 0u, 0u};
  const Route rt = small_dispatch(sel, n, k, E, e, lane, wave, list, sh, blockIdx.x == 0, counts,
                                  offsets, gather, scatter);
  const int cnt = rt.cnt, off = rt.off;
  if (cnt == 0) return;
  const int ft = blockIdx.x;
  const int ksteps = d / kKStep;
  const int kper = ksteps / S;
  const int ks0 = wave * kper;
  const size_t tile_elems = (size_t)ksteps * kBlockElems;
  // the NT interleaved gate/up tiles of columns 16*NT*ft .. (fp8 bank: same
  // tile order, half the bytes per tile)
  const size_t t0 = (size_t)e * (2 * F / kTileRows) + NT * ft;
  const WTiles wt = FP8 ? wtiles(wgu8 + t0 * tile_elems, NT, (int)tile_elems, lane)
                        : wtiles(wgu + t0 * tile_elems, NT, (int)tile_elems * 2, lane);
  const int col = lane & 31;
  // fp8 weights: the row scales of this lane's epilogue elements, loaded
  // before the stream so that their latency hides under it (the S waves take
  // the NT * 8 (gate, up) pairs in turn)
  constexpr int NPL = (NT * 8 + S - 1) / S;
  float sgl[NPL], sul[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int p = wave + j * S;
    sgl[j] = sul[j] = 1.f;
    if (FP8 && p < NT * 8) {  // gate rows 0..15, up rows 16..31 of the tile
      const float* sc = sgu + (size_t)e * 2 * F + 32 * (NT * ft + (p >> 3));
      sgl[j] = sc[c32_row(p & 7, lane)];
      sul[j] = sc[16 + c32_row(p & 7, lane)];
    }
  }

  for (int c0 = 0; c0 < cnt; c0 += 32) {
    const int ntok = min(32, cnt - c0);
    const bool valid = col < ntok;
    const int tok = valid ? list[c0 + col] : 0;
    const uint16_t* xrow = (valid ? xn + (size_t)tok * d : zrow) + (lane >> 5) * 8;
    const float rs = valid ? inv[tok] : 0.f;  // RMSNorm scale of this token
    f32x16 acc[NT];
#pragma unroll
    for (int q = 0; q < NT; ++q)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[q][i] = 0.f;
    if constexpr (FP8) {
      if (ntok * 2 * kper <= NT * kStagePieces) {  // token operands from LDS
        u32x4* bl = reinterpret_cast<u32x4*>(red + wave * NT * 16 * 64);
        const auto pre = [&] {
          stage_b<NT * kStagePieces>(
              bl, [&](int t) { return xn + (size_t)list[c0 + t] * d; }, ntok, ks0, kper, lane);
        };
        const BLds bs{valid ? bl + col * 2 * kper + (lane >> 5) : zp + wave, ks0, valid ? 2 : 0};
        stream_mac_fp8<D, NT>(wt, bs, ks0, kper, acc, pre);
      } else {
        stream_mac_fp8<D, NT>(wt, BGlobal{xrow}, ks0, kper, acc, [] {});
      }
    } else {
      stream_mac<D, NT>(wt, xrow, ks0, kper, acc);
    }
    stash<NT>(acc, red, wave, lane);
    __syncthreads();
    // gate(f) is element i of tile q, up(f) element i + 8, f = 16 (NT ft + q) +
    // c32_row(i, lane); the S waves take the NT * 8 (gate, up) pairs in turn
    uint16_t* dst = act + (size_t)(off + c0 + col) * F + ft * 16 * NT;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int p = wave + j * S;
      if (p >= NT * 8) break;
      const int q = p >> 3, i = p & 7, f = c32_row(i, lane);
      float g = split_sum<NT, S>(red, q, i, lane);
      float u = split_sum<NT, S>(red, q, i + 8, lane);
      if constexpr (FP8) {
        g *= sgl[j];
        u *= sul[j];
      }
      if (valid) dst[16 * q + f] = (uint16_t)f32_to_bf16(silu(rs * g) * (rs * u));
    }
    __syncthreads();  // red is reused by the next pass over the tokens
  }
}

// Down projection for one 32-row d_model tile; k = 1 writes gate * y into the
// output row of the token (in a stack, bf16(res + bf16(gate * y))), k > 1
// writes y (fp32) for the combine kernel.
// SD waves split the reduction axis.
template <int D, bool FP8, int SD>
__global__ __launch_bounds__(64 * SD, 1) void k_down_stream(
    const uint16_t* __restrict__ wd, const uint8_t* __restrict__ wd8,
    const float* __restrict__ sd, const uint16_t* __restrict__ act,
    const int* __restrict__ sel, int n, int k, int E, const float* __restrict__ gate,
    const float* __restrict__ asc, const uint16_t* __restrict__ zrow, uint16_t* __restrict__ out,
    const uint16_t* __restrict__ res, float* __restrict__ ybuf, int d, int F) {
  __shared__ float red[SD * 16 * 64];
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
  const size_t tile_elems = (size_t)ksteps * kBlockElems, t0 = (size_t)e * (d / kTileRows) + mt;
  const WPtr wt = FP8 ? WPtr{reinterpret_cast<const char*>(wd8 + t0 * tile_elems) + lane * 16,
                             (int)tile_elems}
                      : WPtr{reinterpret_cast<const char*>(wd + t0 * tile_elems) + lane * 16,
                             (int)tile_elems * 2};
  const int col = lane & 31;
  const int m0 = mt * kTileRows;
  // fp8 weights: the row scales of this lane's epilogue rows (the SD waves
  // take the 16 accumulator elements in turn), loaded before the stream
  constexpr int NEL = (16 + SD - 1) / SD;
  float sdl[NEL];
#pragma unroll
  for (int j = 0; j < NEL; ++j) {
    const int i = wave + j * SD;
    sdl[j] = FP8 && i < 16 ? sd[(size_t)e * d + m0 + c32_row(i, lane)] : 1.f;
  }

  for (int c0 = 0; c0 < cnt; c0 += 32) {
    const int ntok = min(32, cnt - c0);
    const bool valid = col < ntok;
    const int slot = off + c0 + (valid ? col : 0);
    const uint16_t* arow = (valid ? act + (size_t)slot * F : zrow) + (lane >> 5) * 8;
    const int tok = (k == 1 && valid) ? list[c0 + col] : 0;
    const float gw = (k == 1 && valid) ? gate[tok] : 0.f;
    const float as = FP8 && asc != nullptr ? asc[slot] : 1.f;  // fp8 activations: the row's scale
    // in a stack (res, k = 1): the residual stream's values of this lane's
    // output elements, loaded before the stream (lanes without a token read zrow)
    uint16_t hres[NEL];
#pragma unroll
    for (int j = 0; j < NEL; ++j) {
      const int i = wave + j * SD;
      const bool use = res != nullptr && k == 1 && valid && i < 16;
      hres[j] = *(use ? res + (size_t)tok * d + m0 + c32_row(i, lane) : zrow);
    }
    f32x16 acc[1];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[0][i] = 0.f;
    if constexpr (FP8) stream_mac_fp8<D, 1>(wt, BGlobal{arow}, ks0, kper, acc, [] {});
    else stream_mac<D, 1>(wt, arow, ks0, kper, acc);
    stash<1>(acc, red, wave, lane);
    __syncthreads();
    // the SD waves take the 16 accumulator elements (rows m0 + c32_row(i, lane)) in turn
#pragma unroll
    for (int j = 0; j < NEL; ++j) {
      const int i = wave + j * SD;
      if (i >= 16) break;
      const int r = c32_row(i, lane);
      float y = split_sum<1, SD>(red, 0, i, lane);
      if constexpr (FP8) y = (y * sdl[j]) * as;
      if (valid) {
        if (k == 1) {
          const uint32_t o = f32_to_bf16(gw * y);
          out[(size_t)tok * d + m0 + r] =
              (uint16_t)(res != nullptr ? f32_to_bf16(bf16_lo(hres[j]) + bf16_lo(o)) : o);
        } else {
          ybuf[(size_t)slot * d + m0 + r] = y;
        }
      }
    }
    __syncthreads();  // red is reused by the next pass over the tokens
  }
}

namespace {
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
  const int dmax = FP8 ? kStreamDepth8 : kStreamDepth;
  const int Da = pick_depth(d / kKStep / S / (FP8 ? 2 : 1), dmax);
  const int Db = pick_depth(F / kKStep / SD / (FP8 ? 2 : 1), dmax);
  auto gu = Da == 8 ? k_gateup_stream<8, FP8, NT, S> : Da == 4 ? k_gateup_stream<4, FP8, NT, S>
          : Da == 2 ? k_gateup_stream<2, FP8, NT, S> : k_gateup_stream<1, FP8, NT, S>;
  auto dn = Db == 8 ? k_down_stream<8, FP8, SD> : Db == 4 ? k_down_stream<4, FP8, SD>
          : Db == 2 ? k_down_stream<2, FP8, SD> : k_down_stream<1, FP8, SD>;
  // fp8 activations: the router's row scales take inv_rms's place
  const float* rs = a.dim.act8 ? a.xs_tok : a.inv;
  hipError_t err = launch(gu, dim3(F / (16 * NT), E), dim3(64 * S), a.stream,
                          a.ev[kSlotExpertsA], (const uint16_t*)a.wgu, (const uint8_t*)a.wgu8,
                          a.sgu, (const uint16_t*)a.xn, (const int*)a.sel, a.n, a.dim.k, E,
                          a.counts, a.offsets, a.gather, a.scatter, rs,
                          (const uint16_t*)a.zrow, (uint16_t*)a.act, d, F);
  if (err != hipSuccess) return err;
  if (a.dim.act8) {
    err = launch_quant_act_rows(a);
    if (err != hipSuccess) return err;
  }
  return launch(dn, dim3(d / kTileRows, E), dim3(64 * SD), a.stream, a.ev[kSlotExpertsB],
                (const uint16_t*)a.wd, (const uint8_t*)a.wd8, a.sd, (const uint16_t*)a.act,
                (const int*)a.sel, a.n, a.dim.k, E, (const float*)a.gate,
                (const float*)(a.dim.act8 ? a.sm : nullptr), (const uint16_t*)a.zrow,
                (uint16_t*)a.out, (const uint16_t*)a.res, a.ybuf, d, F);
}
}  // namespace

hipError_t launch_experts_stream(const FwdArgs& a) {
  return a.wgu8 != nullptr ? launch_streams<true, kGuTiles8, kSplit8, kSplitD8>(a)
                           : launch_streams<false, kGuTiles, kSplit, kSplitD>(a);
}

}  // namespace moe
