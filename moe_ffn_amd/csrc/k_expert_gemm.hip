// K3 (prefill shapes): grouped SwiGLU GEMMs over the experts, both operands
// staged through LDS.
//
// Expert FFN y = W_down (SiLU(W_gate x) * (W_up x)) per routed assignment
// (SwiGLU: GLU variants paper on the ZONOS2 report's "Builds on" list; 16
// experts per layer, digest item 5).  Two launches:
//   MODE 0  act[slot, f] = bf16( SiLU(inv * x W_gate^T) * (inv * x W_up^T) )   K = d_model
//   MODE 1  y[slot, m]   = act[slot] W_down^T                                    K = d_ff
//           k = 1: out[token] = bf16(gate * y); k > 1: y kept in fp32.
//
// Work unit: (expert, block of 64*RT weight rows, span of at most 320 of the
// expert's slots).  An expert's slots are cut into the fewest spans of at most
// ten 32-token subtiles, split evenly, so a unit usually holds all of an
// expert's tokens at prefill sizes and every weight byte is read once.
//
// Workgroup: four waves, one per SIMD, as 2 row groups x 2 token groups; a
// wave owns RT 32-row tiles against TT 32-token subtiles (RT*TT accumulators
// of 32x32 fp32).  Both operands are stored as 1 KiB MFMA operand blocks: the
// weights in the packed bank, the tokens in expert-ordered subtiles (gate/up:
// the gathered rows of k_gather_tiles.hip; down: the activations, which the
// gate/up epilogue writes in that layout).  Every wave-wide load therefore
// reads one contiguous KiB (8 full cache lines), which is what keeps the
// L2-to-CU stream fast (16-row gathers of 64 bytes each ran at well under half
// its rate).  Per 32-wide k stage the workgroup copies the blocks into one of
// three LDS stages (slot = lane, conflict-free both ways); two stages of
// global loads are in flight in registers.  The barrier of a stage is passed
// with the next stage's first operands already in registers, so the MFMA pipe
// does not wait on it.
//
// Gate/up rows are packed as 32-row tiles of 16 gate rows followed by the 16
// up rows of the same columns, so the lane that holds gate(f) in accumulator
// element i holds up(f) in element i + 8 and the SiLU * up epilogue needs no
// exchange between lanes.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {
constexpr int kSub = 32;             // tokens per MFMA subtile
constexpr int kTTMax = 5;            // token subtiles per wave, at most
constexpr int kSubCap = 2 * kTTMax;  // token subtiles per work unit
constexpr int kStages = 3;           // LDS stages
constexpr int kStageK = 32;          // k per stage (two MFMA k-steps)

template <int RT>
struct Geo {
  static constexpr int kRowTiles = 2 * RT;         // 32-row weight tiles per unit
  static constexpr int kRows = kRowTiles * 32;
  static constexpr int kABlk = kRowTiles * 2;      // weight blocks (1 KiB) per stage
  static constexpr int kBBlk = kSubCap * 2;        // token blocks per stage, at most
  static constexpr int kStageEnt = (kABlk + kBBlk) * 64;  // 16-byte LDS entries per stage
};

template <int RT, int TT>
struct Ctx {
  static constexpr int NL = RT + TT;  // wave-wide block loads per wave and stage
  const uint16_t* src[NL];            // block of stage 0 (lane offset applied)
  size_t step[NL];                    // elements from one stage to the next (0: zero block)
  int a_rd;                           // LDS entry of this wave's first weight operand
  int b_rd;                           // LDS entry of its first token operand
  int wave;
};

// Blocks of a stage: j < 4 RT are weight blocks (tile j / 2, k-step j % 2),
// the rest token blocks (subtile (j - 4 RT) / 2, k-step j % 2).  Wave w copies
// blocks w, w + 4, ...; block j sits at LDS entries j * 64 .. j * 64 + 63.
template <int RT, int TT>
__device__ __forceinline__ void gload(const Ctx<RT, TT>& c, int st, int nst,
                                      u32x4 (&r)[RT + TT]) {
  const int s = st < nst ? st : nst - 1;  // clamp: surplus loads stay in bounds
#pragma unroll
  for (int q = 0; q < RT + TT; ++q) r[q] = ldg16(c.src[q] + (size_t)s * c.step[q]);
}

template <int RT, int TT>
__device__ __forceinline__ void swrite(const Ctx<RT, TT>& c, u32x4* buf, const u32x4 (&r)[RT + TT]) {
  const int lane = lane_id();
#pragma unroll
  for (int q = 0; q < RT + TT; ++q) buf[(c.wave + 4 * q) * 64 + lane] = r[q];
}

template <int RT, int TT>
__device__ __forceinline__ void sread(const Ctx<RT, TT>& c, const u32x4* buf, int ss,
                                      u32x4 (&xa)[RT], u32x4 (&xb)[TT]) {
#pragma unroll
  for (int r = 0; r < RT; ++r) xa[r] = buf[c.a_rd + (2 * r + ss) * 64];
#pragma unroll
  for (int j = 0; j < TT; ++j) xb[j] = buf[c.b_rd + (2 * j + ss) * 64];
}

template <int RT, int TT>
__device__ __forceinline__ void mac(const u32x4 (&xa)[RT], const u32x4 (&xb)[TT],
                                    f32x16 (&acc)[RT][TT]) {
#pragma unroll
  for (int j = 0; j < TT; ++j)
#pragma unroll
    for (int r = 0; r < RT; ++r) acc[r][j] = mfma_32x32x16(xa[r], xb[j], acc[r][j]);
}

// One stage kt: MFMAs of its two k-steps; meanwhile the registers holding stage
// kt+2 go to LDS buffer (kt+2)%3 (last read in stage kt-1, released by that
// stage's barrier), the loads of stage kt+4 are issued into them, and the first
// operands of stage kt+1 (written one stage earlier) are read.  Scheduling
// barriers keep this order: the operands of a k-step are always read a whole
// k-step of MFMAs ahead of their use (masks: 0x008 MFMA, 0x100 DS read,
// 0x200 DS write, 0x020 VMEM read).
template <int RT, int TT>
__device__ __forceinline__ void stage(const Ctx<RT, TT>& c, u32x4* lds, int& buf, int kt, int nst,
                                      u32x4 (&rg)[RT + TT], u32x4 (&oa)[RT], u32x4 (&ob)[TT],
                                      f32x16 (&acc)[RT][TT]) {
  constexpr int SE = Geo<RT>::kStageEnt;
  constexpr int NL = RT + TT;             // staged 16-byte pieces per thread
  constexpr int NM = RT * TT;             // MFMAs per k-step
  const int b1 = buf == kStages - 1 ? 0 : buf + 1;
  const int b2 = b1 == kStages - 1 ? 0 : b1 + 1;
  u32x4 na[RT], nb[TT];
  sread(c, lds + buf * SE, 1, na, nb);
  __builtin_amdgcn_sched_barrier(0);
  mac(oa, ob, acc);
  swrite(c, lds + b2 * SE, rg);
  gload(c, kt + 4, nst, rg);
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i < NL) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
    else if (i < 2 * NL) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  sread(c, lds + b1 * SE, 0, oa, ob);
  mac(na, nb, acc);
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    if (i < RT + TT) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  buf = b1;
}

template <int RT, int TT>
__device__ __forceinline__ void mainloop(const Ctx<RT, TT>& c, u32x4* lds, int nst,
                                         f32x16 (&acc)[RT][TT]) {
  constexpr int SE = Geo<RT>::kStageEnt;
  u32x4 r0[RT + TT], r1[RT + TT];
  u32x4 oa[RT], ob[TT];
  gload(c, 0, nst, r0);
  gload(c, 1, nst, r1);
  swrite(c, lds, r0);
  gload(c, 2, nst, r0);
  swrite(c, lds + SE, r1);
  gload(c, 3, nst, r1);
  __syncthreads();
  sread(c, lds, 0, oa, ob);
  int buf = 0;
  for (int kt = 0; kt < nst; kt += 2) {
    stage(c, lds, buf, kt, nst, r0, oa, ob, acc);
    stage(c, lds, buf, kt + 1, nst, r1, oa, ob, acc);
  }
}

// Work unit of a workgroup, or false for a surplus workgroup.  Units are
// numbered expert-major, then weight block, then span (the spans sharing a
// weight block are adjacent), and dealt to the 8 XCDs in contiguous ranges
// (workgroup b runs on XCD b % 8) so that units sharing weights or token rows
// run at the same time under one L2.
struct Unit {
  int e, rb, slot0, nrows, nsub;
  int sub0;  // first subtile of the unit in the padded, expert-ordered subtile list
};
__device__ __forceinline__ int span_count(int cnt) {
  const int nsub = (cnt + kSub - 1) / kSub;
  return (nsub + kSubCap - 1) / kSubCap;
}
__device__ __forceinline__ bool find_unit(const int* __restrict__ counts,
                                          const int* __restrict__ offsets, int E, int nrb, Unit& u) {
  int U = 0;
  for (int e = 0; e < E; ++e) U += nrb * span_count(counts[e]);
  const int per = (U + 7) >> 3;
  const int b = blockIdx.x, i = b >> 3;
  const int L = (b & 7) * per + i;
  if (i >= per || L >= U) return false;
  int base = 0, psub = 0;
  for (int e = 0; e < E; ++e) {
    const int cnt = counts[e];
    const int ns = span_count(cnt);
    if (L < base + nrb * ns) {
      const int r = L - base;
      const int sp = r % ns;
      const int nsub = (cnt + kSub - 1) / kSub;
      const int s0 = sp * nsub / ns, s1 = (sp + 1) * nsub / ns;
      u.e = e;
      u.rb = r / ns;
      u.slot0 = offsets[e] + s0 * kSub;
      u.nrows = min(cnt, s1 * kSub) - s0 * kSub;
      u.nsub = s1 - s0;
      u.sub0 = psub + s0;
      return true;
    }
    base += nrb * ns;
    psub += (cnt + kSub - 1) / kSub;
  }
  return false;
}

template <int MODE, int RT, int TT>
__device__ __forceinline__ void run_unit(const Unit& u, u32x4* lds, const uint16_t* __restrict__ wpk,
                                         const uint16_t* __restrict__ src,
                                         const int* __restrict__ gather,
                                         const float* __restrict__ gate,
                                         const float* __restrict__ inv, int k,
                                         const uint16_t* __restrict__ zrow,
                                         uint16_t* __restrict__ dst16, float* __restrict__ ybuf,
                                         int d, int F) {
  using G = Geo<RT>;
  const int K = MODE == 0 ? d : F;
  const int nst = K / kStageK;
  const int rows_e = MODE == 0 ? 2 * F : d;  // weight rows of one expert
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rg = wave & 1, tg = wave >> 1;  // row group, token group
  const size_t tile_elems = (size_t)(K / kKStep) * kBlockElems;
  const int tile0 = u.rb * G::kRowTiles;  // first 32-row tile of the unit within the expert

  Ctx<RT, TT> c;
  c.wave = wave;
#pragma unroll
  for (int q = 0; q < RT + TT; ++q) {
    const int j = wave + 4 * q;  // block of the stage copied by this wave
    if (q < RT) {                // weight tile j / 2, k-step j % 2
      c.src[q] = wpk + ((size_t)u.e * (rows_e / kTileRows) + tile0 + (j >> 1)) * tile_elems +
                 (j & 1) * kBlockElems + lane * 8;
      c.step[q] = 2 * kBlockElems;
    } else {                     // token subtile jb / 2, k-step jb % 2
      const int jb = j - 4 * RT;
      const bool valid = (jb >> 1) < u.nsub;
      c.src[q] = valid ? src + ((size_t)(u.sub0 + (jb >> 1)) * (K / kKStep) + (jb & 1)) * kBlockElems +
                             lane * 8
                       : zrow + lane * 8;
      c.step[q] = valid ? 2 * kBlockElems : 0;
    }
  }
  c.a_rd = (2 * rg * RT) * 64 + lane;
  c.b_rd = (G::kABlk + 2 * tg * TT) * 64 + lane;

  f32x16 acc[RT][TT];
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int j = 0; j < TT; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[r][j][q] = 0.f;

  mainloop(c, lds, nst, acc);

  // epilogue
  const int col = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int j = 0; j < TT; ++j) {
    const int us = tg * TT + j;   // subtile of the unit
    const int r = us * kSub + col;  // unit row
    if constexpr (MODE == 0) {
      // activations in the down projection's operand tiles: subtile sub0 + us,
      // k-step gt (16 columns of d_ff per gate/up tile); each wave store of a
      // (tile, subtile) pair fills one whole 1 KiB block
      if (us >= u.nsub) continue;
      const float sc = r < u.nrows ? inv[gather[u.slot0 + r]] : 0.f;  // RMSNorm scale
      uint16_t* blk = dst16 + (size_t)(u.sub0 + us) * (F / kKStep) * kBlockElems;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int gt = tile0 + rg * RT + rt;  // 16 gate rows + 16 up rows: columns 16*gt ..
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          float v4[4];
#pragma unroll
          for (int t = 0; t < 4; ++t)
            v4[t] = silu(sc * acc[rt][j][4 * g + t]) * (sc * acc[rt][j][4 * g + 8 + t]);
          u32x2 v;
          v[0] = pack_bf16x2(v4[0], v4[1]);
          v[1] = pack_bf16x2(v4[2], v4[3]);
          // operand lane g*32 + col holds columns 8g .. 8g+7 of the k-step
          *reinterpret_cast<u32x2*>(blk + ((size_t)gt * 64 + g * 32 + col) * 8 + 4 * hi) = v;
        }
      }
    } else {
      if (r >= u.nrows) continue;
      const int slot = u.slot0 + r;
      const int tok = k == 1 ? gather[slot] : 0;
      const float gw = k == 1 ? gate[tok] : 0.f;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int m0 = (tile0 + rg * RT + rt) * kTileRows + 4 * hi;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int m = m0 + 8 * q;
          if (k == 1) {
            u32x2 v;
            v[0] = pack_bf16x2(gw * acc[rt][j][4 * q], gw * acc[rt][j][4 * q + 1]);
            v[1] = pack_bf16x2(gw * acc[rt][j][4 * q + 2], gw * acc[rt][j][4 * q + 3]);
            *reinterpret_cast<u32x2*>(dst16 + (size_t)tok * d + m) = v;
          } else {
            f32x4 v = {acc[rt][j][4 * q], acc[rt][j][4 * q + 1], acc[rt][j][4 * q + 2],
                       acc[rt][j][4 * q + 3]};
            *reinterpret_cast<f32x4*>(ybuf + (size_t)slot * d + m) = v;
          }
        }
      }
    }
  }
}
}  // namespace

template <int MODE, int RT>
__global__ __launch_bounds__(256, 1) void k_expert_gemm(
    const uint16_t* __restrict__ wpk, const uint16_t* __restrict__ src,
    const int* __restrict__ counts, const int* __restrict__ offsets,
    const int* __restrict__ gather, const float* __restrict__ gate,
    const float* __restrict__ inv, int k, int E, const uint16_t* __restrict__ zrow,
    uint16_t* __restrict__ dst16, float* __restrict__ ybuf, int d, int F) {
  __shared__ u32x4 lds[kStages * Geo<RT>::kStageEnt];
  const int nrb = (MODE == 0 ? 2 * F : d) / Geo<RT>::kRows;
  Unit u;
  if (!find_unit(counts, offsets, E, nrb, u)) return;
  // token subtiles per wave: the first group takes the larger half
  switch ((u.nsub + 1) >> 1) {
    case 5: run_unit<MODE, RT, 5>(u, lds, wpk, src, gather, gate, inv, k, zrow, dst16, ybuf, d, F); break;
    case 4: run_unit<MODE, RT, 4>(u, lds, wpk, src, gather, gate, inv, k, zrow, dst16, ybuf, d, F); break;
    case 3: run_unit<MODE, RT, 3>(u, lds, wpk, src, gather, gate, inv, k, zrow, dst16, ybuf, d, F); break;
    case 2: run_unit<MODE, RT, 2>(u, lds, wpk, src, gather, gate, inv, k, zrow, dst16, ybuf, d, F); break;
    default: run_unit<MODE, RT, 1>(u, lds, wpk, src, gather, gate, inv, k, zrow, dst16, ybuf, d, F); break;
  }
}

namespace {
// Upper bound on the spans of all experts for n assignments: the subtiles
// number at most floor((n + 31 E) / 32), and each expert adds at most
// kSubCap - 1 to the rounding-up of its span count.
int max_spans(int n, int E) { return ((n + 31 * E) / kSub + E * (kSubCap - 1)) / kSubCap; }

template <int MODE, int RT>
hipError_t launch_gemm(const FwdArgs& a) {
  const int d = a.dim.d, F = a.dim.F;
  const int nrb = (MODE == 0 ? 2 * F : d) / Geo<RT>::kRows;
  const int units = nrb * max_spans(a.n, a.dim.E);
  const int grid = (units + 7) / 8 * 8;
  return launch(k_expert_gemm<MODE, RT>, dim3(grid), dim3(256), a.stream,
                a.ev[MODE == 0 ? kSlotExpertsA : kSlotExpertsB],
                (const uint16_t*)(MODE == 0 ? a.wgu : a.wd),
                (const uint16_t*)(MODE == 0 ? a.xt : a.act), (const int*)a.counts,
                (const int*)a.offsets, (const int*)a.gather, (const float*)a.gate,
                (const float*)a.inv, a.dim.k, a.dim.E, (const uint16_t*)a.zrow,
                (uint16_t*)(MODE == 0 ? a.act : a.out), a.ybuf, d, F);
}
}  // namespace

// Gate/up on 192-row blocks where 2 * d_ff divides into them, else 128-row
// blocks; the down projection on 128-row blocks (d_model / 128 blocks per
// expert, one unit per CU for 16 experts of ~256 tokens at d_model = 2048).
hipError_t launch_experts_tile(const FwdArgs& a) {
  hipError_t err = (2 * a.dim.F) % Geo<3>::kRows == 0 ? launch_gemm<0, 3>(a)
                                                      : launch_gemm<0, 2>(a);
  if (err != hipSuccess) return err;
  return launch_gemm<1, 2>(a);
}

}  // namespace moe
