// K3 (prefill shapes): grouped SwiGLU GEMMs over the experts.
//
// Expert FFN y = W_down (SiLU(W_gate x) * (W_up x)) per routed assignment
// (SwiGLU: GLU variants paper on the ZONOS2 report's "Builds on" list; 16
// experts per layer, digest item 5).  Two launches:
//   MODE 0  act[slot, f] = bf16( SiLU(x W_gate^T) * (x W_up^T) )   K = d_model
//           (x: the normalised rows, RMSNorm applied by the gather)
//   MODE 1  y[slot, m]   = act[slot] W_down^T                                    K = d_ff
//           k = 1: out[token] = bf16(gate * y) (in a stack, bf16(res + that));
//           k > 1: y kept in fp32.
//
// Work unit: (expert, block of 128*RT weight rows, span of at most 32*cap of
// the expert's slots; cap <= TTM, chosen per launch on the host, TTM = 5 for
// gate/up and 6 for down).  An expert's slots are cut into the fewest spans of
// at most cap 32-token subtiles, split evenly; units are ordered so that the
// ones running together on an XCD share a few weight blocks and a few token
// spans, each brought into that XCD's L2 once.
//
// Workgroup (OCC per CU, 1 by default): four waves, one per SIMD, stacked
// along the weight rows; a wave
// owns RT 32-row tiles against the unit's TT token subtiles (RT*TT
// accumulators of 32x32 fp32).  Both operands are stored as 1 KiB MFMA operand
// blocks: the weights in the packed bank, the tokens in expert-ordered
// subtiles (gate/up: the gathered rows of k_gather_tiles.hip; down: the
// activations, which the gate/up epilogue writes in that layout), so every
// wave-wide load reads one contiguous KiB.
//  * Weights go straight from HBM into each wave's operand registers through a
//    queue Q k-steps deep (8: 96 KiB in flight per CU at RT = 3, 64 KiB at
//    RT = 2): the weight stream is what needs latency cover, and a register
//    queue costs no LDS.
//  * Tokens, shared by the four waves, go through three LDS stages of 64 k
//    (two staged in registers in flight); one barrier per stage, passed with
//    the next stage's first operands already read.
//
// Gate/up rows are packed as 32-row tiles of 16 gate rows followed by the 16
// up rows of the same columns, so the lane that holds gate(f) in accumulator
// element i holds up(f) in element i + 8 and the SiLU * up epilogue needs no
// exchange between lanes.  The activation tiles go out with non-temporal
// stores (read back by the down launch, not kept dirty in this XCD's L2).
//
// fp8 (e4m3) expert weights: the GEMMs read a bank of the codes' exact bf16
// values (every e4m3 value is a bf16 value), so the MFMA products are the
// codes' own; the per-row dequantisation scales multiply the fp32
// accumulators in the epilogue (rsc: per gate/up row, or per output row of
// the down projection; null for bf16 weights).
//
// fp8 weights and fp8 activations (F8): both operands are E4M3 codes and the
// products run on v_mfma_f32_32x32x64_f8f6f4.  The weights come from the
// layer's fp8 bank and the tokens from E4M3 operand tiles (k_quant_tiles.hip),
// both as 1 KiB blocks of 32 rows x 32 k (lane l: 16 codes of row l % 32);
// one MFMA takes two consecutive blocks (64 k, 32 bytes per lane).  A block
// carries as many bytes as a bf16 block, so the token stages, the LDS ring
// and the weight queue are the same, counted in blocks: a stage holds two
// MFMA steps instead of four.  The epilogues multiply the accumulators by
// the weight row's scale and the token row's activation scale (asc, one per
// padded slot).
#include <algorithm>
#include <cstdint>
#include <unordered_map>
#include <vector>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {
constexpr int kSub = 32;      // tokens per MFMA subtile
constexpr int kBK = 4;        // k-steps (of 16) per token stage
constexpr int kBStages = 3;   // LDS token stages
// Weight blocks per group of the unit order, for an expert with ns spans.
__host__ __device__ constexpr int grp_width(int ns) { return ns >= 8 ? 4 : 1; }
// 16-byte LDS entries of one token stage of a unit with TT subtiles
template <int TT>
constexpr int stage_ent() { return TT * kBK * 64; }

template <int RT>
struct Geo {
  static constexpr int kTiles = 4 * RT;  // 32-row weight tiles per unit
  static constexpr int kRows = kTiles * 32;
};

// Operand loads are raw buffer loads: a wave-uniform resource (base and byte
// range in scalar registers) per operand, the k-step's byte offset as a
// scalar offset and the lane's 16 bytes as the one vector offset all loads
// share, so no load needs a 64-bit vector address.  The range is the unit's
// own operand extent.
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer of 32-bit elements (gfx9 family)
constexpr int kBlockBytes = kBlockElems * 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kRsrcWord3);
}
__device__ __forceinline__ u32x4 ldb16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}

template <int RT, int TT>
struct Ctx {
  __amdgpu_buffer_rsrc_t wr;  // this wave's RT weight tiles
  int tile_bytes;             // bytes of one packed 32-row tile
  int ksteps;                 // 1 KiB blocks along K
  __amdgpu_buffer_rsrc_t tr;  // the unit's token subtiles
  int boff[TT];               // bytes from tr's base to this wave's stage-0 blocks
  int voff;                   // the lane's 16 bytes of a block
  int wave, lane;
};

template <int RT, int TT>
__device__ __forceinline__ void load_a(const Ctx<RT, TT>& c, int ks, u32x4 (&q)[RT]) {
  const int s = ks < c.ksteps ? ks : c.ksteps - 1;  // clamp: surplus loads stay in bounds
#pragma unroll
  for (int r = 0; r < RT; ++r) q[r] = ldb16(c.wr, c.voff, r * c.tile_bytes + s * kBlockBytes);
}

// Token stage st: blocks j = wave + 4q (subtile q, k-step wave of the stage),
// at LDS entries j * 64 .. j * 64 + 63 of the stage buffer.
template <int RT, int TT>
__device__ __forceinline__ void load_b(const Ctx<RT, TT>& c, int st, int nst, u32x4 (&p)[TT]) {
  const int s = st < nst ? st : nst - 1;
#pragma unroll
  for (int q = 0; q < TT; ++q) p[q] = ldb16(c.tr, c.voff, c.boff[q] + s * kBK * kBlockBytes);
}
template <int RT, int TT>
__device__ __forceinline__ void store_b(const Ctx<RT, TT>& c, u32x4* buf, const u32x4 (&p)[TT]) {
#pragma unroll
  for (int q = 0; q < TT; ++q) buf[(c.wave + 4 * q) * 64 + c.lane] = p[q];
}
template <int TT>
__device__ __forceinline__ void read_b(const u32x4* buf, int s, int lane, u32x4 (&bv)[TT]) {
#pragma unroll
  for (int j = 0; j < TT; ++j) bv[j] = buf[(j * kBK + s) * 64 + lane];
}

// fp8 token operands of MFMA step m of a stage: blocks 2m and 2m+1
template <int TT>
__device__ __forceinline__ void read_b8(const u32x4* buf, int m, int lane, u32x4 (&bv)[TT][2]) {
#pragma unroll
  for (int j = 0; j < TT; ++j) {
    bv[j][0] = buf[(j * kBK + 2 * m) * 64 + lane];
    bv[j][1] = buf[(j * kBK + 2 * m + 1) * 64 + lane];
  }
}

template <int RT, int TT>
__device__ __forceinline__ void mac(const u32x4 (&a)[RT], const u32x4 (&bv)[TT],
                                    f32x16 (&acc)[RT][TT]) {
#pragma unroll
  for (int j = 0; j < TT; ++j)
#pragma unroll
    for (int r = 0; r < RT; ++r) acc[r][j] = mfma_32x32x16(a[r], bv[j], acc[r][j]);
}

template <int RT, int TT>
__device__ __forceinline__ void mac8(const u32x4 (&a0)[RT], const u32x4 (&a1)[RT],
                                     const u32x4 (&bv)[TT][2], f32x16 (&acc)[RT][TT]) {
#pragma unroll
  for (int j = 0; j < TT; ++j)
#pragma unroll
    for (int r = 0; r < RT; ++r)
      acc[r][j] = mfma_32x32x64_fp8(a0[r], a1[r], bv[j][0], bv[j][1], acc[r][j]);
}

// After each of the NM MFMAs of a step, up to two of the step's other
// instructions, in this order: R DS reads, W DS writes, V global loads.
template <int NM, int R, int W, int V>
__device__ __forceinline__ void sched_pairs() {
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
    for (int t = 2 * m; t < 2 * m + 2; ++t) {
      if (t < R) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      else if (t < R + W) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
      else if (t < R + W + V) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
  }
}

// One token stage kb (k-steps 4kb .. 4kb+3).  Per k-step: the token operands
// of the next k-step are read from LDS while this k-step's MFMAs run, and the
// weight queue slot just consumed is refilled eight k-steps ahead.  In the
// second k-step the staged registers holding token stage kb+2 go to LDS buffer
// (kb+2)%3 (last read in stage kb-1, released by its barrier) and the loads of
// stage kb+4 are issued into them.  The last k-step reads the first operands
// of stage kb+1 (written one stage earlier).  Scheduling barriers keep this
// order (masks: 0x008 MFMA, 0x100 DS read, 0x200 DS write, 0x020 VMEM read).
template <int RT, int TT, int Q, int P>
__device__ __forceinline__ void bstage(const Ctx<RT, TT>& c, u32x4* lds, int& buf, int kb,
                                       int nsb, u32x4 (&qa)[Q][RT], u32x4 (&rb)[TT],
                                       u32x4 (&bc)[TT], f32x16 (&acc)[RT][TT]) {
  constexpr int NM = RT * TT;
  const int b1 = buf == kBStages - 1 ? 0 : buf + 1;
  const int b2 = b1 == kBStages - 1 ? 0 : b1 + 1;
  constexpr int SE = stage_ent<TT>();
  const u32x4* cur = lds + buf * SE;
#pragma unroll
  for (int i = 0; i < kBK; ++i) {
    const int slot = (P * kBK + i) % Q;  // weight queue slot of this k-step
    u32x4 bn[TT];
    if (i < kBK - 1) read_b<TT>(cur, i + 1, c.lane, bn);
    else read_b<TT>(lds + b1 * SE, 0, c.lane, bn);
    mac(qa[slot], bc, acc);
    load_a(c, (kb * kBK + i) + Q, qa[slot]);
    if (i == 1) {
      store_b(c, lds + b2 * SE, rb);
      load_b(c, kb + 4, nsb, rb);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (m < TT) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        else if (m < 2 * TT) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
        else if (m < 3 * TT + RT) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
    } else {
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (m < TT) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        else if (m < TT + RT) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < TT; ++j) bc[j] = bn[j];
  }
  __syncthreads();
  buf = b1;
}

// The fp8 form of bstage: the stage's four blocks are two MFMA steps, each
// taking two weight queue slots (refilled Q blocks ahead) and two token
// blocks per subtile; the second step copies token stage kb+2 to LDS and
// issues the loads of stage kb+4, as the second k-step of bstage does.
template <int RT, int TT, int Q, int P>
__device__ __forceinline__ void bstage8(const Ctx<RT, TT>& c, u32x4* lds, int& buf, int kb,
                                        int nsb, u32x4 (&qa)[Q][RT], u32x4 (&rb)[TT],
                                        u32x4 (&bc)[TT][2], f32x16 (&acc)[RT][TT]) {
  constexpr int NM = RT * TT;
  const int b1 = buf == kBStages - 1 ? 0 : buf + 1;
  const int b2 = b1 == kBStages - 1 ? 0 : b1 + 1;
  constexpr int SE = stage_ent<TT>();
  const u32x4* cur = lds + buf * SE;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int s0 = (P * kBK + 2 * m) % Q;  // weight queue slots of this step: s0, s0 + 1
    u32x4 bn[TT][2];
    if (m == 0) read_b8<TT>(cur, 1, c.lane, bn);
    else read_b8<TT>(lds + b1 * SE, 0, c.lane, bn);
    mac8(qa[s0], qa[s0 + 1], bc, acc);
    load_a(c, kb * kBK + 2 * m + Q, qa[s0]);
    load_a(c, kb * kBK + 2 * m + 1 + Q, qa[s0 + 1]);
    if (m == 1) {
      store_b(c, lds + b2 * SE, rb);
      load_b(c, kb + 4, nsb, rb);
      sched_pairs<NM, 2 * TT, TT, TT + 2 * RT>();
    } else {
      sched_pairs<NM, 2 * TT, 0, 2 * RT>();
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < TT; ++j) {
      bc[j][0] = bn[j][0];
      bc[j][1] = bn[j][1];
    }
  }
  __syncthreads();
  buf = b1;
}

// Q: depth of the weight queue in k-steps: kBK, 2 kBK or 4 kBK, so that one
// loop iteration (two token stages, four at Q = 4 kBK) returns the queue to
// its first slot; the token stages of the reduction are a multiple of that.
// (F8: k-steps are 1 KiB blocks of 32 k; two make one MFMA step.)
template <int RT, int TT, int Q, bool F8>
__device__ __forceinline__ void mainloop(const Ctx<RT, TT>& c, u32x4* lds, f32x16 (&acc)[RT][TT]) {
  constexpr int NP = Q / kBK < 2 ? 2 : Q / kBK;  // token stages per loop iteration
  static_assert(NP == 2 || NP == 4, "the loop body holds two or four token stages");
  static_assert(Q == kBK || Q == 2 * kBK || Q == 4 * kBK, "queue depth must match the loop body");
  const int nsb = c.ksteps / kBK;                // token stages (a multiple of NP)
  u32x4 qa[Q][RT], rb0[TT], rb1[TT];
  load_b(c, 0, nsb, rb0);
  load_b(c, 1, nsb, rb1);
  store_b(c, lds, rb0);
  load_b(c, 2, nsb, rb0);
  store_b(c, lds + stage_ent<TT>(), rb1);
  load_b(c, 3, nsb, rb1);
#pragma unroll
  for (int i = 0; i < Q; ++i) load_a(c, i, qa[i]);
  __syncthreads();
  int buf = 0;
  if constexpr (F8) {
    static_assert(Q % 2 == 0, "an fp8 MFMA step takes two queue slots");
    u32x4 bc[TT][2];
    read_b8<TT>(lds, 0, c.lane, bc);
    for (int kb = 0; kb < nsb; kb += NP) {
      bstage8<RT, TT, Q, 0>(c, lds, buf, kb, nsb, qa, rb0, bc, acc);
      bstage8<RT, TT, Q, 1>(c, lds, buf, kb + 1, nsb, qa, rb1, bc, acc);
      if constexpr (NP == 4) {
        bstage8<RT, TT, Q, 2>(c, lds, buf, kb + 2, nsb, qa, rb0, bc, acc);
        bstage8<RT, TT, Q, 3>(c, lds, buf, kb + 3, nsb, qa, rb1, bc, acc);
      }
    }
  } else {
    u32x4 bc[TT];
    read_b<TT>(lds, 0, c.lane, bc);
    for (int kb = 0; kb < nsb; kb += NP) {
      bstage<RT, TT, Q, 0>(c, lds, buf, kb, nsb, qa, rb0, bc, acc);
      bstage<RT, TT, Q, 1>(c, lds, buf, kb + 1, nsb, qa, rb1, bc, acc);
      if constexpr (NP == 4) {
        bstage<RT, TT, Q, 2>(c, lds, buf, kb + 2, nsb, qa, rb0, bc, acc);
        bstage<RT, TT, Q, 3>(c, lds, buf, kb + 3, nsb, qa, rb1, bc, acc);
      }
    }
  }
}

// Work units.  Units are numbered expert-major; inside an expert, its weight
// blocks are taken in groups of kGrp, and a group's units are numbered
// span-major (span 0 of the group's blocks, then span 1, ...).  A round of an
// XCD's workgroups, which walk K nearly in lockstep, then covers a few weight
// blocks against several token spans, so that each block and each span is
// pulled into the XCD's L2 once per round: 32 units of the hottest expert of
// a skewed batch touch 4 blocks and 8 spans rather than 1 block and 32 spans
// (half the bytes from beyond L2).  The grid is persistent,
// one workgroup per CU: the unit list is cut into 8 contiguous ranges, one per
// XCD (workgroup b runs on XCD b % 8), so that units sharing weights or token
// rows run at the same time under one L2; inside a range the XCD's workgroups
// take units in snake order (round r deals left to right for even r, right to
// left for odd r), which pairs large and small units of neighbouring spans.
struct Unit {
  int e, rb, slot0, nrows, nsub;
  int sub0;  // first subtile of the unit in the padded, expert-ordered subtile list
};
// The launch's expert table in LDS (E <= 64), built once per workgroup so
// that decoding a unit costs a few LDS reads and one ballot instead of a
// dependent scan over the experts in global memory.
struct ExpTab {
  int cnt[64], off[64];  // assignments and first slot of each expert
  int ns[64];            // 32-token subtiles of each expert
  int psub[64];          // subtiles of the experts before it
  int sp[64];            // spans of each expert under the launch's cap
  int ubase[64];         // first unit of each expert
};

__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

// Fill the table for span cap `cap` and return the launch's unit count.
__device__ __forceinline__ int build_table(ExpTab& tab, const int* __restrict__ counts,
                                           const int* __restrict__ offsets, int E, int nrb,
                                           int cap) {
  const int tid = threadIdx.x;
  if (tid < 64) {
    const int c = tid < E ? counts[tid] : 0;
    const int ns = (c + kSub - 1) / kSub;
    tab.cnt[tid] = c;
    tab.off[tid] = tid < E ? offsets[tid] : 0;
    tab.ns[tid] = ns;
    tab.psub[tid] = wave_incl_scan(ns) - ns;
  }
  __syncthreads();
  if (tid < 64) {
    const int n = nrb * ((tab.ns[tid] + cap - 1) / cap);  // 0 past the last expert
    tab.sp[tid] = n / nrb;
    tab.ubase[tid] = wave_incl_scan(n) - n;
  }
  __syncthreads();
  return tab.ubase[63] + nrb * tab.sp[63];
}

// Unit L: the one lane whose expert's unit range holds L names the expert.
__device__ __forceinline__ void decode_unit(const ExpTab& tab, int nrb, int L, Unit& u) {
  const int lane = threadIdx.x & 63;
  const int lo = tab.ubase[lane];
  const unsigned long long m = __ballot(L >= lo && L < lo + nrb * tab.sp[lane]);
  const int e = __builtin_amdgcn_readfirstlane(__ffsll((long long)m) - 1);
  const int ns = __builtin_amdgcn_readfirstlane(tab.sp[e]);
  const int nsub = __builtin_amdgcn_readfirstlane(tab.ns[e]);
  const int r = L - __builtin_amdgcn_readfirstlane(tab.ubase[e]);
  const int G = grp_width(ns);
  const int g = r / (G * ns), i = r - g * G * ns;  // block group, unit inside it
  const int gw = min(G, nrb - g * G);              // blocks in the group
  const int sp = i / gw;
  const int s0 = sp * nsub / ns, s1 = (sp + 1) * nsub / ns;
  u.e = e;
  u.rb = g * G + i % gw;
  u.slot0 = __builtin_amdgcn_readfirstlane(tab.off[e]) + s0 * kSub;
  u.nrows = min(__builtin_amdgcn_readfirstlane(tab.cnt[e]), s1 * kSub) - s0 * kSub;
  u.nsub = s1 - s0;
  u.sub0 = __builtin_amdgcn_readfirstlane(tab.psub[e]) + s0;
}

// SC: fp8 weights (row scales in rsc); bf16 weights compile without them.
// F8: fp8 weights and activations (row scales in rsc, activation scales in asc).
template <int MODE, int RT, int Q, int TT, bool SC, bool F8>
__device__ __forceinline__ void run_unit(const Unit& u, u32x4* lds, const uint16_t* __restrict__ wpk,
                                         const uint16_t* __restrict__ src,
                                         const int* __restrict__ gather,
                                         const float* __restrict__ gate,
                                         const float* __restrict__ rsc,
                                         const float* __restrict__ asc, float* __restrict__ pmax,
                                         int k, const uint16_t* __restrict__ zrow,
                                         uint16_t* __restrict__ dst16,
                                         const uint16_t* __restrict__ res, float* __restrict__ ybuf,
                                         int d, int F) {
  using G = Geo<RT>;
  const int K = MODE == 0 ? d : F;
  const int rows_e = MODE == 0 ? 2 * F : d;  // weight rows of one expert
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile0 = u.rb * G::kTiles + wave * RT;  // this wave's first tile within the expert

  Ctx<RT, TT> c;
  c.wave = wave;
  c.lane = lane;
  c.voff = lane * 16;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  c.ksteps = K / (F8 ? 2 * kKStep : kKStep);  // 1 KiB blocks along K
  c.tile_bytes = c.ksteps * kBlockBytes;
  c.wr = rsrc(reinterpret_cast<const char*>(wpk) +
                  ((size_t)u.e * (rows_e / kTileRows) + u.rb * G::kTiles + wv * RT) *
                      c.tile_bytes,
              RT * c.tile_bytes);
  // subtiles sub0 .. sub0 + TT - 1 of the unit (run_any gives TT == u.nsub)
  c.tr = rsrc(reinterpret_cast<const char*>(src) + (size_t)u.sub0 * c.tile_bytes,
              TT * c.tile_bytes);
#pragma unroll
  for (int q = 0; q < TT; ++q) c.boff[q] = q * c.tile_bytes + wv * kBlockBytes;

  f32x16 acc[RT][TT];
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int j = 0; j < TT; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[r][j][q] = 0.f;

  // down, k = 1: the token of each of the lane's output rows, loaded before
  // the main loop so that the epilogue's gate loads find them in registers
  // (one memory round trip at the end of the unit instead of two; the fp8
  // form has no registers to spare for them)
  constexpr bool kTokPre = MODE == 1 && !F8;
  int tokp[kTokPre ? TT : 1];
  if constexpr (kTokPre) {
#pragma unroll
    for (int j = 0; j < TT; ++j) {
      const int r = j * kSub + (lane & 31);
      tokp[j] = k == 1 && r < u.nrows ? gather[u.slot0 + r] : 0;
    }
  }

  mainloop<RT, TT, Q, F8>(c, lds, acc);

  // epilogue
  const int col = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int j = 0; j < TT; ++j) {
    const int r = j * kSub + col;  // unit row
    if constexpr (MODE == 0) {
      // activations in the down projection's operand tiles: subtile sub0 + j,
      // k-step gt (16 columns of d_ff per gate/up tile); each wave store of a
      // (tile, subtile) pair fills one whole 1 KiB block
      uint16_t* blk = dst16 + (size_t)(u.sub0 + j) * (F / kKStep) * kBlockElems;
      float amax = 0.f;  // F8: the token's largest |activation| over this wave's columns
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int gt = tile0 + rt;  // 16 gate rows + 16 up rows: columns 16*gt ..
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          // fp8 weights: per-row dequantisation scales of the gate rows
          // 16*gt + 8g + 4hi .. +3 and of the matching up rows
          float v4[4];
          if constexpr (F8) {  // weight row scales times the token's activation scale
            const float* rs = rsc + (size_t)u.e * 2 * F + 32 * gt + 8 * g + 4 * hi;
            const f32x4 sg = *reinterpret_cast<const f32x4*>(rs);
            const f32x4 su = *reinterpret_cast<const f32x4*>(rs + 16);
            const float xs = asc[(size_t)(u.sub0 + j) * kSub + col];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              v4[t] = silu((sg[t] * xs) * acc[rt][j][4 * g + t]) *
                      ((su[t] * xs) * acc[rt][j][4 * g + 8 + t]);
              amax = fmaxf(amax, fabsf(v4[t]));
            }
          } else if constexpr (SC) {
            const float* rs = rsc + (size_t)u.e * 2 * F + 32 * gt + 8 * g + 4 * hi;
            const f32x4 sg = *reinterpret_cast<const f32x4*>(rs);
            const f32x4 su = *reinterpret_cast<const f32x4*>(rs + 16);
#pragma unroll
            for (int t = 0; t < 4; ++t)
              v4[t] = silu(sg[t] * acc[rt][j][4 * g + t]) * (su[t] * acc[rt][j][4 * g + 8 + t]);
          } else {
#pragma unroll
            for (int t = 0; t < 4; ++t)
              v4[t] = silu(acc[rt][j][4 * g + t]) * acc[rt][j][4 * g + 8 + t];
          }
          u32x2 v;
          v[0] = pack_bf16x2(v4[0], v4[1]);
          v[1] = pack_bf16x2(v4[2], v4[3]);
          // operand lane g*32 + col holds columns 8g .. 8g+7 of the k-step
          stg8_stream(blk + ((size_t)gt * 64 + g * 32 + col) * 8 + 4 * hi, v);
        }
      }
      if constexpr (F8) {
        // the two lanes of a token hold different rows; bf16 rounding is
        // monotone, so the bf16 value of the max is the max of the bf16 values
        amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
        if (hi == 0)
          pmax[((size_t)(u.sub0 + j) * (F / (16 * RT)) + tile0 / RT) * kSub + col] =
              bf16_lo(f32_to_bf16(amax));
      }
    } else {
      // Output rows leave through LDS as whole row pieces: the wave's 64
      // output rows of the subtile's 32 tokens go to a wave-private LDS tile
      // [32 tokens][64 rows] (its 16-byte chunks swizzled by token against
      // bank conflicts; the token stages are free after the main loop), and
      // come back 16 bytes per lane, so that one store instruction writes 8
      // tokens' contiguous 128-byte bf16 pieces (4 tokens' 256-byte fp32
      // pieces for k > 1) instead of 16 bytes of each of 32 tokens.
      static_assert(MODE == 0 || RT == 2, "the down epilogue's LDS tile holds 64 rows");
      char* wl = reinterpret_cast<char*>(lds) + wave * 8192;
      const bool ok = r < u.nrows;
      int tok;
      if constexpr (kTokPre) tok = tokp[j];
      else tok = k == 1 && ok ? gather[u.slot0 + r] : 0;
      const float gw = k == 1 && ok ? gate[tok] : 0.f;
      float ms = 1.f;  // F8: the token row's activation scale
      if constexpr (F8) ms = asc[(size_t)(u.sub0 + j) * kSub + col];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if constexpr (F8) {  // per-row weight scales times the activation scale
            const int m = (tile0 + rt) * kTileRows + 4 * hi + 8 * q;
            const f32x4 s4 = *reinterpret_cast<const f32x4*>(rsc + (size_t)u.e * d + m);
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[rt][j][4 * q + t] *= s4[t] * ms;
          } else if constexpr (SC) {  // fp8 weights: per-row scales of output rows m .. m+3
            const int m = (tile0 + rt) * kTileRows + 4 * hi + 8 * q;
            const f32x4 s4 = *reinterpret_cast<const f32x4*>(rsc + (size_t)u.e * d + m);
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[rt][j][4 * q + t] *= s4[t];
          }
          // local rows rt*32 + 8q + 4hi .. +3 of token col
          if (k == 1) {
            u32x2 v;
            v[0] = pack_bf16x2(gw * acc[rt][j][4 * q], gw * acc[rt][j][4 * q + 1]);
            v[1] = pack_bf16x2(gw * acc[rt][j][4 * q + 2], gw * acc[rt][j][4 * q + 3]);
            const int ch = rt * 4 + q;
            *reinterpret_cast<u32x2*>(wl + col * 128 + ((ch ^ (col & 7)) << 4) + 8 * hi) = v;
          } else {
            const f32x4 v = {acc[rt][j][4 * q], acc[rt][j][4 * q + 1], acc[rt][j][4 * q + 2],
                             acc[rt][j][4 * q + 3]};
            const int ch = rt * 8 + 2 * q + hi;
            *reinterpret_cast<f32x4*>(wl + col * 256 + ((ch ^ (col & 15)) << 4)) = v;
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int mw = tile0 * kTileRows;  // the wave's first output row
      if (k == 1) {
        // in a stack (res): out = bf16(res + bf16(gate * y)); the residual
        // pieces are all loaded first (rows past the unit read token 0's)
        u32x4 hv[4];
        if (res != nullptr) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tr = __shfl(tok, (lane >> 3) + 8 * i, 64);
            hv[i] = ldg16(res + (size_t)tr * d + mw + (lane & 7) * 8);
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tl = (lane >> 3) + 8 * i, ch = lane & 7;
          const int tr = __shfl(tok, tl, 64);
          u32x4 v = *reinterpret_cast<const u32x4*>(wl + tl * 128 + ((ch ^ (tl & 7)) << 4));
          if (res != nullptr) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              v[q] = pack_bf16x2(bf16_lo(hv[i][q]) + bf16_lo(v[q]),
                                 bf16_hi(hv[i][q]) + bf16_hi(v[q]));
          }
          if (j * kSub + tl < u.nrows)
            *reinterpret_cast<u32x4*>(dst16 + (size_t)tr * d + mw + ch * 8) = v;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int tl = (lane >> 4) + 4 * i, ch = lane & 15;
          const f32x4 v = *reinterpret_cast<const f32x4*>(wl + tl * 256 + ((ch ^ (tl & 15)) << 4));
          if (j * kSub + tl < u.nrows)
            *reinterpret_cast<f32x4*>(ybuf + (size_t)(u.slot0 + j * kSub + tl) * d + mw + ch * 4) =
                v;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
}
}  // namespace

namespace {
// run_unit for the unit's subtile count (at most TTM)
template <int MODE, int RT, int Q, int TT, bool SC, bool F8>
__device__ __forceinline__ void run_any(const Unit& u, u32x4* lds, const uint16_t* __restrict__ wpk,
                                        const uint16_t* __restrict__ src,
                                        const int* __restrict__ gather,
                                        const float* __restrict__ gate,
                                        const float* __restrict__ rsc,
                                        const float* __restrict__ asc, float* __restrict__ pmax,
                                        int k, const uint16_t* __restrict__ zrow,
                                        uint16_t* __restrict__ dst16,
                                        const uint16_t* __restrict__ res, float* __restrict__ ybuf,
                                        int d, int F) {
  if constexpr (TT > 1) {
    if (u.nsub != TT) {
      run_any<MODE, RT, Q, TT - 1, SC, F8>(u, lds, wpk, src, gather, gate, rsc, asc, pmax, k,
                                           zrow, dst16, res, ybuf, d, F);
      return;
    }
  }
  run_unit<MODE, RT, Q, TT, SC, F8>(u, lds, wpk, src, gather, gate, rsc, asc, pmax, k, zrow, dst16,
                                    res, ybuf, d, F);
}
}  // namespace

// OCC workgroups per CU; spans of at most TTM subtiles.
template <int MODE, int RT, int Q, int OCC, int TTM, bool SC, bool F8>
__global__ __launch_bounds__(256, OCC) void k_expert_gemm(
    const uint16_t* __restrict__ wpk, const uint16_t* __restrict__ src,
    const int* __restrict__ counts, const int* __restrict__ offsets,
    const int* __restrict__ gather, const float* __restrict__ gate,
    const float* __restrict__ rsc, const float* __restrict__ asc, float* __restrict__ pmax, int k,
    int E, int cap,
    const uint16_t* __restrict__ zrow, uint16_t* __restrict__ dst16,
    const uint16_t* __restrict__ res, float* __restrict__ ybuf, int d, int F) {
  static_assert(TTM >= 1 && TTM <= 8, "token subtiles per unit");
  __shared__ u32x4 lds[kBStages * stage_ent<TTM>()];
  static_assert(MODE == 0 || sizeof(lds) >= 4 * 8192, "the down epilogue's per-wave LDS tiles");
  const int nrb = (MODE == 0 ? 2 * F : d) / Geo<RT>::kRows;
  __shared__ ExpTab tab;
  const int U = build_table(tab, counts, offsets, E, nrb, cap);
  const int per = (U + 7) >> 3;          // units per XCD range
  const int nw = gridDim.x >> 3;         // workgroups per XCD (the grid is a multiple of 8)
  const int x = blockIdx.x & 7, w = blockIdx.x >> 3;
  const int lo = x * per, hi = min(U, lo + per);
  for (int r = 0; r * nw < per; ++r) {
    const int L = lo + ((r & 1) ? (r + 1) * nw - 1 - w : r * nw + w);
    if (L >= hi) continue;
    Unit u;
    decode_unit(tab, nrb, L, u);
    __syncthreads();  // the previous unit's last LDS reads are done everywhere
    run_any<MODE, RT, Q, TTM, SC, F8>(u, lds, wpk, src, gather, gate, rsc, asc, pmax, k, zrow, dst16,
                                      res, ybuf, d, F);
  }
}

namespace {
// Span cap of a launch: the most token subtiles a unit holds (1..TTM).
// Fewer, larger units save per-unit cost (the weight stream's start, the
// epilogue), but the dealing can leave the grid's last round mostly idle.
// Each cap from TTM - 2 to TTM is priced on the host by replaying the
// kernel's dealing (ranges per XCD, snake order) for n assignments spread
// evenly over the experts, a unit costing 2 + its token subtiles (a fit to
// measured unit times of both GEMMs: a unit's fixed cost is about that of
// two subtiles of MFMA work); the busiest workgroup's total decides, ties
// to the larger cap.  The counts themselves are on the device; pricing them
// there took longer than the choice saved.  Results are cached per shape.
int span_cap(int n, int E, int nrb, int grid, int TTM) {
  static thread_local std::unordered_map<uint64_t, int> memo;
  const uint64_t key = (uint64_t)n << 32 ^ (uint64_t)E << 24 ^ (uint64_t)nrb << 12 ^
                       (uint64_t)grid << 4 ^ (uint64_t)TTM;
  if (auto it = memo.find(key); it != memo.end()) return it->second;
  std::vector<int> ns(E);
  for (int e = 0; e < E; ++e) ns[e] = (n / E + (e < n % E ? 1 : 0) + kSub - 1) / kSub;
  const int nw = grid / 8;
  int best = TTM;
  long long best_cost = -1;
  std::vector<uint8_t> cost;
  for (int t = TTM; t >= 1 && t >= TTM - 2; --t) {
    cost.clear();
    for (int e = 0; e < E; ++e) {
      const int sp = (ns[e] + t - 1) / t;
      const int G = grp_width(sp);
      for (int g = 0; g < nrb; g += G)  // the kernel's order: block groups, span-major
        for (int q = 0; q < sp; ++q)
          for (int rb = g; rb < std::min(nrb, g + G); ++rb)
            cost.push_back((uint8_t)(2 + (q + 1) * ns[e] / sp - q * ns[e] / sp));
    }
    const int U = (int)cost.size(), per = (U + 7) / 8;
    long long mx = 0;
    for (int b = 0; b < grid; ++b) {
      const int x = b & 7, w = b >> 3, lo = x * per, hi = std::min(U, lo + per);
      long long c = 0;
      for (int r = 0; r * nw < per; ++r) {
        const int L = lo + ((r & 1) ? (r + 1) * nw - 1 - w : r * nw + w);
        if (L < hi) c += cost[L];
      }
      mx = std::max(mx, c);
    }
    if (best_cost < 0 || mx < best_cost) {
      best_cost = mx;
      best = t;
    }
  }
  if (memo.size() > 4096) memo.clear();
  memo.emplace(key, best);
  return best;
}

// F8: fp8 weights and activations (the fp8 banks, the E4M3 token tiles and
// their scales).
template <int MODE, int RT, int Q, int OCC, int TTM, bool F8 = false>
hipError_t launch_gemm(const FwdArgs& a) {
  const int grid = (a.num_cu * OCC + 7) / 8 * 8;  // persistent: OCC workgroups per CU
  const int nrb = (MODE == 0 ? 2 * a.dim.F : a.dim.d) / Geo<RT>::kRows;
  const int cap = span_cap(a.n, a.dim.E, nrb, grid, TTM);
  const float* rsc = MODE == 0 ? a.sgu : a.sd;
  auto kern = F8 ? k_expert_gemm<MODE, RT, Q, OCC, TTM, true, F8>
                 : rsc != nullptr ? k_expert_gemm<MODE, RT, Q, OCC, TTM, true, false>
                                  : k_expert_gemm<MODE, RT, Q, OCC, TTM, false, false>;
  const void* wsrc = F8 ? (MODE == 0 ? a.wgu8 : a.wd8) : (MODE == 0 ? a.wgu : a.wd);
  const void* tsrc = F8 ? (MODE == 0 ? a.xq : a.actq) : (MODE == 0 ? a.xt : a.act);
  const float* asc = F8 ? (MODE == 0 ? a.sx : a.sm) : nullptr;
  return launch(kern, dim3(grid), dim3(256), a.stream,
                a.ev[MODE == 0 ? kSlotExpertsA : kSlotExpertsB],
                (const uint16_t*)wsrc, (const uint16_t*)tsrc, (const int*)a.counts,
                (const int*)a.offsets, (const int*)a.gather, (const float*)a.gate,
                rsc, asc, F8 && MODE == 0 ? a.pmm : nullptr, a.dim.k, a.dim.E, cap,
                (const uint16_t*)a.zrow,
                (uint16_t*)(MODE == 0 ? a.act : a.out),
                (const uint16_t*)(MODE == 0 ? nullptr : a.res), a.ybuf, a.dim.d, a.dim.F);
}
}  // namespace

// Gate/up on 384-row blocks (192 columns of d_ff) with an 8-k-step weight
// queue and spans of up to 5 subtiles where 2 * d_ff divides into them, else
// on 256-row blocks with a 16-k-step queue (d_model % 256 == 0 makes d/16 a
// multiple of 16); the down projection on 256-row blocks, an 8-k-step queue
// and spans of up to 6 subtiles (the registers' limit at that queue; a
// 16-k-step queue at 5 subtiles times the same).  On the prefill workloads the
// 384-row gate/up units are faster (fewer re-reads of the token tiles per
// weight byte); the deeper queue that fits the 256-row units' registers did
// not make up for it.
hipError_t launch_experts_tile(const FwdArgs& a) {
  hipError_t err = (2 * a.dim.F) % Geo<3>::kRows == 0 ? launch_gemm<0, 3, 8, 1, 5>(a)
                                                      : launch_gemm<0, 2, 16, 1, 5>(a);
  if (err != hipSuccess) return err;
  return launch_gemm<1, 2, 8, 1, 6>(a);  // d_ff % 128 == 0: the k-steps fill whole loop bodies
}

// fp8 weights and activations: the gate/up GEMM over the E4M3 token tiles,
// then (after k_quant_tiles has quantised its activations) the down GEMM.
// Blocks of 32 k: d_model % 256 == 0 and d_ff % 256 == 0 fill whole loop
// bodies of two stages (8 blocks) with an 8-block weight queue.
hipError_t launch_experts_tile_fp8_gateup(const FwdArgs& a) {
  return fp8_gateup_rt(a.dim.F) == 3 ? launch_gemm<0, 3, 8, 1, 5, true>(a)
                                     : launch_gemm<0, 2, 8, 1, 5, true>(a);
}
hipError_t launch_experts_tile_fp8_down(const FwdArgs& a) {
  return launch_gemm<1, 2, 8, 1, 6, true>(a);
}

}  // namespace moe
