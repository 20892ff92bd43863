// fp8 activations: per-row E4M3 quantisation of the expert GEMMs' inputs.
//
// The SGLang-Omni ZONOS2 cookbook page ("Benchmark Results") serves the model
// in "fp8"; read here (besides weight-only fp8) as E4M3 weights and E4M3
// activations with one dynamic scale per row: every routed row u of the
// expert input and every row m = SiLU(G) * V of the SwiGLU intermediate is
// quantised from its bf16 value with a = max|row| / 448 and codes
// RNE_E4M3(v * fl32(1 / a)) (quant4_e4m3), so that both operands of the
// expert GEMMs are E4M3 and the products run on the fp8 MFMA.
//
// The gathered rows are quantised by the gather itself (k_gather_tiles.hip:
// the router leaves each token's scale).  k_quant_tiles: the activation tiles
// of the gate/up epilogue, bf16 operand tiles [P][K/16][64 lanes][8] (lane l
// holds row l % 32, k = 16 s + 8 (l / 32) + 0..7) -> E4M3 tiles [P][K/32][64 lanes][16]
// in the order of the layer's fp8 weight banks (block b, lane l: bytes 0-7
// from bf16 block 2b, bytes 8-15 from bf16 block 2b + 1, both of lane l) and
// one scale per padded slot, a[32 P + row].  One workgroup per subtile in
// use (the subtiles of expert e are ceil(count_e / 32)); padding rows are
// zero and get a = 0.  Each row's amax is the largest of the partial maxima
// that the fp8 gate/up epilogue left, so the subtile is read once.
//
// k_quant_rows: the same quantisation on row-major bf16 rows [R][K] ->
// codes [R][K] and scales [R], one wave per row (moe_fp8_quantize_rows); with
// VALS the rows are overwritten by the codes' values (exact in bf16) instead:
// the activation rows of decode batches, which the fp8 down stream multiplies
// as they are before it scales its sums by the row's scale.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// Each subtile in use is cut into parts of at most 8 * kQuantCh blocks, one
// workgroup of eight waves per part, so that every wave loads its blocks at
// once.  Every workgroup of a subtile reduces the G x 32 partial maxima to
// the 32 row scales (the first part writes them); the loads of the data are
// issued before that reduction, so the two overlap.
constexpr int kQuantCh = 4;  // fp8 blocks per wave

__global__ __launch_bounds__(512) void k_quant_tiles(const uint16_t* __restrict__ src,
                                                     const float* __restrict__ pmax, int G,
                                                     const int* __restrict__ counts, int E, int K,
                                                     int parts, uint8_t* __restrict__ dst,
                                                     float* __restrict__ scale) {
  __shared__ int s_nsub;
  __shared__ float sa[32];
  __shared__ float red[16][32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < 64) {
    int ns = tid < E ? (counts[tid] + 31) >> 5 : 0;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ns += __shfl_xor(ns, o, 64);
    if (tid == 0) s_nsub = ns;
  }
  __syncthreads();
  const int P = blockIdx.x / parts, part = blockIdx.x - P * parts;
  if (P >= s_nsub) return;  // uniform over the workgroup
  const int nb = K / (2 * kKStep);  // fp8 blocks of the subtile
  const uint16_t* s0 = src + (size_t)P * (2 * nb) * kBlockElems + lane * 8;
  uint8_t* d0 = dst + (size_t)P * nb * 1024 + lane * 16;
  const int b0 = part * 8 * kQuantCh + wave;
  u32x4 v[kQuantCh][2];
#pragma unroll
  for (int c = 0; c < kQuantCh; ++c) {
    const int b = b0 + 8 * c;
    if (b < nb) {
      v[c][0] = ldg16(s0 + (size_t)(2 * b) * kBlockElems);
      v[c][1] = ldg16(s0 + (size_t)(2 * b + 1) * kBlockElems);
    }
  }
  {
    // the subtile's G x 32 partial maxima, [group][row]: thread t reads the
    // entries t, t + 512, ... (all of row t % 32), then 16 threads per row meet in LDS
    const float* pm = pmax + (size_t)P * G * 32;
    float m = 0.f;
    for (int i = tid; i < G * 32; i += 512) m = fmaxf(m, pm[i]);
    red[tid >> 5][tid & 31] = m;
  }
  __syncthreads();
  if (tid < 32) {
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, red[i][tid]);
    const float sc = m / 448.f;
    sa[tid] = sc;
    if (part == 0) scale[(size_t)P * 32 + tid] = sc;
  }
  __syncthreads();
  const float r = e4m3_recip(sa[lane & 31]);
#pragma unroll
  for (int c = 0; c < kQuantCh; ++c) {
    const int b = b0 + 8 * c;
    if (b < nb) {
      u32x4 o;
      o[0] = quant4_e4m3(v[c][0][0], v[c][0][1], r);
      o[1] = quant4_e4m3(v[c][0][2], v[c][0][3], r);
      o[2] = quant4_e4m3(v[c][1][0], v[c][1][1], r);
      o[3] = quant4_e4m3(v[c][1][2], v[c][1][3], r);
      stg16_stream(d0 + (size_t)b * 1024, o);
    }
  }
}

// One 16-byte piece (8 values from column c) of row `row`: the codes, or with
// VALS their values written back over the row (each lane rewrites only the 16
// bytes it read).
template <bool VALS>
__device__ __forceinline__ void put8(uint16_t* __restrict__ x, uint8_t* __restrict__ codes,
                                     size_t at, const u32x4& v, float r) {
  const uint32_t c0 = quant4_e4m3(v[0], v[1], r), c1 = quant4_e4m3(v[2], v[3], r);
  if constexpr (VALS) {
    u32x4 o;
    o[0] = e4m3_pair_to_bf16x2<false>(c0);
    o[1] = e4m3_pair_to_bf16x2<true>(c0);
    o[2] = e4m3_pair_to_bf16x2<false>(c1);
    o[3] = e4m3_pair_to_bf16x2<true>(c1);
    stg16(x + at, o);
  } else {
    u32x2 o;
    o[0] = c0;
    o[1] = c1;
    *reinterpret_cast<u32x2*>(codes + at) = o;
  }
}

// RC > 0: rows of at most 512 RC values, which each wave holds in registers
// (RC pieces per lane, all loads in flight at once, the row read once); the
// decode activation rows (d_ff = 3072) took 5.0 us with two passes of
// dependent loads over the row.  RC = 0: any K, two passes.
template <bool VALS, int RC>
__global__ __launch_bounds__(256) void k_quant_rows(uint16_t* __restrict__ x, int R, int K,
                                                    uint8_t* __restrict__ codes,
                                                    float* __restrict__ scale) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= R) return;  // no barrier in this kernel
  const size_t r0 = (size_t)row * K;
  float m = 0.f;
  if constexpr (RC > 0) {
    u32x4 v[RC];
#pragma unroll
    for (int i = 0; i < RC; ++i) {
      const int c = lane * 8 + 512 * i;
      v[i] = c < K ? ldg16(x + r0 + c) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < RC; ++i) m = absmax8_bf16(v[i], m);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    const float a = m / 448.f;
    if (lane == 0) scale[row] = a;
    const float r = e4m3_recip(a);
#pragma unroll
    for (int i = 0; i < RC; ++i) {
      const int c = lane * 8 + 512 * i;
      if (c < K) put8<VALS>(x, codes, r0 + c, v[i], r);
    }
  } else {
    for (int c = lane * 8; c < K; c += 512) m = absmax8_bf16(ldg16(x + r0 + c), m);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    const float a = m / 448.f;
    if (lane == 0) scale[row] = a;
    const float r = e4m3_recip(a);
    for (int c = lane * 8; c < K; c += 512) put8<VALS>(x, codes, r0 + c, ldg16(x + r0 + c), r);
  }
}

hipError_t launch_quant_act(const FwdArgs& a) {
  const int G = a.dim.F / (16 * fp8_gateup_rt(a.dim.F));
  const int nb = a.dim.F / (2 * kKStep);
  const int parts = (nb + 8 * kQuantCh - 1) / (8 * kQuantCh);
  return launch(k_quant_tiles, dim3(max_subtiles(a.n, a.dim.E) * parts), dim3(512), a.stream,
                a.ev[kSlotQuantAct], (const uint16_t*)a.act, (const float*)a.pmm, G,
                (const int*)a.counts, a.dim.E, a.dim.F, parts, (uint8_t*)a.actq, a.sm);
}

namespace {
constexpr int kRowChunks = 8;  // register-resident rows up to 512 * 8 = 4096 values
}

hipError_t launch_quant_rows(const void* x, int R, int K, void* codes, float* scale,
                             hipStream_t s) {
  auto kern = K <= 512 * kRowChunks ? k_quant_rows<false, kRowChunks> : k_quant_rows<false, 0>;
  hipLaunchKernelGGL(kern, dim3((unsigned)((R + 3) / 4)), dim3(256), 0, s,
                     (uint16_t*)const_cast<void*>(x), R, K, (uint8_t*)codes, scale);
  return hipGetLastError();
}

hipError_t launch_quant_act_rows(const FwdArgs& a) {
  return launch(a.dim.F <= 512 * kRowChunks ? k_quant_rows<true, kRowChunks>
                                            : k_quant_rows<true, 0>,
                dim3((unsigned)((a.n + 3) / 4)), dim3(256), a.stream, a.ev[kSlotQuantAct],
                (uint16_t*)a.act, a.n, a.dim.F, (uint8_t*)nullptr, a.sm);
}

}  // namespace moe
