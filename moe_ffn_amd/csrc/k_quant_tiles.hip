// fp8 activations: per-row E4M3 quantisation of the expert GEMMs' inputs.
//
// The SGLang-Omni ZONOS2 cookbook page ("Benchmark Results") serves the model
// in "fp8"; read here (besides weight-only fp8) as E4M3 weights and E4M3
// activations with one dynamic scale per row: every routed row u of the
// expert input and every row m = SiLU(G) * V of the SwiGLU intermediate is
// quantised from its bf16 value with a = max|row| / 448 and codes
// RNE_E4M3(v / a) (quant4_e4m3), so that both operands of the expert GEMMs
// are E4M3 and the products run on the fp8 MFMA.
//
// k_quant_tiles: bf16 operand tiles [P][K/16][64 lanes][8] (the gather's token
// tiles, or the activation tiles of the gate/up epilogue; lane l holds row
// l % 32, k = 16 s + 8 (l / 32) + 0..7) -> E4M3 tiles [P][K/32][64 lanes][16]
// in the order of the layer's fp8 weight banks (block b, lane l: bytes 0-7
// from bf16 block 2b, bytes 8-15 from bf16 block 2b + 1, both of lane l) and
// one scale per padded slot, a[32 P + row].  One workgroup per subtile in
// use (the subtiles of expert e are ceil(count_e / 32)); padding rows are
// zero and get a = 0.  Pass 1 finds the rows' amax, pass 2 reads the subtile
// again (from cache) and converts.
//
// k_quant_rows: the same quantisation on row-major bf16 rows [R][K] ->
// codes [R][K] and scales [R], one wave per row (moe_fp8_quantize_rows).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

__global__ __launch_bounds__(256) void k_quant_tiles(const uint16_t* __restrict__ src,
                                                     const int* __restrict__ counts, int E, int K,
                                                     uint8_t* __restrict__ dst,
                                                     float* __restrict__ scale) {
  __shared__ int s_nsub;
  __shared__ float red[4][64];
  __shared__ float sa[32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < 64) {
    int ns = tid < E ? (counts[tid] + 31) >> 5 : 0;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ns += __shfl_xor(ns, o, 64);
    if (tid == 0) s_nsub = ns;
  }
  __syncthreads();
  const int P = blockIdx.x;
  if (P >= s_nsub) return;  // uniform over the workgroup
  const int ks = K / kKStep;  // bf16 blocks of the subtile
  const uint16_t* s0 = src + (size_t)P * ks * kBlockElems + lane * 8;
  float m = 0.f;
  for (int b = wave; b < ks; b += 4) m = absmax8_bf16(ldg16(s0 + (size_t)b * kBlockElems), m);
  red[wave][lane] = m;
  __syncthreads();
  if (tid < 32) {
    float a = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) a = fmaxf(a, fmaxf(red[w][tid], red[w][tid + 32]));
    const float sc = a / 448.f;
    sa[tid] = sc;
    scale[(size_t)P * 32 + tid] = sc;
  }
  __syncthreads();
  const float a = sa[lane & 31];
  uint8_t* d0 = dst + (size_t)P * (ks / 2) * 1024 + lane * 16;
  for (int b = wave; b < ks / 2; b += 4) {
    const u32x4 v0 = ldg16(s0 + (size_t)(2 * b) * kBlockElems);
    const u32x4 v1 = ldg16(s0 + (size_t)(2 * b + 1) * kBlockElems);
    u32x4 o;
    o[0] = quant4_e4m3(v0[0], v0[1], a);
    o[1] = quant4_e4m3(v0[2], v0[3], a);
    o[2] = quant4_e4m3(v1[0], v1[1], a);
    o[3] = quant4_e4m3(v1[2], v1[3], a);
    stg16_stream(d0 + (size_t)b * 1024, o);
  }
}

__global__ __launch_bounds__(256) void k_quant_rows(const uint16_t* __restrict__ x, int R, int K,
                                                    uint8_t* __restrict__ codes,
                                                    float* __restrict__ scale) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= R) return;  // no barrier in this kernel
  const uint16_t* xr = x + (size_t)row * K;
  float m = 0.f;
  for (int c = lane * 8; c < K; c += 512) m = absmax8_bf16(ldg16(xr + c), m);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  const float a = m / 448.f;
  if (lane == 0) scale[row] = a;
  for (int c = lane * 8; c < K; c += 512) {
    const u32x4 v = ldg16(xr + c);
    u32x2 o;
    o[0] = quant4_e4m3(v[0], v[1], a);
    o[1] = quant4_e4m3(v[2], v[3], a);
    *reinterpret_cast<u32x2*>(codes + (size_t)row * K + c) = o;
  }
}

hipError_t launch_quant_tiles(const FwdArgs& a, int which) {
  const bool x = which == 0;
  return launch(k_quant_tiles, dim3(max_subtiles(a.n, a.dim.E)), dim3(256), a.stream,
                a.ev[x ? kSlotQuantX : kSlotQuantAct], (const uint16_t*)(x ? a.xt : a.act),
                (const int*)a.counts, a.dim.E, x ? a.dim.d : a.dim.F,
                (uint8_t*)(x ? a.xq : a.actq), x ? a.sx : a.sm);
}

hipError_t launch_quant_rows(const void* x, int R, int K, void* codes, float* scale,
                             hipStream_t s) {
  hipLaunchKernelGGL(k_quant_rows, dim3((unsigned)((R + 3) / 4)), dim3(256), 0, s,
                     (const uint16_t*)x, R, K, (uint8_t*)codes, scale);
  return hipGetLastError();
}

}  // namespace moe
