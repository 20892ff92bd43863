// Create-time preparation of the layer's parameters.
//
// Expert weights (bf16) are repacked once from the caller's row-major tensors
// into 1 KiB blocks in MFMA 32x32x16 operand order, so that at run time each
// wave-wide load is one contiguous KiB of HBM and lands in the operand
// registers (or an LDS stage) without any shuffle:
//   W_gu : [E][2F/32][d/16][64 lanes][8]   lane = row % 32 + 32 * (k-group); tile t
//          holds the gate rows of columns 16t .. 16t+15, then their up rows
//   W_d  : [E][d/32][F/16][64 lanes][8]
// The router rows are stored in fp32 with the RMSNorm gain folded in,
// wrg[e][i] = W_r[e][i] * g[i] (exact for bf16 operands), padded with zero rows
// up to a power-of-two expert count.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

__global__ void k_pack_gateup(const uint16_t* __restrict__ wg, const uint16_t* __restrict__ wu,
                              uint16_t* __restrict__ packed, int E, int F, int d) {
  const size_t q = (size_t)blockIdx.x * 256 + threadIdx.x;  // 16-byte chunk index
  const int ks = d / kKStep;
  const int nt = 2 * F / kTileRows;  // interleaved 32-row tiles per expert
  const size_t total = (size_t)E * nt * ks * 64;
  if (q >= total) return;
  const int lane = (int)(q % 64);
  size_t r = q / 64;
  const int s = (int)(r % ks);
  r /= ks;
  const int gt = (int)(r % nt);
  const int e = (int)(r / nt);
  const int rr = lane & 31;  // rows 0-15: gate, rows 16-31: up, of columns 16*gt ..
  const int f = gt * 16 + (rr & 15);
  const int kk = s * kKStep + (lane >> 5) * 8;
  const uint16_t* src = (rr < 16 ? wg : wu) + ((size_t)e * F + f) * d + kk;
  stg16(packed + q * 8, ldg16(src));
}

__global__ void k_pack_down(const uint16_t* __restrict__ wd, uint16_t* __restrict__ packed, int E,
                            int d, int F) {
  const size_t q = (size_t)blockIdx.x * 256 + threadIdx.x;
  const int ks = F / kKStep;
  const size_t total = (size_t)E * (d / kTileRows) * ks * 64;
  if (q >= total) return;
  const int lane = (int)(q % 64);
  size_t r = q / 64;
  const int s = (int)(r % ks);
  r /= ks;
  const int mt = (int)(r % (d / kTileRows));
  const int e = (int)(r / (d / kTileRows));
  const int row = mt * kTileRows + (lane & 31);
  const int kk = s * kKStep + (lane >> 5) * 8;
  stg16(packed + q * 8, ldg16(wd + ((size_t)e * d + row) * F + kk));
}

template <bool BF16>
__global__ void k_prep_router(const void* __restrict__ w_router, const void* __restrict__ gain,
                              int E, int EP, int d, float* __restrict__ wrg,
                              float* __restrict__ gain32) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)EP * d) return;
  const int e = (int)(idx / d), i = (int)(idx % d);
  float g, w = 0.f;
  if constexpr (BF16) {
    g = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(gain)[i] << 16);
    if (e < E)
      w = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(w_router)[(size_t)e * d + i]
                          << 16);
  } else {
    g = reinterpret_cast<const float*>(gain)[i];
    if (e < E) w = reinterpret_cast<const float*>(w_router)[(size_t)e * d + i];
  }
  wrg[idx] = w * g;
  if (e == 0) gain32[i] = g;
}

hipError_t launch_pack_gateup(const uint16_t* w_gate, const uint16_t* w_up, uint16_t* packed,
                              int E, int F, int d, hipStream_t s) {
  const size_t total = (size_t)E * (2 * F / kTileRows) * (d / kKStep) * 64;
  hipLaunchKernelGGL(k_pack_gateup, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, w_gate,
                     w_up, packed, E, F, d);
  return hipGetLastError();
}

hipError_t launch_pack_down(const uint16_t* w_down, uint16_t* packed, int E, int d, int F,
                            hipStream_t s) {
  const size_t total = (size_t)E * (d / kTileRows) * (F / kKStep) * 64;
  hipLaunchKernelGGL(k_pack_down, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, w_down,
                     packed, E, d, F);
  return hipGetLastError();
}

hipError_t launch_prep_router(const void* w_router, const void* gain, int dtype, int E, int EP,
                              int d, float* wrg, float* gain32, hipStream_t s) {
  const size_t total = (size_t)EP * d;
  const unsigned grid = (unsigned)((total + 255) / 256);
  if (dtype == 1)
    hipLaunchKernelGGL((k_prep_router<true>), dim3(grid), dim3(256), 0, s, w_router, gain, E, EP,
                       d, wrg, gain32);
  else
    hipLaunchKernelGGL((k_prep_router<false>), dim3(grid), dim3(256), 0, s, w_router, gain, E, EP,
                       d, wrg, gain32);
  return hipGetLastError();
}

}  // namespace moe
