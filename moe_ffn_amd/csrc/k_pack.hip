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


// ---- fp8 (OCP E4M3) expert weights ------------------------------------------
// The caller gives byte codes and one fp32 scale per output row.  Two copies are
// packed: an fp8 bank for the weight-streaming decode kernels, in which lane l
// of a 16-byte piece holds the codes of row l % 32 for two consecutive k-steps,
//   W_gu8 : [E][2F/32][d/32][64 lanes][16]   bytes 0-7: k-step 2p, 8-15: 2p+1
//   W_d8  : [E][d/32][F/32][64 lanes][16]
// (k-group l / 32 of each k-step), and the bf16 banks above holding the code
// values themselves (every E4M3 value is exact in bf16) for the prefill GEMM.
// The scales are applied to the fp32 accumulators, so no weight is rounded.
// Layers with fp8 activations keep only the fp8 banks, which the fp8 MFMA
// GEMMs read as they are (a 16-byte piece is one lane's share of a 1 KiB
// block of 32 rows x 32 k).
// gate/up or down codes -> bf16 bank in the layout of k_pack_gateup / k_pack_down
__global__ void k_pack_gateup_fp8_bf16(const uint8_t* __restrict__ wg, const uint8_t* __restrict__ wu,
                                       uint16_t* __restrict__ packed, int E, int F, int d) {
  const size_t q = (size_t)blockIdx.x * 256 + threadIdx.x;
  const int ks = d / kKStep;
  const int nt = 2 * F / kTileRows;
  const size_t total = (size_t)E * nt * ks * 64;
  if (q >= total) return;
  const int lane = (int)(q % 64);
  size_t r = q / 64;
  const int s = (int)(r % ks);
  r /= ks;
  const int gt = (int)(r % nt);
  const int e = (int)(r / nt);
  const int rr = lane & 31;
  const int f = gt * 16 + (rr & 15);
  const int kk = s * kKStep + (lane >> 5) * 8;
  const uint8_t* src = (rr < 16 ? wg : wu) + ((size_t)e * F + f) * d + kk;
  const u32x2 c = *reinterpret_cast<const u32x2*>(src);
  stg16(packed + q * 8, e4m3x8_to_bf16x8(c[0], c[1]));
}

__global__ void k_pack_down_fp8_bf16(const uint8_t* __restrict__ wd, uint16_t* __restrict__ packed,
                                     int E, int d, int F) {
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
  const u32x2 c = *reinterpret_cast<const u32x2*>(wd + ((size_t)e * d + row) * F + kk);
  stg16(packed + q * 8, e4m3x8_to_bf16x8(c[0], c[1]));
}

// codes -> fp8 decode banks (16 bytes per lane: k-steps 2p and 2p+1)
__global__ void k_pack_gateup_fp8(const uint8_t* __restrict__ wg, const uint8_t* __restrict__ wu,
                                  uint8_t* __restrict__ packed, int E, int F, int d) {
  const size_t q = (size_t)blockIdx.x * 256 + threadIdx.x;
  const int kp = d / (2 * kKStep);
  const int nt = 2 * F / kTileRows;
  const size_t total = (size_t)E * nt * kp * 64;
  if (q >= total) return;
  const int lane = (int)(q % 64);
  size_t r = q / 64;
  const int p = (int)(r % kp);
  r /= kp;
  const int gt = (int)(r % nt);
  const int e = (int)(r / nt);
  const int rr = lane & 31;
  const int f = gt * 16 + (rr & 15);
  const uint8_t* row = (rr < 16 ? wg : wu) + ((size_t)e * F + f) * d;
  const int k0 = 2 * p * kKStep + (lane >> 5) * 8;
  u32x4 o;
  const u32x2 a = *reinterpret_cast<const u32x2*>(row + k0);
  const u32x2 b = *reinterpret_cast<const u32x2*>(row + k0 + kKStep);
  o[0] = a[0]; o[1] = a[1]; o[2] = b[0]; o[3] = b[1];
  stg16(packed + q * 16, o);
}

__global__ void k_pack_down_fp8(const uint8_t* __restrict__ wd, uint8_t* __restrict__ packed,
                                int E, int d, int F) {
  const size_t q = (size_t)blockIdx.x * 256 + threadIdx.x;
  const int kp = F / (2 * kKStep);
  const size_t total = (size_t)E * (d / kTileRows) * kp * 64;
  if (q >= total) return;
  const int lane = (int)(q % 64);
  size_t r = q / 64;
  const int p = (int)(r % kp);
  r /= kp;
  const int mt = (int)(r % (d / kTileRows));
  const int e = (int)(r / (d / kTileRows));
  const uint8_t* row = wd + ((size_t)e * d + mt * kTileRows + (lane & 31)) * F;
  const int k0 = 2 * p * kKStep + (lane >> 5) * 8;
  u32x4 o;
  const u32x2 a = *reinterpret_cast<const u32x2*>(row + k0);
  const u32x2 b = *reinterpret_cast<const u32x2*>(row + k0 + kKStep);
  o[0] = a[0]; o[1] = a[1]; o[2] = b[0]; o[3] = b[1];
  stg16(packed + q * 16, o);
}

// gate/up scales in the interleaved tile-row order: sgu[e][32 t + r] is the
// scale of row r of tile t (r < 16: gate column 16t + r; else up column 16t + r - 16)
__global__ void k_pack_gateup_scales(const float* __restrict__ sg, const float* __restrict__ su,
                                     float* __restrict__ sgu, int E, int F) {
  const size_t q = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= (size_t)E * 2 * F) return;
  const int e = (int)(q / (2 * F)), i = (int)(q % (2 * F));
  const int t = i / 32, r = i % 32;
  const int f = t * 16 + (r & 15);
  sgu[q] = (r < 16 ? sg : su)[(size_t)e * F + f];
}

hipError_t launch_pack_fp8(const uint8_t* w_gate, const uint8_t* w_up, const uint8_t* w_down,
                           const float* s_gate, const float* s_up, int E, int F, int d,
                           uint16_t* wgu16, uint16_t* wd16, uint8_t* wgu8, uint8_t* wd8,
                           float* sgu, hipStream_t s) {
  auto grid = [](size_t n) { return dim3((unsigned)((n + 255) / 256)); };
  const size_t n_gu16 = (size_t)E * (2 * F / kTileRows) * (d / kKStep) * 64;
  const size_t n_d16 = (size_t)E * (d / kTileRows) * (F / kKStep) * 64;
  if (wgu16 != nullptr)
    hipLaunchKernelGGL(k_pack_gateup_fp8_bf16, grid(n_gu16), dim3(256), 0, s, w_gate, w_up, wgu16, E, F, d);
  if (wd16 != nullptr)
    hipLaunchKernelGGL(k_pack_down_fp8_bf16, grid(n_d16), dim3(256), 0, s, w_down, wd16, E, d, F);
  hipLaunchKernelGGL(k_pack_gateup_fp8, grid(n_gu16 / 2), dim3(256), 0, s, w_gate, w_up, wgu8, E, F, d);
  hipLaunchKernelGGL(k_pack_down_fp8, grid(n_d16 / 2), dim3(256), 0, s, w_down, wd8, E, d, F);
  hipLaunchKernelGGL(k_pack_gateup_scales, grid((size_t)E * 2 * F), dim3(256), 0, s, s_gate, s_up, sgu, E, F);
  return hipGetLastError();
}

}  // namespace moe
