// Device-side helpers shared by the MoE layer's HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
// Two fp32 -> one word of two bf16 (lo in the low half), round to nearest even:
// one v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// Unpack 8 bf16 held in a 16-byte vector into fp32.
__device__ __forceinline__ void unpack8(const u32x4& v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(v[i]);
    f[2 * i + 1] = bf16_hi(v[i]);
  }
}

__device__ __forceinline__ u32x4 ldg16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void stg16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }

// Streaming load for data read exactly once (expert weights): bypass reuse in L2/MALL.
__device__ __forceinline__ u32x4 ldg16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
// Non-temporal stores for large intermediates that the next kernel reads back
// (prefill token tiles and activation tiles): they do not stay dirty in the
// writing XCD's L2.  Measured on the prefill workloads: the GEMMs that read
// them back ran 3-9% faster than with ordinary stores; the layer's output
// rows, stored the same way, made the down projection 20-40% slower.
__device__ __forceinline__ void stg16_stream(void* p, const u32x4& v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void stg8_stream(void* p, const u32x2& v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p));
}

// D = A * B + C on a 32x32 output tile with K = 16, bf16 inputs, fp32 accumulation.
// Operand lane layout: lane l carries row (l % 32) of A (column (l % 32) of B) and
// the 8 consecutive k values of k-group (l / 32).  Output lane layout: lane l holds
// column (l % 32), rows 8*(i/4) + 4*(l/32) + (i%4) for accumulator element i.
__device__ __forceinline__ f32x16 mfma_32x32x16(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// D = A * B + C on a 32x32 output tile with K = 64, both operands OCP E4M3
// (v_mfma_f32_32x32x64_f8f6f4; the scaled form with zero scale operands is the
// plain instruction), fp32 accumulation.  Each operand is 32 bytes per lane,
// given as two 16-byte halves; A and B use the same lane order, so any fixed
// assignment of k to (lane / 32, byte) that both operands share gives the
// same sums.  The output lane layout is that of mfma_32x32x16.
__device__ __forceinline__ f32x16 mfma_32x32x64_fp8(const u32x4& a0, const u32x4& a1,
                                                    const u32x4& b0, const u32x4& b1,
                                                    const f32x16& c) {
  typedef int i32x8 __attribute__((ext_vector_type(8)));
  const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                   (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
  const i32x8 b = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3],
                   (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
__device__ __forceinline__ int c32_row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

// SiLU(v) = v * sigmoid(v), the reciprocal from v_rcp_f32 (1 ulp) instead of an
// IEEE division (a ten-instruction sequence); the result is rounded to bf16.
__device__ __forceinline__ float silu(float v) {
  return v * __builtin_amdgcn_rcpf(1.0f + __expf(-v));
}

// Butterfly reduction of N per-lane values over the 64 lanes of a wave that
// leaves the sums spread over the lanes instead of replicated: each halving
// step exchanges half of the remaining values with the partner lane.
// Afterwards lane l holds, in v[0 .. max(N/64,1)-1], the full sums of value
// indices spread_index<N>(l, i).
template <int N, int DELTA>
struct WaveSpread {
  static __device__ __forceinline__ void run(float* v, int lane) {
    if constexpr (DELTA == 0) {
      return;
    } else if constexpr (N > 1) {
      constexpr int H = N / 2;
      const bool upper = (lane & DELTA) != 0;
#pragma unroll
      for (int i = 0; i < H; ++i) {
        const float send = upper ? v[i] : v[i + H];
        const float keep = upper ? v[i + H] : v[i];
        v[i] = keep + __shfl_xor(send, DELTA, kWave);
      }
      WaveSpread<H, DELTA / 2>::run(v, lane);
    } else {
      v[0] += __shfl_xor(v[0], DELTA, kWave);
      WaveSpread<1, DELTA / 2>::run(v, lane);
    }
  }
};

constexpr int ilog2(int n) { return n <= 1 ? 0 : 1 + ilog2(n / 2); }

template <int N>
__device__ __forceinline__ int spread_index(int lane, int i) {
  constexpr int L = ilog2(N);
  if constexpr (L >= 6) return (lane << (L - 6)) + i;
  else return lane >> (6 - L);
}
// True for the lanes that own distinct sums (one owner per index when N < 64).
template <int N>
__device__ __forceinline__ bool spread_owner(int lane) {
  constexpr int L = ilog2(N);
  if constexpr (L >= 6) return true;
  else return (lane & ((1 << (6 - L)) - 1)) == 0;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Four OCP E4M3 codes (bytes of `four`) -> two of them as bf16x2 bits: the
// low two bytes (HI = false) or the high two (HI = true).  The hardware
// conversion to fp32 is exact and every E4M3 value fits bf16, so the high
// halves of the fp32 results are the exact bf16 values.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3_pair_to_bf16x2(uint32_t four) {
  const auto f = __builtin_amdgcn_cvt_pk_f32_fp8((int)four, HI);
  return (__float_as_uint(f[0]) >> 16) | (__float_as_uint(f[1]) & 0xffff0000u);
}
// 8 codes (u32x2) -> 8 bf16 operand values (u32x4)
__device__ __forceinline__ u32x4 e4m3x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  u32x4 o;
  o[0] = e4m3_pair_to_bf16x2<false>(lo);
  o[1] = e4m3_pair_to_bf16x2<true>(lo);
  o[2] = e4m3_pair_to_bf16x2<false>(hi);
  o[3] = e4m3_pair_to_bf16x2<true>(hi);
  return o;
}

// Per-row E4M3 quantisation with a dynamic scale (fp8 activations): with a
// = max|row| / 448 and r = 1 / a (fp32, correctly rounded divisions, once per
// row: e4m3_recip), the code of v is the E4M3 nearest to fl32(v * r)
// (v_cvt_pk_fp8_f32 rounds to nearest even), clamped to +-448 first (|v * r|
// exceeds 448 by at most a few roundings, which the clamp takes back to the
// value round-to-nearest gives); a = 0 (a zero row) gives code 0.
__device__ __forceinline__ float e4m3_recip(float a) { return a > 0.f ? 1.f / a : 0.f; }
__device__ __forceinline__ float e4m3_quotient(float v, float r) {
  return r > 0.f ? fminf(fmaxf(v * r, -448.f), 448.f) : 0.f;
}
// four bf16 values (two bf16x2 words) -> four codes, in order, in one word;
// r = e4m3_recip(a)
__device__ __forceinline__ uint32_t quant4_e4m3(uint32_t w0, uint32_t w1, float r) {
  uint32_t c = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_quotient(bf16_lo(w0), r),
                                               e4m3_quotient(bf16_hi(w0), r), 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_quotient(bf16_lo(w1), r),
                                         e4m3_quotient(bf16_hi(w1), r), (int)c, true);
}
__device__ __forceinline__ float absmax8_bf16(const u32x4& v, float m) {
#pragma unroll
  for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaxf(fabsf(bf16_lo(v[i])), fabsf(bf16_hi(v[i]))));
  return m;
}

}  // namespace moe
