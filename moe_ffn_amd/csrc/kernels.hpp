// Host-side launchers of the MoE layer's kernels (private to the library).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Kernel slots of one forward (per-kernel timing).  Launch order: router,
// permutation, gather (bf16 prefill only), gate/up, [quantisation of the
// activations: fp8 activations only], down, combine.
enum Slot { kSlotNormRouter = 0, kSlotPermute = 1, kSlotExpertsA = 2, kSlotExpertsB = 3,
            kSlotCombine = 4, kSlotGather = 5, kSlotQuantAct = 6, kNumSlots = 7 };

// Optional start/stop events carried by a kernel's own dispatch packet.
struct KEv {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

// Plain launch unless per-kernel timing events are attached, so that a
// forward can be captured into a HIP graph.
template <typename F, typename... Args>
inline hipError_t launch(F kernel, dim3 grid, dim3 block, hipStream_t s, const KEv& ev,
                         Args... args) {
  if (ev.start == nullptr && ev.stop == nullptr)
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
  else
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, ev.start, ev.stop, 0, args...);
  return hipGetLastError();
}

// Packed expert-weight geometry (bf16).  Both banks are stored as 1 KiB blocks,
// one per (32-row tile, 16-wide k step), each block in MFMA 32x32x16 operand
// order: 64 lanes x 8 consecutive k of row (lane % 32), k-group (lane / 32).
//   W_gu : [E][2F/32 tiles][d/16 k-steps][64][8], tile t = gate rows of columns
//          16t .. 16t+15 then the up rows of the same columns (an MFMA output
//          lane holds gate(f) in element i and up(f) in element i + 8, i < 8)
//   W_d  : [E][d/32 m-tiles][F/16 k-steps][64][8]
constexpr int kTileRows = 32;
constexpr int kKStep = 16;
constexpr int kBlockElems = 64 * 8;  // 512 bf16 = 1 KiB

// Decode path is used while T * top_k is at most this many assignments.
constexpr int kStreamMaxAssign = 64;

struct LayerDims {
  int d, F, E, k, EP;  // EP = n_experts rounded up to a power of two
  float eps;
  int dtype;           // 0 = f32, 1 = bf16
  int act8 = 0;        // fp8 weights and fp8 activations (bf16 layers with fp8 banks)
};

struct FwdArgs {
  LayerDims dim;
  int T, n;            // tokens, assignments (T * k)
  const void* hidden;  // [T, d]
  void* out;           // [T, d]
  // bf16 layers in a stack: the residual stream [T, d] that the layer's output
  // is added to (out = bf16(res + bf16(y)), the layer output's rounding then
  // the sum's, as a separate add of the two bf16 rows would); null otherwise
  const void* res = nullptr;
  // layer-owned parameters
  const float* wrg;    // [EP, d] fp32: W_r[e][i] * g[i] (zero rows e >= E), fp32 layers
  const float* gain;   // [d] fp32
  const void* wr16;    // [E, d] bf16 router weights as given (bf16 layers)
  const void* gain16;  // [d] bf16 gain as given (bf16 layers)
  const float* bias;   // [E] fp32
  const void* wgu;     // packed gate/up bank (bf16) or canonical [E,F,d] (f32)
  const void* wup;     // f32 only: canonical up weights [E,F,d]
  const void* wd;      // packed down bank (bf16) or canonical [E,d,F] (f32)
  // fp8 layers (else null): E4M3 decode banks, per-row scales of gate/up (in
  // interleaved tile-row order, [E][2F]) and of down ([E][d]); the bf16 banks
  // then hold the code values and the scales multiply the accumulators
  const void* wgu8;
  const void* wd8;
  const float* sgu;
  const float* sd;
  // fp8 activations (dim.act8): E4M3 token and activation tiles in the fp8
  // banks' block order, and their per-row scales (one per padded slot); the
  // router's per-token scales of the gathered rows; the activations' per-row
  // partial maxima that the fp8 gate/up epilogue leaves for the quantiser,
  // [subtile][group][32 rows], groups of 16 * fp8_gateup_rt(F) columns
  void* xq = nullptr;
  void* actq = nullptr;
  float* sx = nullptr;
  float* sm = nullptr;
  float* xs_tok = nullptr;
  float* pmm = nullptr;
  // per-call buffers (workspace or caller-provided routing outputs)
  void* xn;            // [T, d] gain-scaled activations g * h (bf16 or f32)
  float* inv;          // [T] 1 / rms of each token's hidden state
  int* sel;            // [T, k]
  float* gate;         // [T, k]
  int* counts;         // [E]
  int* offsets;        // [E + 1]
  int* gather;         // [n]
  int* scatter;        // [n]
  int* slot_expert;    // [n]
  int* hist;           // [kPermuteMaxGroups][64] per-group expert counts (permutation scratch)
  void* xt;            // bf16 prefill: gathered token rows in operand tiles (k_gather_tiles.hip)
  void* act;           // [n, F] SwiGLU activations (decode, f32); operand tiles (bf16 prefill)
  float* ybuf;         // [n, d] fp32 expert outputs (k >= 2 only)
  const void* zrow;    // max(d, F) zero elements (16-byte aligned), read-only
  void* sink;          // max(d, F) elements that absorb stores of lanes without a token
  // depth averaging of the router logits across a stack's MoE layers (bf16
  // routers): eda = [max_tokens][64] fp32 state or null, z~ = eda_alpha *
  // state + (1 - eda_alpha) * z, the state read unless eda_first
  float* eda = nullptr;
  float eda_alpha = 0.f;
  int eda_first = 0;
  int num_cu;          // compute units of the device (persistent grids)
  hipStream_t stream;
  KEv ev[kNumSlots];   // per-kernel timing events (null when not timing)
};

hipError_t launch_norm_router(const FwdArgs& a);   // fp32 layers
hipError_t launch_router_mfma(const FwdArgs& a);   // bf16 layers, T*k > kStreamMaxAssign
hipError_t launch_router_token(const FwdArgs& a);  // bf16 layers, T*k <= kStreamMaxAssign
hipError_t launch_route_permute(const FwdArgs& a);
hipError_t launch_gather_tiles(const FwdArgs& a);
// 32-slot subtiles of all experts for n assignments, each expert padded to whole subtiles
int max_subtiles(int n, int E);
hipError_t launch_experts_stream(const FwdArgs& a);
hipError_t launch_experts_tile(const FwdArgs& a);
// weight tiles per wave of the fp8 gate/up GEMM (its activation column group is 16 * this)
inline int fp8_gateup_rt(int F) { return (2 * F) % 384 == 0 ? 3 : 2; }
hipError_t launch_experts_tile_fp8_gateup(const FwdArgs& a);  // dim.act8 layers
hipError_t launch_experts_tile_fp8_down(const FwdArgs& a);
// per-row E4M3 quantisation of the bf16 activation tiles (act -> actq, sm)
hipError_t launch_quant_act(const FwdArgs& a);
// the decode path's activation rows [n][F] in place: the E4M3 values as bf16, scales in sm
hipError_t launch_quant_act_rows(const FwdArgs& a);
// the same on row-major bf16 rows [R][K] (K % 8 == 0)
hipError_t launch_quant_rows(const void* x, int R, int K, void* codes, float* scale,
                             hipStream_t s);
hipError_t launch_experts_f32(const FwdArgs& a);
hipError_t launch_combine(const FwdArgs& a);

// balancing step on the router bias (between forwards)
constexpr int kPermuteMaxGroups = 256;  // workgroups of the permutation, at most
hipError_t launch_bias_update(const int* counts, int E, float rate, float* bias, hipStream_t s);

// residual add of an fp32 FFN stack: out = h + y (n elements; bf16 layers add
// theirs in their last kernel, FwdArgs::res)
hipError_t launch_residual_f32(const float* h, const float* y, float* out, size_t n,
                               hipStream_t s);

// zero fill by a kernel (graph-capturable): bytes a multiple of 16, p 16-byte aligned
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);

// create-time packing
hipError_t launch_pack_gateup(const uint16_t* w_gate, const uint16_t* w_up, uint16_t* packed, int E,
                              int F, int d, hipStream_t s);
hipError_t launch_pack_down(const uint16_t* w_down, uint16_t* packed, int E, int d, int F,
                            hipStream_t s);
// wgu16 / wd16 null: only the fp8 banks and the gate/up scales
hipError_t launch_pack_fp8(const uint8_t* w_gate, const uint8_t* w_up, const uint8_t* w_down,
                           const float* s_gate, const float* s_up, int E, int F, int d,
                           uint16_t* wgu16, uint16_t* wd16, uint8_t* wgu8, uint8_t* wd8,
                           float* sgu, hipStream_t s);
hipError_t launch_prep_router(const void* w_router, const void* gain, int dtype, int E, int EP,
                              int d, float* wrg, float* gain32, hipStream_t s);

}  // namespace moe
