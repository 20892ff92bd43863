/*
 * moe_layer.h - C ABI of one ZONOS2 MoE feed-forward layer on an MI355X (gfx950).
 *
 * The layer (ZONOS2 Technical Report, audio-paper-digest page, "Method overview
 * and architecture", item 5: an RMSNorm-normalised input, 16 experts per MoE
 * layer with top-1 routing and top-2 in the last MoE layer; item 6: a per-expert
 * bias vector b_l; mlsanity index page, "Builds on": RMSNorm, GLU variants and
 * auxiliary-loss-free load balancing) computes, for every token t of a batch:
 *
 *   x_t   = g * h_t / sqrt(mean(h_t^2) + eps)                       RMSNorm
 *   z_t   = W_r x_t,  s_t = z_t + b                               router logits / scores
 *   sel_t = top-k experts of s_t (descending s, ties to the lower index)
 *   gate  = softmax(z_t)[sel] for k = 1; softmax of z_t over sel for k >= 2
 *   y     = W_down[e] (SiLU(W_gate[e] x_t) * (W_up[e] x_t))  for each e in sel_t
 *   out_t = sum_j gate_{t,j} y_{t,j}            (the residual is NOT added)
 *
 * The bias b steers which experts are chosen; it never enters a gate.
 *
 * Conventions
 *   - Every pointer argument named as device memory must be a HIP device
 *     pointer (or managed memory) on the device that is current when the call
 *     is made, 16-byte aligned, and laid out row-major as stated.
 *   - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 *   - Calls return a moe_status_t; nothing throws across the ABI.  On failure
 *     moe_last_error() returns a message for the calling thread.
 *   - Device faults inside launched kernels surface at the caller's next
 *     synchronisation, as for any asynchronous HIP work.  With the environment
 *     variable MOE_DEBUG_SYNC=1 every forward synchronises its stream and maps
 *     a failure to MOE_ERR_HIP.
 */
#ifndef MOE_LAYER_H
#define MOE_LAYER_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 6

typedef struct moe_layer moe_layer_t; /* opaque; owned by the library */

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* a NULL, misaligned or out-of-range argument */
  MOE_ERR_OOM = 2,         /* a device allocation failed */
  MOE_ERR_HIP = 3,         /* a HIP runtime call or kernel launch failed */
  MOE_ERR_UNSUPPORTED = 4  /* a shape or device the kernels do not cover */
} moe_status_t;

typedef enum { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1 } moe_dtype_t;

/* Layer shape.  Limits: 1 <= n_experts <= 64; 1 <= top_k <= min(n_experts, 8);
 * bf16: d_model a multiple of 256 and d_ff of 128 (of 256 with fp8 expert
 * weights), both at most 65536; f32: both multiples of 4; 1 <= max_tokens <=
 * 2^20.
 * dtype is the storage type of activations, gain, router and expert weights;
 * arithmetic accumulates in fp32 either way. */
typedef struct {
  int32_t d_model;
  int32_t d_ff;
  int32_t n_experts;
  int32_t top_k;
  int32_t dtype;      /* moe_dtype_t */
  float rms_eps;      /* e.g. 1e-6 */
  int32_t max_tokens; /* workspace is sized for this many tokens per forward */
} moe_layer_config_t;

/* Weights, DEVICE pointers in the config's dtype (b_router is always fp32),
 * canonical row-major layouts.  They are read during moe_layer_create only:
 * the library copies and repacks them into memory it owns, on `stream`; the
 * caller may free them once that stream has been synchronised. */
typedef struct {
  const void* rms_gain;   /* [d_model]                 g   */
  const void* w_router;   /* [n_experts, d_model]      W_r */
  const float* b_router;  /* [n_experts] fp32           b   */
  const void* w_gate;     /* [n_experts, d_ff, d_model]    */
  const void* w_up;       /* [n_experts, d_ff, d_model]    */
  const void* w_down;     /* [n_experts, d_model, d_ff]    */
} moe_layer_weights_t;

/* Optional routing outputs of one forward, DEVICE pointers owned by the caller.
 * Any member may be NULL (that output is then not written).  Sizes for a call
 * with T tokens: sel, gate [T, top_k]; counts [n_experts]; offsets
 * [n_experts + 1]; gather, scatter [T * top_k].
 *   sel[t,j]    expert of assignment a = t*top_k + j (descending score)
 *   gate[t,j]   its gate weight
 *   counts[e]   assignments routed to expert e; offsets = exclusive prefix sum
 *   gather[p]   token of expert-ordered slot p (stable: increasing a per expert)
 *   scatter[a]  slot of assignment a  (gather[scatter[a]] == a / top_k)       */
typedef struct {
  int32_t* sel;
  float* gate;
  int32_t* counts;
  int32_t* offsets;
  int32_t* gather;
  int32_t* scatter;
} moe_routing_out_t;

/* Returns MOE_ABI_VERSION of the loaded library. */
int32_t moe_abi_version(void);

/* Message of the last failure on the calling thread ("" if none).  The string
 * stays valid until the next call into the library from this thread. */
const char* moe_last_error(void);

/* Create a layer on the current device.  Validates `cfg`, allocates the packed
 * weight bank and a workspace sized for cfg->max_tokens, and enqueues the
 * weight packing on `stream`.  On success *out receives the handle; on failure
 * *out is set to NULL and nothing stays allocated.
 * Errors: INVALID_ARG (NULL pointer, bad config, misaligned weight pointer),
 * UNSUPPORTED (shape outside the limits above, device is not gfx950),
 * OOM, HIP. */
moe_status_t moe_layer_create(const moe_layer_config_t* cfg, const moe_layer_weights_t* w,
                              void* stream, moe_layer_t** out);

/* Expert weights as OCP FP8 E4M3 codes (the SGLang-Omni ZONOS2 cookbook page,
 * "Benchmark Results", serves the model with "fp8" and names nothing more; this
 * ABI reads it as weight-only fp8 with bf16 activations.  E4M3: sign, 4
 * exponent bits with bias 7, 3 mantissa bits, no infinities) with one fp32
 * scale per output row: W_gate[e][f][:] = value(code) * gate[e*F + f], W_up
 * likewise with up, W_down[e][m][:] = value(code) * down[e*d + m].
 * All DEVICE pointers, 4-byte aligned, borrowed for the duration of create. */
typedef struct {
  const float* gate;  /* [E, F] */
  const float* up;    /* [E, F] */
  const float* down;  /* [E, d] */
} moe_fp8_scales_t;

/* As moe_layer_create, with w->w_gate, w_up, w_down pointing to uint8 E4M3
 * codes ([E,F,d], [E,F,d], [E,d,F], 16-byte aligned) and `scales` giving their
 * per-row scales; cfg->dtype must be MOE_DTYPE_BF16 (bf16 activations, gain
 * and router) and d_ff a multiple of 256.  Decode-sized batches
 * (T * top_k <= 64) stream the codes (half the bytes of bf16); larger batches
 * run the bf16 MFMA GEMMs on the codes' values (every E4M3 value is a bf16
 * value).  In both the scales multiply the fp32 accumulators, so no weight
 * value is rounded.  The layer keeps both banks: 3 bytes per expert weight.
 * Errors: as moe_layer_create; INVALID_ARG also for NULL `scales`, a NULL or
 * misaligned scale pointer or an F32 dtype; UNSUPPORTED for d_ff % 256 != 0. */
moe_status_t moe_layer_create_fp8(const moe_layer_config_t* cfg, const moe_layer_weights_t* w,
                                  const moe_fp8_scales_t* scales, void* stream,
                                  moe_layer_t** out);

/* fp8 weights AND fp8 activations (the cookbook page's "fp8" read as both GEMM
 * operands in E4M3, so the expert products run on gfx950's fp8 MFMA,
 * v_mfma_f32_32x32x64_f8f6f4).  Weights and scales as for
 * moe_layer_create_fp8.  In every forward, each routed row u of the expert
 * input (the bf16 RMSNorm output) and each row m = SiLU(G) * V of the SwiGLU
 * intermediate (rounded to bf16) is quantised to E4M3 with one dynamic fp32
 * scale per row, exactly as moe_fp8_quantize_rows does; the weight scales and
 * the row scales multiply the fp32 accumulators:
 *   G[r, f] = a_u[r] * s_gate[f] * sum_i code(u_r)_i * code(W_gate[f])_i   (V likewise)
 *   y[r, m] = a_m[r] * s_down[m] * sum_f code(m_r)_f * code(W_down[m])_f
 * Router, gates, dispatch and combine are those of the bf16 layer.  Batches
 * with T * top_k > 64 run the tiled path (router, permutation, the gather that
 * quantises the rows, the fp8 gate/up GEMM, the quantisation of the
 * intermediate, the fp8 down GEMM); decode-sized batches stream the fp8
 * weights against the exact E4M3 values of the quantised rows (bf16 matrix
 * operands; the same products), with the same scales.  The layer keeps only
 * the fp8 banks: 1 byte per expert weight plus the row scales.  Shape limits
 * and errors as moe_layer_create_fp8. */
moe_status_t moe_layer_create_w8a8(const moe_layer_config_t* cfg, const moe_layer_weights_t* w,
                                   const moe_fp8_scales_t* scales, void* stream,
                                   moe_layer_t** out);

/* Per-row E4M3 quantisation with a dynamic scale, the step that layers made by
 * moe_layer_create_w8a8 apply to their expert inputs and SwiGLU intermediates
 * (for callers that quantise activations themselves, and to check the step).
 * x: DEVICE bf16 [R, K] (16-byte aligned, K a multiple of 8); codes: DEVICE
 * uint8 [R, K] (8-byte aligned) receives OCP E4M3 codes; scales: DEVICE fp32
 * [R] (4-byte aligned).  Row r: a = max_i |x[r,i]| / 448 and its reciprocal
 * q = 1 / a in fp32 (correctly rounded divisions), code(x) = the E4M3 value
 * nearest to fl32(x * q) (ties to the even code; |x * q| is at most 448 up to
 * rounding and is clamped to +-448); a row of zeros gives a = 0 and codes 0.  Then
 * x[r,i] ~= a * value(code).  Enqueued on `stream`; R == 0 does nothing.
 * NaN or Inf inputs give undefined codes.  Errors: INVALID_ARG (NULL or
 * misaligned pointers, R < 0, K not a positive multiple of 8), HIP. */
moe_status_t moe_fp8_quantize_rows(const void* x, int32_t R, int32_t K, void* codes,
                                   float* scales, void* stream);

/* One forward over T tokens: hidden [T, d_model] -> out [T, d_model], both
 * DEVICE memory in the layer's dtype; `out` must not overlap `hidden`.
 * Asynchronous on `stream`: no host synchronisation and no allocation.
 * T == 0 returns MOE_OK and launches nothing.  `routing` may be NULL.
 * A handle must not run two forwards concurrently (on two streams): they share
 * the layer's workspace.  Inputs with NaN or Inf give undefined values in
 * `out` but every index stays in range.
 * Errors: INVALID_ARG (NULL handle/pointers, T < 0, T > max_tokens, misaligned
 * or overlapping buffers), HIP (launch failure). */
moe_status_t moe_layer_forward(moe_layer_t* layer, const void* hidden, int32_t T, void* out,
                               void* stream, const moe_routing_out_t* routing);

/* As moe_layer_forward, for callers that cannot allocate device memory at the
 * time of the call (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the forward's per-call buffers (router
 * outputs, dispatch arrays, token and activation tiles) come from one static
 * 16 MiB device array of the library instead of the layer's workspace, and
 * nothing is allocated or freed.  The array is per device and shared by every
 * call on that device: it keeps the last call's contents, the parts that must
 * start at zero are cleared by a kernel at the start of each call, and calls
 * that overlap on one device (on two streams, or with two host threads) race.
 * Sizes: the buffers needed for T tokens must fit in 16 MiB (at d_model 2048,
 * d_ff 3072 and 16 experts: T up to 815 with top-1, 286 with top-2; layers
 * with fp8 activations carve other buffers: 699 and 249); larger T
 * is rejected with INVALID_ARG and a message giving the bytes needed.  Outputs and routing are
 * those moe_layer_forward gives for the same arguments.
 * Errors: as moe_layer_forward; INVALID_ARG also when T needs more scratch. */
moe_status_t moe_layer_forward_static(moe_layer_t* layer, const void* hidden, int32_t T,
                                      void* out, void* stream, const moe_routing_out_t* routing);

/* Replace the router bias b with n_experts fp32 values from DEVICE memory,
 * enqueued on `stream` (the update is ordered with forwards on that stream).
 * Errors: INVALID_ARG, HIP. */
moe_status_t moe_layer_set_bias(moe_layer_t* layer, const float* b_router, void* stream);

/* Copy the layer's current router bias (n_experts fp32) into DEVICE memory
 * b_out (4-byte aligned), enqueued on `stream`.  Errors: INVALID_ARG, HIP. */
moe_status_t moe_layer_get_bias(moe_layer_t* layer, float* b_out, void* stream);

/* One step of auxiliary-loss-free load balancing on the router bias (the
 * ZONOS2 report keeps b_l to push expert usage toward uniform, digest item 6;
 * the step is that of the auxiliary-loss-free load-balancing paper listed on
 * the index page's "Builds on" list):
 *   b_e <- b_e + rate * sign(mean(c) - c_e),  e = 0 .. n_experts-1,
 * the sign taken exactly as the sign of the integer sum(c) - n_experts * c_e
 * (0 leaves b_e unchanged), the float32 sum b_e + rate * sign rounded once.
 *   counts  DEVICE int32[n_experts], 4-byte aligned: assignment counts of a
 *           batch (e.g. moe_routing_out_t.counts of a forward).  NULL means the
 *           layer's own counts buffer, which holds the counts of the latest
 *           forward whose routing argument was NULL or had a NULL counts.
 *   rate    the step size (finite; negative values push away from balance).
 * Enqueued on `stream` after the forward that produced the counts; the next
 * forward on that stream routes with the updated bias.  Nothing is
 * allocated; the host is not synchronised.  Errors: INVALID_ARG, HIP. */
moe_status_t moe_layer_update_bias(moe_layer_t* layer, const int32_t* counts, float rate,
                                   void* stream);

/* Per-kernel timing, for measurement tools.  moe_layer_timing_start() makes
 * the next `max_forwards` forwards launch every kernel with a start and a stop
 * HIP event carried by the kernel's own dispatch (no extra packets on the
 * stream).  moe_layer_timing_stop() waits for those events, writes into
 * ms_sum[MOE_TIMED_SLOTS] each slot's summed kernel milliseconds and into
 * *n_forwards the number of forwards recorded, then releases the events.
 * Slots: 0 RMSNorm+router+top-k, 1 histogram+permutation (0 for bf16 layers
 * with T*top_k <= 64, whose expert kernels dispatch), 2 first expert kernel
 * (gate/up), 3 second expert kernel (down), 4 combine (0 when top_k = 1, where
 * the combine is part of slot 3), 5 gather of the routed rows into expert
 * order (bf16 layers with T*top_k > 64 and fp8-activation layers, whose
 * gather also quantises the rows; it runs between slots 1 and 2), 6
 * quantisation of the SwiGLU intermediate (fp8-activation layers only; between
 * slots 2 and 3).
 * Errors: INVALID_ARG (bad handle, max_forwards outside [1, 65536], stop
 * without start), HIP. */
#define MOE_TIMED_SLOTS 7
moe_status_t moe_layer_timing_start(moe_layer_t* layer, int32_t max_forwards);
moe_status_t moe_layer_timing_stop(moe_layer_t* layer, float* ms_sum, int32_t* n_forwards);

/* ---- FFN stack ------------------------------------------------------------
 * The feed-forward half of the backbone's layers in order (digest item 5: a
 * 28-layer stack, the first three and the last one dense, the middle ones MoE,
 * top-1 except the last MoE layer, top-2), each followed by its residual add:
 *   h_0 = hidden_in;  h_{l+1} = h_l + FFN_l(h_l);  hidden_out = h_L,
 * the sum rounded once to the activations' type (bf16: round to nearest even
 * of the fp32 sum of the two bf16 values).  A dense layer is a layer created
 * with n_experts = top_k = 1.  Attention and the rest of each layer are not
 * part of the stack. */
typedef struct moe_stack moe_stack_t;

/* layers: n_layers handles (1..4096) created by moe_layer_create on the
 * current device, all with the same d_model and dtype and max_tokens >=
 * max_tokens; BORROWED: they must outlive the stack, which never destroys
 * them.  The stack allocates two residual buffers and one FFN output buffer of
 * [max_tokens, d_model] and, for bf16 layers, the [max_tokens, 64] fp32 router
 * state of moe_stack_set_eda.  Errors: INVALID_ARG, OOM, HIP. */
moe_status_t moe_stack_create(int32_t n_layers, moe_layer_t* const* layers, int32_t max_tokens,
                              moe_stack_t** out);

/* Exponential depth averaging of the router state across the stack's MoE
 * layers (those with n_experts > 1), in stack order.  ZONOS2 digest (audio-
 * paper-digest page, "Method overview and architecture", item 5): the router
 * follows ZAYA1 in smoothing its state between layers by exponential depth
 * averaging; the page defines neither the state nor the rate.  This library
 * reads the state as the router logits z (before the bias) and applies, per
 * token and expert, z~_l = alpha * z~_{l-1} + (1 - alpha) * z_l with z~ = z
 * at the first MoE layer; selection uses z~ + b_l and the gates use z~.
 * enable = 0 turns it off (the default); alpha in [0, 1) is the caller's
 * (alpha = 0 gives the plain routing).  The state is a [max_tokens, 64] fp32
 * buffer the stack allocated at create; a later moe_stack_forward or capture
 * uses the setting current at that call.  The averaged logit of expert e
 * passes from one MoE layer to the next, so every MoE layer of the stack must
 * have the same n_experts.  Errors: INVALID_ARG (handle, alpha, MoE layers
 * with different n_experts; moe_stack_forward and moe_stack_capture check the
 * last again), UNSUPPORTED (fp32 layers). */
moe_status_t moe_stack_set_eda(moe_stack_t* stack, int32_t enable, float alpha);

/* One pass through the stack, enqueued on `stream` (no host synchronisation,
 * no allocation).  hidden_in / hidden_out: DEVICE [T, d_model] of the layers'
 * dtype, 16-byte aligned; hidden_out may equal hidden_in.  T in [0, max_tokens].
 * The layers' workspaces and the stack's buffers are shared by every call:
 * calls that overlap (on two streams) race.  Errors: INVALID_ARG, HIP. */
moe_status_t moe_stack_forward(moe_stack_t* stack, const void* hidden_in, int32_t T,
                               void* hidden_out, void* stream);

/* As moe_stack_forward, and also writes each layer's routing of this pass:
 * routing points to n_layers moe_routing_out_t structs in HOST memory, the
 * l-th naming (as for moe_layer_forward) DEVICE buffers for layer l, each
 * member NULL or sized for T tokens and that layer's top_k and n_experts.
 * Meant for checking a stack's routing layer by layer (for instance with
 * depth averaging on).  Errors: as moe_stack_forward; INVALID_ARG for a NULL
 * `routing` or a misaligned routing buffer. */
moe_status_t moe_stack_forward_routing(moe_stack_t* stack, const void* hidden_in, int32_t T,
                                       void* hidden_out, void* stream,
                                       const moe_routing_out_t* routing);

/* Record the launch sequence of moe_stack_forward(stack, hidden_in, T,
 * hidden_out) on `stream` (a created stream, not NULL) into a HIP graph owned
 * by the stack, replacing any earlier one; nothing runs.  moe_stack_replay()
 * launches the recorded graph on a stream: the same pointers, T and layer
 * parameters at replay time (a bias changed in between is used).  Layers with
 * per-kernel timing on cannot be recorded.  Errors: INVALID_ARG, HIP. */
moe_status_t moe_stack_capture(moe_stack_t* stack, const void* hidden_in, int32_t T,
                               void* hidden_out, void* stream);
moe_status_t moe_stack_replay(moe_stack_t* stack, void* stream);

/* Release the stack (NULL-safe) after synchronising the device; the layers
 * stay valid. */
void moe_stack_destroy(moe_stack_t* stack);

/* Release the layer (NULL-safe).  Synchronises the device first, so work still
 * in flight on any stream that uses the layer completes before its memory goes. */
void moe_layer_destroy(moe_layer_t* layer);

#ifdef __cplusplus
}
#endif

#endif /* MOE_LAYER_H */
