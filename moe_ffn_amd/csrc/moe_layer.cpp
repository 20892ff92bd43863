// C ABI of the ZONOS2 MoE feed-forward layer: validation, device memory, the
// create-time weight packing and the launch sequence of one forward.
//
// Forward on one stream, no host synchronisation, no allocation:
// bf16 layers, decode-sized batches (T * top_k <= 64):
//   K1 per-token RMSNorm + router + top-k + gates (k_router_token.hip)
//   K3 weight-streaming gate/up and down kernels, each workgroup deriving its
//      expert's dispatch from the routing choice (k_expert_stream.hip)
// bf16 layers, larger batches:
//   K1 RMSNorm statistics + router on bf16 MFMA + top-k + gates (k_router_mfma.hip)
//   K2 per-group expert histograms, then the stable permutation from their
//      prefix (two launches, k_route_permute.hip); the routed rows normalised
//      and gathered into expert-ordered operand tiles (k_gather_tiles.hip)
//   K3 LDS-staged grouped GEMMs, gate/up with SiLU epilogue then down (k_expert_gemm.hip)
// fp32 layers: VALU router (k_norm_router.hip), K2, VALU experts (k_expert_f32.hip)
//   K4 gate-weighted combine (k >= 2; folded into K3 for k = 1)
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "kernels.hpp"
#include "moe_layer.h"

namespace {

thread_local std::string g_err;
constexpr uint32_t kMagic = 0x314d6f45u;  // "EoM1"
constexpr int kMaxTokensLimit = 1 << 20;
constexpr int kMaxWidth = 1 << 16;  // bf16 d_model and d_ff

moe_status_t fail(moe_status_t st, const std::string& msg) {
  g_err = msg;
  return st;
}
moe_status_t hip_fail(hipError_t e, const char* what) {
  return fail(MOE_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
int next_pow2(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}
size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Carves sub-buffers out of one allocation, 256-byte aligned.
struct Carver {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  }
};

// Per-call buffers of one forward (device memory): the layer's workspace, or
// the library's static scratch array for moe_layer_forward_static.
struct Work {
  void* xn;
  float* inv;
  int* sel;
  float* gate;
  int* counts;
  int* offsets;
  int* gather;
  int* scatter;
  int* slot_expert;
  int* hist;
  void* xt;
  void* act;
  void* xq;    // fp8 activations: E4M3 token tiles, activation tiles, their row scales
  void* actq;
  float* sx;
  float* sm;
  float* xs_tok;  // per-token quantisation scales of the gathered rows (router)
  float* pmm;     // partial row maxima of the activations (fp8 gate/up epilogue)
  float* ybuf;
  void* zrow;  // max(d, F) zero elements: must hold zeros before a forward runs
  void* sink;
  size_t zbytes;
  bool clear_zrow;  // zero zrow at the start of the forward (shared static scratch)
};

// Lay out the buffers of a forward over up to `tokens` tokens from `base`
// (nullptr: only measure); returns the bytes needed.
size_t carve_work(const moe::LayerDims& dim, size_t tokens, char* base, Work* w) {
  const size_t d = dim.d, F = dim.F, E = dim.E, k = dim.k;
  const bool bf16 = dim.dtype == MOE_DTYPE_BF16;
  const size_t es = bf16 ? 2 : 4;
  const size_t nmax = tokens * k;
  Carver wc;
  const size_t o_xn = wc.take(tokens * d * es);
  const size_t o_inv = wc.take(tokens * 4);
  const size_t o_sel = wc.take(nmax * 4);
  const size_t o_gate = wc.take(nmax * 4);
  const size_t o_cnt = wc.take(E * 4);
  const size_t o_off = wc.take((E + 1) * 4);
  const size_t o_gat = wc.take(nmax * 4);
  const size_t o_sca = wc.take(nmax * 4);
  const size_t o_sle = wc.take(nmax * 4);
  const size_t o_hist = wc.take((size_t)moe::kPermuteMaxGroups * 64 * 4);
  // bf16: slot-ordered activations (decode) or padded operand tiles (prefill)
  const size_t npad = bf16 ? (size_t)moe::max_subtiles((int)nmax, (int)E) * 32 : 0;
  const bool a8 = dim.act8 != 0;  // fp8 activations: E4M3 token tiles instead of bf16 ones
  const size_t o_xt = bf16 && !a8 ? wc.take(npad * d * 2) : 0;
  const size_t o_act = wc.take((nmax > npad ? nmax : npad) * F * es);
  const size_t o_xq = a8 ? wc.take(npad * d) : 0;
  const size_t o_actq = a8 ? wc.take(npad * F) : 0;
  const size_t o_sx = a8 ? wc.take(npad * 4) : 0;
  const size_t o_sm = a8 ? wc.take(npad * 4) : 0;
  const size_t o_xst = a8 ? wc.take(tokens * 4) : 0;
  const size_t o_pmm = a8 ? wc.take(npad * (F / 32) * 4) : 0;  // groups of 32 or 48 columns
  const size_t o_y = k > 1 ? wc.take(nmax * d * 4) : 0;
  const size_t zbytes = (d > F ? d : F) * 4;
  const size_t o_z = wc.take(zbytes);
  const size_t o_sink = wc.take(zbytes);
  if (base != nullptr) {
    w->xn = base + o_xn;
    w->inv = reinterpret_cast<float*>(base + o_inv);
    w->sel = reinterpret_cast<int*>(base + o_sel);
    w->gate = reinterpret_cast<float*>(base + o_gate);
    w->counts = reinterpret_cast<int*>(base + o_cnt);
    w->offsets = reinterpret_cast<int*>(base + o_off);
    w->gather = reinterpret_cast<int*>(base + o_gat);
    w->scatter = reinterpret_cast<int*>(base + o_sca);
    w->slot_expert = reinterpret_cast<int*>(base + o_sle);
    w->hist = reinterpret_cast<int*>(base + o_hist);
    w->xt = bf16 && !a8 ? base + o_xt : nullptr;
    w->act = base + o_act;
    w->xq = a8 ? base + o_xq : nullptr;
    w->actq = a8 ? base + o_actq : nullptr;
    w->sx = a8 ? reinterpret_cast<float*>(base + o_sx) : nullptr;
    w->sm = a8 ? reinterpret_cast<float*>(base + o_sm) : nullptr;
    w->xs_tok = a8 ? reinterpret_cast<float*>(base + o_xst) : nullptr;
    w->pmm = a8 ? reinterpret_cast<float*>(base + o_pmm) : nullptr;
    w->ybuf = k > 1 ? reinterpret_cast<float*>(base + o_y) : nullptr;
    w->zrow = base + o_z;
    w->sink = base + o_sink;
    w->zbytes = zbytes;
    w->clear_zrow = false;
  }
  return wc.off;
}

// ---------------------------------------------------------------------------
// Static scratch for moe_layer_forward_static: a forward's per-call buffers
// for callers that cannot allocate device memory.  Every device the library
// runs on holds its own copy of this array until the process ends; on the
// host `scratch` names a host-side stand-in, so the device address of each
// device's copy is looked up once (with that device current) and kept.
constexpr size_t kScratchBytes = size_t(16) << 20;  // 16 MiB
constexpr int kMaxDevices = 64;
}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device (null: not looked up)

// Looks up this device's copy of `scratch` if not done yet; `dev` must be the
// current device.
moe_status_t scratch_setup(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device index above 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] != nullptr) return MOE_OK;
  void* p = nullptr;
  const hipError_t he = hipGetSymbolAddress((void**)&p, HIP_SYMBOL(scratch));
  if (he != hipSuccess || p == nullptr) {
    (void)hipGetLastError();
    return hip_fail(he != hipSuccess ? he : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
  }
  g_scratch_ptr[dev] = p;
  return MOE_OK;
}

void* scratch_base(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return g_scratch_ptr[dev];
}

}  // namespace

struct moe_layer {
  uint32_t magic;
  moe::LayerDims dim;
  int max_tokens;
  int device;
  int num_cu;
  bool debug_sync;
  // parameters (one allocation)
  void* params;
  float* wrg;
  float* gain32;
  float* bias;
  void* wr16;
  void* gain16;
  void* wgu;
  void* wup;
  void* wd;
  // fp8 layers: decode banks and per-row scales (null otherwise)
  void* wgu8;
  void* wd8;
  float* sgu;
  float* sd;
  // workspace (one allocation) and its buffers
  void* ws;
  Work w;
  // optional per-kernel event timing (start/stop per kernel of a recorded forward)
  std::vector<hipEvent_t> tev;
  std::vector<uint8_t> tslots;  // per recorded forward: bit i set if slot i ran
  int t_max;
  int t_used;
  bool timing;
};

namespace {

template <typename T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(base) + off);
}

static_assert(moe::kNumSlots == MOE_TIMED_SLOTS, "timing slots");
constexpr int kEventsPerForward = 2 * MOE_TIMED_SLOTS;  // start and stop per kernel

void drop_events(moe_layer* L) {
  for (hipEvent_t e : L->tev) (void)hipEventDestroy(e);
  L->tev.clear();
  L->tslots.clear();
  L->timing = false;
  L->t_max = L->t_used = 0;
}

void release(moe_layer* L) {
  if (L == nullptr) return;
  drop_events(L);
  if (L->params) (void)hipFree(L->params);
  if (L->ws) (void)hipFree(L->ws);
  L->magic = 0;
  delete L;
}

moe_status_t check_config(const moe_layer_config_t* c) {
  if (c->dtype != MOE_DTYPE_F32 && c->dtype != MOE_DTYPE_BF16)
    return fail(MOE_ERR_INVALID_ARG, "dtype must be MOE_DTYPE_F32 or MOE_DTYPE_BF16");
  if (c->d_model <= 0 || c->d_ff <= 0 || c->n_experts <= 0 || c->top_k <= 0 || c->max_tokens <= 0)
    return fail(MOE_ERR_INVALID_ARG, "d_model, d_ff, n_experts, top_k and max_tokens must be > 0");
  if (!(c->rms_eps >= 0.f) || !std::isfinite(c->rms_eps))
    return fail(MOE_ERR_INVALID_ARG, "rms_eps must be finite and >= 0");
  if (c->top_k > c->n_experts) return fail(MOE_ERR_INVALID_ARG, "top_k exceeds n_experts");
  if (c->n_experts > 64) return fail(MOE_ERR_UNSUPPORTED, "n_experts above 64");
  if (c->top_k > 8) return fail(MOE_ERR_UNSUPPORTED, "top_k above 8");
  if (c->max_tokens > kMaxTokensLimit) return fail(MOE_ERR_UNSUPPORTED, "max_tokens above 2^20");
  if (c->dtype == MOE_DTYPE_BF16) {
    if (c->d_model % 256 != 0 || c->d_ff % 128 != 0)
      return fail(MOE_ERR_UNSUPPORTED, "bf16 layers need d_model % 256 == 0 and d_ff % 128 == 0");
    // the grouped GEMMs address a unit's operands with 32-bit byte offsets
    if (c->d_model > kMaxWidth || c->d_ff > kMaxWidth)
      return fail(MOE_ERR_UNSUPPORTED, "bf16 layers need d_model and d_ff <= 65536");
  } else {
    if (c->d_model % 4 != 0 || c->d_ff % 4 != 0)
      return fail(MOE_ERR_UNSUPPORTED, "fp32 layers need d_model and d_ff multiples of 4");
  }
  const double n = (double)c->max_tokens * c->top_k;
  if (n * c->d_ff >= 9.0e18 / 4 || n * c->d_model >= 9.0e18 / 4)
    return fail(MOE_ERR_UNSUPPORTED, "workspace size overflows");
  return MOE_OK;
}

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_last_error(void) { return g_err.c_str(); }

}  // extern "C"

namespace {
// sc != nullptr: expert weights are E4M3 codes with per-row scales; act8:
// activations in E4M3 too (only the fp8 banks are kept).
moe_status_t create_impl(const moe_layer_config_t* cfg, const moe_layer_weights_t* w,
                         const moe_fp8_scales_t* sc, bool act8, void* stream, moe_layer_t** out) {
  if (out == nullptr) return fail(MOE_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (cfg == nullptr || w == nullptr) return fail(MOE_ERR_INVALID_ARG, "cfg or weights is NULL");
  moe_status_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  const bool fp8 = sc != nullptr;
  if (fp8) {
    if (cfg->dtype != MOE_DTYPE_BF16)
      return fail(MOE_ERR_INVALID_ARG, "fp8 expert weights need dtype MOE_DTYPE_BF16 activations");
    // the decode streams read k-step pairs: an even count per wave of each split
    if (cfg->d_ff % 256 != 0)
      return fail(MOE_ERR_UNSUPPORTED, "fp8 expert weights need d_ff % 256 == 0");
    const void* sp[] = {sc->gate, sc->up, sc->down};
    for (const void* p : sp)
      if (p == nullptr || !aligned(p, 4))
        return fail(MOE_ERR_INVALID_ARG, "an fp8 scale pointer is NULL or misaligned");
  }
  const void* wp[] = {w->rms_gain, w->w_router, w->w_gate, w->w_up, w->w_down};
  for (const void* p : wp) {
    if (p == nullptr) return fail(MOE_ERR_INVALID_ARG, "a weight pointer is NULL");
    if (!aligned(p, 16)) return fail(MOE_ERR_INVALID_ARG, "weight pointers must be 16-byte aligned");
  }
  if (w->b_router == nullptr || !aligned(w->b_router, 4))
    return fail(MOE_ERR_INVALID_ARG, "b_router is NULL or misaligned");

  int dev = 0;
  hipError_t he = hipGetDevice(&dev);
  if (he != hipSuccess) return hip_fail(he, "hipGetDevice");
  hipDeviceProp_t prop;
  he = hipGetDeviceProperties(&prop, dev);
  if (he != hipSuccess) return hip_fail(he, "hipGetDeviceProperties");
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(MOE_ERR_UNSUPPORTED, std::string("device is ") + prop.gcnArchName +
                                         ", the kernels are built for gfx950");
  st = scratch_setup(dev);  // the device's static scratch, for moe_layer_forward_static
  if (st != MOE_OK) return st;

  moe_layer* L = new (std::nothrow) moe_layer();
  if (L == nullptr) return fail(MOE_ERR_OOM, "host allocation failed");
  L->dim.d = cfg->d_model;
  L->dim.F = cfg->d_ff;
  L->dim.E = cfg->n_experts;
  L->dim.k = cfg->top_k;
  L->dim.EP = next_pow2(cfg->n_experts);
  L->dim.eps = cfg->rms_eps;
  L->dim.dtype = cfg->dtype;
  L->dim.act8 = fp8 && act8 ? 1 : 0;
  L->max_tokens = cfg->max_tokens;
  L->device = dev;
  L->num_cu = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1;
  const char* dbg = std::getenv("MOE_DEBUG_SYNC");
  L->debug_sync = dbg != nullptr && dbg[0] == '1';

  const size_t d = L->dim.d, F = L->dim.F, E = L->dim.E, EP = L->dim.EP;
  const size_t es = cfg->dtype == MOE_DTYPE_BF16 ? 2 : 4;

  // parameters
  Carver pc;
  const size_t o_wrg = pc.take(EP * d * 4);
  const size_t o_gain = pc.take(d * 4);
  const size_t o_bias = pc.take(64 * 4);  // zero-padded to 64 experts
  const bool bf16 = cfg->dtype == MOE_DTYPE_BF16;
  const size_t o_wr16 = bf16 ? pc.take(E * d * 2) : 0;
  const size_t o_g16 = bf16 ? pc.take(d * 2) : 0;
  const bool banks16 = !L->dim.act8;  // bf16 (or fp8-valued bf16) banks
  const size_t o_wgu = banks16 ? pc.take(E * F * d * es * (cfg->dtype == MOE_DTYPE_BF16 ? 2 : 1)) : 0;
  const size_t o_wup = cfg->dtype == MOE_DTYPE_F32 ? pc.take(E * F * d * es) : 0;
  const size_t o_wd = banks16 ? pc.take(E * d * F * es) : 0;
  const size_t o_wgu8 = fp8 ? pc.take(E * 2 * F * d) : 0;
  const size_t o_wd8 = fp8 ? pc.take(E * d * F) : 0;
  const size_t o_sgu = fp8 ? pc.take(E * 2 * F * 4) : 0;
  const size_t o_sd = fp8 ? pc.take(E * d * 4) : 0;
  he = hipMalloc(&L->params, pc.off);
  if (he != hipSuccess) {
    L->params = nullptr;
    release(L);
    (void)hipGetLastError();
    return fail(MOE_ERR_OOM, std::string("parameter allocation: ") + hipGetErrorString(he));
  }
  L->wrg = at<float>(L->params, o_wrg);
  L->gain32 = at<float>(L->params, o_gain);
  L->bias = at<float>(L->params, o_bias);
  L->wr16 = bf16 ? at<void>(L->params, o_wr16) : nullptr;
  L->gain16 = bf16 ? at<void>(L->params, o_g16) : nullptr;
  L->wgu = banks16 ? at<void>(L->params, o_wgu) : nullptr;
  L->wup = cfg->dtype == MOE_DTYPE_F32 ? at<void>(L->params, o_wup) : nullptr;
  L->wd = banks16 ? at<void>(L->params, o_wd) : nullptr;
  L->wgu8 = fp8 ? at<void>(L->params, o_wgu8) : nullptr;
  L->wd8 = fp8 ? at<void>(L->params, o_wd8) : nullptr;
  L->sgu = fp8 ? at<float>(L->params, o_sgu) : nullptr;
  L->sd = fp8 ? at<float>(L->params, o_sd) : nullptr;

  // workspace
  const size_t ws_bytes = carve_work(L->dim, (size_t)L->max_tokens, nullptr, nullptr);
  he = hipMalloc(&L->ws, ws_bytes);
  if (he != hipSuccess) {
    L->ws = nullptr;
    release(L);
    (void)hipGetLastError();
    return fail(MOE_ERR_OOM, std::string("workspace allocation: ") + hipGetErrorString(he));
  }
  carve_work(L->dim, (size_t)L->max_tokens, static_cast<char*>(L->ws), &L->w);

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  he = moe::launch_prep_router(w->w_router, w->rms_gain, cfg->dtype, (int)E, (int)EP, (int)d,
                               L->wrg, L->gain32, s);
  if (he == hipSuccess) he = hipMemsetAsync(L->bias, 0, 64 * 4, s);
  if (he == hipSuccess)
    he = hipMemcpyAsync(L->bias, w->b_router, E * 4, hipMemcpyDeviceToDevice, s);
  if (he == hipSuccess) he = hipMemsetAsync(L->w.zrow, 0, L->w.zbytes, s);
  if (he == hipSuccess && bf16)
    he = hipMemcpyAsync(L->wr16, w->w_router, E * d * 2, hipMemcpyDeviceToDevice, s);
  if (he == hipSuccess && bf16)
    he = hipMemcpyAsync(L->gain16, w->rms_gain, d * 2, hipMemcpyDeviceToDevice, s);
  if (he == hipSuccess) {
    if (fp8) {
      he = moe::launch_pack_fp8(static_cast<const uint8_t*>(w->w_gate),
                                static_cast<const uint8_t*>(w->w_up),
                                static_cast<const uint8_t*>(w->w_down), sc->gate, sc->up, (int)E,
                                (int)F, (int)d, static_cast<uint16_t*>(L->wgu),  // null for act8
                                static_cast<uint16_t*>(L->wd), static_cast<uint8_t*>(L->wgu8),
                                static_cast<uint8_t*>(L->wd8), L->sgu, s);
      if (he == hipSuccess)
        he = hipMemcpyAsync(L->sd, sc->down, E * d * 4, hipMemcpyDeviceToDevice, s);
    } else if (cfg->dtype == MOE_DTYPE_BF16) {
      he = moe::launch_pack_gateup(static_cast<const uint16_t*>(w->w_gate),
                                   static_cast<const uint16_t*>(w->w_up),
                                   static_cast<uint16_t*>(L->wgu), (int)E, (int)F, (int)d, s);
      if (he == hipSuccess)
        he = moe::launch_pack_down(static_cast<const uint16_t*>(w->w_down),
                                   static_cast<uint16_t*>(L->wd), (int)E, (int)d, (int)F, s);
    } else {
      he = hipMemcpyAsync(L->wgu, w->w_gate, E * F * d * 4, hipMemcpyDeviceToDevice, s);
      if (he == hipSuccess)
        he = hipMemcpyAsync(L->wup, w->w_up, E * F * d * 4, hipMemcpyDeviceToDevice, s);
      if (he == hipSuccess)
        he = hipMemcpyAsync(L->wd, w->w_down, E * d * F * 4, hipMemcpyDeviceToDevice, s);
    }
  }
  if (he == hipSuccess && L->debug_sync) he = hipStreamSynchronize(s);
  if (he != hipSuccess) {
    (void)hipStreamSynchronize(s);
    release(L);
    return hip_fail(he, "weight preparation");
  }
  L->magic = kMagic;
  *out = L;
  return MOE_OK;
}
}  // namespace

extern "C" {

moe_status_t moe_layer_create(const moe_layer_config_t* cfg, const moe_layer_weights_t* w,
                              void* stream, moe_layer_t** out) {
  g_err.clear();
  return create_impl(cfg, w, nullptr, false, stream, out);
}

moe_status_t moe_layer_create_fp8(const moe_layer_config_t* cfg, const moe_layer_weights_t* w,
                                  const moe_fp8_scales_t* scales, void* stream,
                                  moe_layer_t** out) {
  g_err.clear();
  if (scales == nullptr) {
    if (out != nullptr) *out = nullptr;
    return fail(MOE_ERR_INVALID_ARG, "scales is NULL");
  }
  return create_impl(cfg, w, scales, false, stream, out);
}

moe_status_t moe_layer_create_w8a8(const moe_layer_config_t* cfg, const moe_layer_weights_t* w,
                                   const moe_fp8_scales_t* scales, void* stream,
                                   moe_layer_t** out) {
  g_err.clear();
  if (scales == nullptr) {
    if (out != nullptr) *out = nullptr;
    return fail(MOE_ERR_INVALID_ARG, "scales is NULL");
  }
  return create_impl(cfg, w, scales, true, stream, out);
}

moe_status_t moe_fp8_quantize_rows(const void* x, int32_t R, int32_t K, void* codes,
                                   float* scales, void* stream) {
  g_err.clear();
  if (R < 0 || K <= 0 || K % 8 != 0)
    return fail(MOE_ERR_INVALID_ARG, "R must be >= 0 and K a positive multiple of 8");
  if (R == 0) return MOE_OK;
  if (x == nullptr || codes == nullptr || scales == nullptr)
    return fail(MOE_ERR_INVALID_ARG, "x, codes or scales is NULL");
  if (!aligned(x, 16) || !aligned(codes, 8) || !aligned(scales, 4))
    return fail(MOE_ERR_INVALID_ARG, "x must be 16-byte, codes 8-byte and scales 4-byte aligned");
  const hipError_t he = moe::launch_quant_rows(x, R, K, codes, scales,
                                               reinterpret_cast<hipStream_t>(stream));
  if (he != hipSuccess) return hip_fail(he, "quantize launch");
  return MOE_OK;
}

}  // extern "C"

namespace {
// One forward; `allow_sync` is false inside a HIP graph capture, where the
// MOE_DEBUG_SYNC synchronisation must not run.
// eda: a stack's depth-averaging state for this layer's router (bf16 MoE
// layers only; null otherwise), eda_first: the stack's first MoE layer.
// wk: the per-call buffers (null: the layer's workspace).  res: bf16 layers in
// a stack, the residual stream that the output is added to (else null).
moe_status_t forward_impl(moe_layer_t* L, const void* hidden, int32_t T, void* out, void* stream,
                          const moe_routing_out_t* routing, bool allow_sync,
                          float* eda = nullptr, float eda_alpha = 0.f, bool eda_first = false,
                          const Work* wk = nullptr, const void* res = nullptr) {
  if (L == nullptr || L->magic != kMagic) return fail(MOE_ERR_INVALID_ARG, "invalid layer handle");
  if (T < 0 || T > L->max_tokens)
    return fail(MOE_ERR_INVALID_ARG, "T must be in [0, max_tokens] (max_tokens = " +
                                         std::to_string(L->max_tokens) + ")");
  if (T == 0) return MOE_OK;
  if (hidden == nullptr || out == nullptr) return fail(MOE_ERR_INVALID_ARG, "hidden or out is NULL");
  if (!aligned(hidden, 16) || !aligned(out, 16))
    return fail(MOE_ERR_INVALID_ARG, "hidden and out must be 16-byte aligned");
  const size_t es = L->dim.dtype == MOE_DTYPE_BF16 ? 2 : 4;
  const size_t bytes = (size_t)T * L->dim.d * es;
  const uintptr_t h0 = reinterpret_cast<uintptr_t>(hidden), o0 = reinterpret_cast<uintptr_t>(out);
  // a one-layer stack pass in place: out, hidden and res are the same rows,
  // and every element is read and rewritten by one lane of the layer's last
  // kernel, after every read of the hidden rows (router, gather) has ended
  const bool in_place = res != nullptr && out == hidden && res == hidden;
  if (!in_place && h0 < o0 + bytes && o0 < h0 + bytes)
    return fail(MOE_ERR_INVALID_ARG, "out overlaps hidden");
  if (routing != nullptr) {
    const void* rp[] = {routing->sel, routing->gate, routing->counts, routing->offsets,
                        routing->gather, routing->scatter};
    for (const void* p : rp)
      if (p != nullptr && !aligned(p, 4))
        return fail(MOE_ERR_INVALID_ARG, "routing buffers must be 4-byte aligned");
  }
  int dev = -1;
  hipError_t he = hipGetDevice(&dev);
  if (he != hipSuccess) return hip_fail(he, "hipGetDevice");
  if (dev != L->device)
    return fail(MOE_ERR_INVALID_ARG, "the current device is not the layer's device");

  moe::FwdArgs a;
  a.dim = L->dim;
  a.T = T;
  a.n = T * L->dim.k;
  a.hidden = hidden;
  a.out = out;
  a.res = res;
  a.wrg = L->wrg;
  a.gain = L->gain32;
  a.bias = L->bias;
  a.wr16 = L->wr16;
  a.gain16 = L->gain16;
  a.wgu = L->wgu;
  a.wup = L->wup;
  a.wd = L->wd;
  a.wgu8 = L->wgu8;
  a.wd8 = L->wd8;
  a.sgu = L->sgu;
  a.sd = L->sd;
  const Work& w = wk != nullptr ? *wk : L->w;
  a.xn = w.xn;
  a.inv = w.inv;
  a.sel = (routing && routing->sel) ? routing->sel : w.sel;
  a.gate = (routing && routing->gate) ? routing->gate : w.gate;
  a.counts = (routing && routing->counts) ? routing->counts : w.counts;
  a.offsets = (routing && routing->offsets) ? routing->offsets : w.offsets;
  a.gather = (routing && routing->gather) ? routing->gather : w.gather;
  a.scatter = (routing && routing->scatter) ? routing->scatter : w.scatter;
  a.slot_expert = w.slot_expert;
  a.hist = w.hist;
  a.xt = w.xt;
  a.act = w.act;
  a.xq = w.xq;
  a.actq = w.actq;
  a.sx = w.sx;
  a.sm = w.sm;
  a.xs_tok = w.xs_tok;
  a.pmm = w.pmm;
  a.ybuf = w.ybuf;
  a.zrow = w.zrow;
  a.sink = w.sink;
  a.num_cu = L->num_cu;
  a.eda = eda;
  a.eda_alpha = eda_alpha;
  a.eda_first = eda_first ? 1 : 0;
  a.stream = reinterpret_cast<hipStream_t>(stream);
  if (L->timing && L->t_used < L->t_max) {
    const hipEvent_t* ev = &L->tev[(size_t)L->t_used * kEventsPerForward];
    for (int i = 0; i < moe::kNumSlots; ++i) {
      a.ev[i].start = ev[2 * i];
      a.ev[i].stop = ev[2 * i + 1];
    }
    ++L->t_used;
  }
  const bool bf16 = L->dim.dtype == MOE_DTYPE_BF16;
  const bool act8 = L->dim.act8 != 0;  // fp8 activations
  const bool decode = bf16 && a.n <= moe::kStreamMaxAssign;
  if (L->timing && L->t_used > 0 && a.ev[0].start != nullptr)
    L->tslots[L->t_used - 1] = (uint8_t)(0x0d | (decode ? 0 : 0x02) | (L->dim.k > 1 ? 0x10 : 0) |
                                         (bf16 && !decode ? 0x20 : 0) | (act8 ? 0x40 : 0));

  if (wk != nullptr && wk->clear_zrow) {
    he = moe::launch_zero(wk->zrow, wk->zbytes, a.stream);
    if (he != hipSuccess) return hip_fail(he, "scratch clear launch");
  }
  if (decode) {
    he = moe::launch_router_token(a);
    if (he != hipSuccess) return hip_fail(he, "router launch");
    he = moe::launch_experts_stream(a);
  } else {
    he = bf16 ? moe::launch_router_mfma(a) : moe::launch_norm_router(a);
    if (he != hipSuccess) return hip_fail(he, "router launch");
    he = moe::launch_route_permute(a);
    if (he != hipSuccess) return hip_fail(he, "permute launch");
    if (bf16) {
      he = moe::launch_gather_tiles(a);
      if (he != hipSuccess) return hip_fail(he, "gather launch");
    }
    if (act8) {
      he = moe::launch_experts_tile_fp8_gateup(a);
      if (he == hipSuccess) he = moe::launch_quant_act(a);
      if (he == hipSuccess) he = moe::launch_experts_tile_fp8_down(a);
    } else {
      he = bf16 ? moe::launch_experts_tile(a) : moe::launch_experts_f32(a);
    }
  }
  if (he != hipSuccess) return hip_fail(he, "expert launch");
  if (L->dim.k > 1) {
    he = moe::launch_combine(a);
    if (he != hipSuccess) return hip_fail(he, "combine launch");
  }
  if (L->debug_sync && allow_sync) {
    he = hipStreamSynchronize(a.stream);
    if (he != hipSuccess) return hip_fail(he, "forward (MOE_DEBUG_SYNC)");
  }
  return MOE_OK;
}
}  // namespace

extern "C" {

moe_status_t moe_layer_forward(moe_layer_t* L, const void* hidden, int32_t T, void* out,
                               void* stream, const moe_routing_out_t* routing) {
  g_err.clear();
  return forward_impl(L, hidden, T, out, stream, routing, true);
}

moe_status_t moe_layer_forward_static(moe_layer_t* L, const void* hidden, int32_t T, void* out,
                                      void* stream, const moe_routing_out_t* routing) {
  g_err.clear();
  if (L == nullptr || L->magic != kMagic) return fail(MOE_ERR_INVALID_ARG, "invalid layer handle");
  if (T < 0 || T > L->max_tokens)
    return fail(MOE_ERR_INVALID_ARG, "T must be in [0, max_tokens] (max_tokens = " +
                                         std::to_string(L->max_tokens) + ")");
  const size_t need = carve_work(L->dim, (size_t)T, nullptr, nullptr);
  if (need > kScratchBytes)
    return fail(MOE_ERR_INVALID_ARG,
                "T = " + std::to_string(T) + " needs " + std::to_string(need) +
                    " bytes of per-call buffers; the static scratch holds " +
                    std::to_string(kScratchBytes) + " (use moe_layer_forward)");
  char* base = static_cast<char*>(scratch_base(L->device));
  if (base == nullptr) return fail(MOE_ERR_HIP, "static scratch of the layer's device not set up");
  Work w;
  carve_work(L->dim, (size_t)T, base, &w);
  w.clear_zrow = true;  // the array keeps whatever the previous call left there
  return forward_impl(L, hidden, T, out, stream, routing, true, nullptr, 0.f, false, &w);
}

moe_status_t moe_layer_set_bias(moe_layer_t* L, const float* b_router, void* stream) {
  g_err.clear();
  if (L == nullptr || L->magic != kMagic) return fail(MOE_ERR_INVALID_ARG, "invalid layer handle");
  if (b_router == nullptr || !aligned(b_router, 4))
    return fail(MOE_ERR_INVALID_ARG, "b_router is NULL or misaligned");
  hipError_t he = hipMemcpyAsync(L->bias, b_router, (size_t)L->dim.E * 4, hipMemcpyDeviceToDevice,
                                 reinterpret_cast<hipStream_t>(stream));
  if (he != hipSuccess) return hip_fail(he, "set_bias copy");
  return MOE_OK;
}

moe_status_t moe_layer_get_bias(moe_layer_t* L, float* b_out, void* stream) {
  g_err.clear();
  if (L == nullptr || L->magic != kMagic) return fail(MOE_ERR_INVALID_ARG, "invalid layer handle");
  if (b_out == nullptr || !aligned(b_out, 4))
    return fail(MOE_ERR_INVALID_ARG, "b_out is NULL or misaligned");
  hipError_t he = hipMemcpyAsync(b_out, L->bias, (size_t)L->dim.E * 4, hipMemcpyDeviceToDevice,
                                 reinterpret_cast<hipStream_t>(stream));
  if (he != hipSuccess) return hip_fail(he, "get_bias copy");
  return MOE_OK;
}

moe_status_t moe_layer_update_bias(moe_layer_t* L, const int32_t* counts, float rate,
                                   void* stream) {
  g_err.clear();
  if (L == nullptr || L->magic != kMagic) return fail(MOE_ERR_INVALID_ARG, "invalid layer handle");
  if (!std::isfinite(rate)) return fail(MOE_ERR_INVALID_ARG, "rate must be finite");
  if (counts != nullptr && !aligned(counts, 4))
    return fail(MOE_ERR_INVALID_ARG, "counts must be 4-byte aligned");
  const int* c = counts != nullptr ? counts : L->w.counts;
  hipError_t he = moe::launch_bias_update(c, L->dim.E, rate, L->bias,
                                          reinterpret_cast<hipStream_t>(stream));
  if (he != hipSuccess) return hip_fail(he, "bias update launch");
  if (L->debug_sync) {
    he = hipStreamSynchronize(reinterpret_cast<hipStream_t>(stream));
    if (he != hipSuccess) return hip_fail(he, "bias update (MOE_DEBUG_SYNC)");
  }
  return MOE_OK;
}

moe_status_t moe_layer_timing_start(moe_layer_t* L, int32_t max_forwards) {
  g_err.clear();
  if (L == nullptr || L->magic != kMagic) return fail(MOE_ERR_INVALID_ARG, "invalid layer handle");
  if (max_forwards < 1 || max_forwards > 65536)
    return fail(MOE_ERR_INVALID_ARG, "max_forwards must be in [1, 65536]");
  drop_events(L);
  L->tev.resize((size_t)max_forwards * kEventsPerForward);
  L->tslots.assign((size_t)max_forwards, 0);
  for (size_t i = 0; i < L->tev.size(); ++i) {
    hipError_t he = hipEventCreate(&L->tev[i]);
    if (he != hipSuccess) {
      L->tev.resize(i);
      drop_events(L);
      return hip_fail(he, "hipEventCreate");
    }
  }
  L->t_max = max_forwards;
  L->t_used = 0;
  L->timing = true;
  return MOE_OK;
}

moe_status_t moe_layer_timing_stop(moe_layer_t* L, float* ms_sum, int32_t* n_forwards) {
  g_err.clear();
  if (L == nullptr || L->magic != kMagic) return fail(MOE_ERR_INVALID_ARG, "invalid layer handle");
  if (!L->timing) return fail(MOE_ERR_INVALID_ARG, "timing was not started");
  if (ms_sum == nullptr || n_forwards == nullptr)
    return fail(MOE_ERR_INVALID_ARG, "ms_sum or n_forwards is NULL");
  for (int i = 0; i < MOE_TIMED_SLOTS; ++i) ms_sum[i] = 0.f;
  *n_forwards = L->t_used;
  hipError_t he = hipSuccess;
  for (int f = 0; f < L->t_used && he == hipSuccess; ++f) {
    const hipEvent_t* ev = &L->tev[(size_t)f * kEventsPerForward];
    for (int i = 0; i < MOE_TIMED_SLOTS && he == hipSuccess; ++i) {
      if (!((L->tslots[f] >> i) & 1)) continue;
      float ms = 0.f;
      he = hipEventSynchronize(ev[2 * i + 1]);
      if (he == hipSuccess) he = hipEventElapsedTime(&ms, ev[2 * i], ev[2 * i + 1]);
      ms_sum[i] += ms;
    }
  }
  drop_events(L);
  if (he != hipSuccess) return hip_fail(he, "event timing");
  return MOE_OK;
}

void moe_layer_destroy(moe_layer_t* L) {
  if (L == nullptr || L->magic != kMagic) return;
  const int dev = L->device;
  int cur = -1;
  (void)hipGetDevice(&cur);
  if (cur != dev) (void)hipSetDevice(dev);
  (void)hipDeviceSynchronize();
  release(L);
  if (cur >= 0 && cur != dev) (void)hipSetDevice(cur);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// FFN stack: the feed-forward half of the ZONOS2 backbone's layers in order
// (digest item 5: 28 layers, the first three and the last one dense, the
// MoE layers top-1 except the last one, top-2), each followed by the residual
// add, h_{l+1} = h_l + FFN_l(h_l).  The stack borrows layer handles created by
// the caller (a dense layer is a one-expert layer) and owns two residual
// buffers, one FFN output buffer (fp32 stacks; bf16 layers add their output
// to the residual stream in their last kernel) and, once captured, a HIP
// graph of the whole sequence.

struct moe_stack {
  uint32_t magic;
  std::vector<moe_layer_t*> layers;
  int d, dtype, max_tokens, device;
  void* buf;   // one allocation: residual A, residual B, FFN output, each [max_tokens, d]
  void* hA;
  void* hB;
  void* y;
  hipGraphExec_t exec;
  hipStream_t exec_stream;
  float* eda;       // [max_tokens][64] fp32 depth-averaging state of the router logits
  bool eda_on;
  float eda_alpha;
};

namespace {
constexpr uint32_t kStackMagic = 0x4b745345u;  // "EStK"

void stack_release(moe_stack* S) {
  if (S == nullptr) return;
  if (S->exec) (void)hipGraphExecDestroy(S->exec);
  if (S->buf) (void)hipFree(S->buf);
  if (S->eda) (void)hipFree(S->eda);
  S->magic = 0;
  delete S;
}

// Depth averaging carries one expert's logit from a MoE layer to the next, so
// every MoE layer (n_experts > 1) of the stack must have the same n_experts.
bool stack_moe_experts_agree(const moe_stack* S) {
  int E = 0;
  for (const moe_layer_t* L : S->layers) {
    if (L->dim.E <= 1) continue;
    if (E != 0 && L->dim.E != E) return false;
    E = L->dim.E;
  }
  return true;
}

moe_status_t stack_check(moe_stack* S, const void* hin, int32_t T, void* hout) {
  if (S == nullptr || S->magic != kStackMagic) return fail(MOE_ERR_INVALID_ARG, "invalid stack handle");
  if (T < 0 || T > S->max_tokens)
    return fail(MOE_ERR_INVALID_ARG, "T must be in [0, max_tokens] (max_tokens = " +
                                         std::to_string(S->max_tokens) + ")");
  if (T > 0 && (hin == nullptr || hout == nullptr))
    return fail(MOE_ERR_INVALID_ARG, "hidden_in or hidden_out is NULL");
  if (!aligned(hin, 16) || !aligned(hout, 16))
    return fail(MOE_ERR_INVALID_ARG, "hidden_in and hidden_out must be 16-byte aligned");
  int dev = -1;
  hipError_t he = hipGetDevice(&dev);
  if (he != hipSuccess) return hip_fail(he, "hipGetDevice");
  if (dev != S->device) return fail(MOE_ERR_INVALID_ARG, "the current device is not the stack's device");
  for (moe_layer_t* L : S->layers)
    if (L == nullptr || L->magic != kMagic) return fail(MOE_ERR_INVALID_ARG, "a layer of the stack was destroyed");
  if (S->eda_on && !stack_moe_experts_agree(S))
    return fail(MOE_ERR_INVALID_ARG,
                "depth averaging needs the same n_experts in every MoE layer of the stack");
  return MOE_OK;
}

// The launch sequence of one stack forward (no validation, no synchronisation).
// routing: null, or one routing-output struct per layer.
moe_status_t stack_enqueue(moe_stack* S, const void* hin, int32_t T, void* hout, hipStream_t s,
                           bool allow_sync, const moe_routing_out_t* routing = nullptr) {
  if (T == 0) return MOE_OK;
  const size_t n = (size_t)T * S->d;
  const void* cur = hin;
  const int nl = (int)S->layers.size();
  bool first_moe = true;
  // bf16: each layer's last kernel adds its output to the residual stream
  // (out = bf16(h + bf16(y)), the same two roundings as a separate add);
  // fp32: a residual launch after each layer
  const bool fused = S->dtype == MOE_DTYPE_BF16;
  for (int l = 0; l < nl; ++l) {
    const bool moe = S->layers[l]->dim.E > 1;
    float* eda = S->eda_on && moe ? S->eda : nullptr;
    void* nxt = l == nl - 1 ? hout : ((l & 1) ? S->hB : S->hA);
    moe_status_t st = forward_impl(S->layers[l], cur, T, fused ? nxt : S->y, s,
                                   routing != nullptr ? &routing[l] : nullptr, allow_sync, eda,
                                   S->eda_alpha, first_moe, nullptr, fused ? cur : nullptr);
    if (moe) first_moe = false;
    if (st != MOE_OK) return st;
    if (!fused) {
      hipError_t he = moe::launch_residual_f32(static_cast<const float*>(cur),
                                               static_cast<const float*>(S->y),
                                               static_cast<float*>(nxt), n, s);
      if (he != hipSuccess) return hip_fail(he, "residual launch");
    }
    cur = nxt;
  }
  return MOE_OK;
}
}  // namespace

extern "C" {

moe_status_t moe_stack_create(int32_t n_layers, moe_layer_t* const* layers, int32_t max_tokens,
                              moe_stack_t** out) {
  g_err.clear();
  if (out == nullptr) return fail(MOE_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (n_layers < 1 || n_layers > 4096 || layers == nullptr)
    return fail(MOE_ERR_INVALID_ARG, "need 1 to 4096 layers");
  if (max_tokens < 1) return fail(MOE_ERR_INVALID_ARG, "max_tokens must be > 0");
  int d = 0, dtype = 0, dev = 0;
  for (int l = 0; l < n_layers; ++l) {
    moe_layer_t* L = layers[l];
    if (L == nullptr || L->magic != kMagic) return fail(MOE_ERR_INVALID_ARG, "invalid layer handle");
    if (l == 0) {
      d = L->dim.d;
      dtype = L->dim.dtype;
      dev = L->device;
    } else if (L->dim.d != d || L->dim.dtype != dtype || L->device != dev) {
      return fail(MOE_ERR_INVALID_ARG, "stack layers must share d_model, dtype and device");
    }
    if (L->max_tokens < max_tokens)
      return fail(MOE_ERR_INVALID_ARG, "a layer's max_tokens is below the stack's");
  }
  int cur = -1;
  hipError_t he = hipGetDevice(&cur);
  if (he != hipSuccess) return hip_fail(he, "hipGetDevice");
  if (cur != dev) return fail(MOE_ERR_INVALID_ARG, "the current device is not the layers' device");
  moe_stack* S = new (std::nothrow) moe_stack();
  if (S == nullptr) return fail(MOE_ERR_OOM, "host allocation failed");
  S->layers.assign(layers, layers + n_layers);
  S->d = d;
  S->dtype = dtype;
  S->max_tokens = max_tokens;
  S->device = dev;
  const size_t es = dtype == MOE_DTYPE_BF16 ? 2 : 4;
  const size_t one = align_up((size_t)max_tokens * d * es, 256);
  he = hipMalloc(&S->buf, 3 * one);
  if (he != hipSuccess) {
    S->buf = nullptr;
    stack_release(S);
    (void)hipGetLastError();
    return fail(MOE_ERR_OOM, std::string("stack buffers: ") + hipGetErrorString(he));
  }
  S->hA = S->buf;
  S->hB = at<void>(S->buf, one);
  S->y = at<void>(S->buf, 2 * one);
  if (dtype == MOE_DTYPE_BF16) {
    he = hipMalloc(&S->eda, (size_t)max_tokens * 64 * 4);
    if (he != hipSuccess) {
      S->eda = nullptr;
      stack_release(S);
      (void)hipGetLastError();
      return fail(MOE_ERR_OOM, std::string("stack router state: ") + hipGetErrorString(he));
    }
    // never read before the first MoE layer of a pass writes it; cleared so
    // that no path can see uninitialised memory
    he = hipMemset(S->eda, 0, (size_t)max_tokens * 64 * 4);
    if (he != hipSuccess) {
      stack_release(S);
      return hip_fail(he, "stack router state");
    }
  }
  S->magic = kStackMagic;
  *out = S;
  return MOE_OK;
}

moe_status_t moe_stack_set_eda(moe_stack_t* S, int32_t enable, float alpha) {
  g_err.clear();
  if (S == nullptr || S->magic != kStackMagic) return fail(MOE_ERR_INVALID_ARG, "invalid stack handle");
  if (enable && S->eda == nullptr)
    return fail(MOE_ERR_UNSUPPORTED, "depth averaging needs bf16 layers");
  if (enable && !(alpha >= 0.f && alpha < 1.f))
    return fail(MOE_ERR_INVALID_ARG, "alpha must be in [0, 1)");
  if (enable && !stack_moe_experts_agree(S))
    return fail(MOE_ERR_INVALID_ARG,
                "depth averaging needs the same n_experts in every MoE layer of the stack");
  S->eda_on = enable != 0;
  S->eda_alpha = enable ? alpha : 0.f;
  return MOE_OK;
}

moe_status_t moe_stack_forward(moe_stack_t* S, const void* hidden_in, int32_t T, void* hidden_out,
                               void* stream) {
  g_err.clear();
  moe_status_t st = stack_check(S, hidden_in, T, hidden_out);
  if (st != MOE_OK) return st;
  return stack_enqueue(S, hidden_in, T, hidden_out, reinterpret_cast<hipStream_t>(stream), true);
}

moe_status_t moe_stack_forward_routing(moe_stack_t* S, const void* hidden_in, int32_t T,
                                       void* hidden_out, void* stream,
                                       const moe_routing_out_t* routing) {
  g_err.clear();
  moe_status_t st = stack_check(S, hidden_in, T, hidden_out);
  if (st != MOE_OK) return st;
  if (routing == nullptr) return fail(MOE_ERR_INVALID_ARG, "routing is NULL");
  return stack_enqueue(S, hidden_in, T, hidden_out, reinterpret_cast<hipStream_t>(stream), true,
                       routing);
}

moe_status_t moe_stack_capture(moe_stack_t* S, const void* hidden_in, int32_t T, void* hidden_out,
                               void* stream) {
  g_err.clear();
  moe_status_t st = stack_check(S, hidden_in, T, hidden_out);
  if (st != MOE_OK) return st;
  if (stream == nullptr) return fail(MOE_ERR_INVALID_ARG, "capture needs a created (non-null) stream");
  for (moe_layer_t* L : S->layers)
    if (L->timing) return fail(MOE_ERR_INVALID_ARG, "a layer of the stack has per-kernel timing on");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (S->exec) {
    (void)hipGraphExecDestroy(S->exec);
    S->exec = nullptr;
  }
  hipError_t he = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal);
  if (he != hipSuccess) return hip_fail(he, "hipStreamBeginCapture");
  st = stack_enqueue(S, hidden_in, T, hidden_out, s, false);
  const std::string enqueue_err = st != MOE_OK ? g_err : std::string();
  hipGraph_t graph = nullptr;
  he = hipStreamEndCapture(s, &graph);
  if (st != MOE_OK) {
    if (graph) (void)hipGraphDestroy(graph);
    return fail(st, enqueue_err);
  }
  if (he != hipSuccess) return hip_fail(he, "hipStreamEndCapture");
  he = hipGraphInstantiate(&S->exec, graph, nullptr, nullptr, 0);
  (void)hipGraphDestroy(graph);
  if (he != hipSuccess) {
    S->exec = nullptr;
    return hip_fail(he, "hipGraphInstantiate");
  }
  S->exec_stream = s;
  return MOE_OK;
}

moe_status_t moe_stack_replay(moe_stack_t* S, void* stream) {
  g_err.clear();
  if (S == nullptr || S->magic != kStackMagic) return fail(MOE_ERR_INVALID_ARG, "invalid stack handle");
  if (S->exec == nullptr) return fail(MOE_ERR_INVALID_ARG, "nothing captured");
  for (moe_layer_t* L : S->layers)
    if (L == nullptr || L->magic != kMagic) return fail(MOE_ERR_INVALID_ARG, "a layer of the stack was destroyed");
  hipError_t he = hipGraphLaunch(S->exec, reinterpret_cast<hipStream_t>(stream));
  if (he != hipSuccess) return hip_fail(he, "hipGraphLaunch");
  return MOE_OK;
}

void moe_stack_destroy(moe_stack_t* S) {
  if (S == nullptr || S->magic != kStackMagic) return;
  const int dev = S->device;
  int cur = -1;
  (void)hipGetDevice(&cur);
  if (cur != dev) (void)hipSetDevice(dev);
  (void)hipDeviceSynchronize();
  stack_release(S);
  if (cur >= 0 && cur != dev) (void)hipSetDevice(cur);
}

}  // extern "C"
