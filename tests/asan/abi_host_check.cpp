// Host-side checks of the C ABI (include/moe_layer.h) for a build whose host
// code carries AddressSanitizer: every argument-validation and error path
// that runs without launching a kernel, including create on a machine with no
// usable device (the device lookup fails and everything allocated so far is
// released).  Prints "ok <n> checks" and exits 0, or names the failed check
// and exits 1; heap errors abort through the sanitizer.  With the argument
// --plant it reads one element past a heap buffer instead (host memory only),
// which the sanitizer must report: the check that the build really carries it.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "moe_layer.h"

static int g_checks = 0;

static bool expect(bool cond, const char* what) {
  ++g_checks;
  if (!cond) std::fprintf(stderr, "FAILED: %s (last error: \"%s\")\n", what, moe_last_error());
  return cond;
}
#define EXPECT(c) \
  do {            \
    if (!expect((c), #c)) return 1; \
  } while (0)

static moe_layer_config_t good_cfg() {
  moe_layer_config_t c;
  c.d_model = 256;
  c.d_ff = 512;
  c.n_experts = 4;
  c.top_k = 1;
  c.dtype = MOE_DTYPE_BF16;
  c.rms_eps = 1e-6f;
  c.max_tokens = 64;
  return c;
}

int main(int argc, char** argv) {
  if (argc > 1 && std::strcmp(argv[1], "--plant") == 0) {
    volatile int* h = static_cast<int*>(std::malloc(8 * sizeof(int)));
    const int v = h[8];  // one past the end
    std::free(const_cast<int*>(h));
    return v == 12345 ? 3 : 2;
  }
  alignas(256) static unsigned char buf[4096];  // stands in for device memory; never dereferenced
  void* p = buf;
  EXPECT(moe_abi_version() == MOE_ABI_VERSION);
  EXPECT(std::strcmp(moe_last_error(), "") == 0);

  moe_layer_weights_t w{p, p, reinterpret_cast<const float*>(p), p, p, p};
  moe_layer_t* L = reinterpret_cast<moe_layer_t*>(&buf[1]);

  // create: argument validation
  moe_layer_config_t c = good_cfg();
  EXPECT(moe_layer_create(&c, &w, nullptr, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_layer_create(nullptr, &w, nullptr, &L) == MOE_ERR_INVALID_ARG && L == nullptr);
  EXPECT(moe_layer_create(&c, nullptr, nullptr, &L) == MOE_ERR_INVALID_ARG);
  EXPECT(std::strlen(moe_last_error()) > 0);
  struct Bad {
    const char* what;
    void (*edit)(moe_layer_config_t&);
    moe_status_t want;
  };
  const Bad bads[] = {
      {"dtype", [](moe_layer_config_t& x) { x.dtype = 7; }, MOE_ERR_INVALID_ARG},
      {"d_model 0", [](moe_layer_config_t& x) { x.d_model = 0; }, MOE_ERR_INVALID_ARG},
      {"d_ff < 0", [](moe_layer_config_t& x) { x.d_ff = -128; }, MOE_ERR_INVALID_ARG},
      {"top_k 0", [](moe_layer_config_t& x) { x.top_k = 0; }, MOE_ERR_INVALID_ARG},
      {"top_k > E", [](moe_layer_config_t& x) { x.top_k = 5; }, MOE_ERR_INVALID_ARG},
      {"max_tokens 0", [](moe_layer_config_t& x) { x.max_tokens = 0; }, MOE_ERR_INVALID_ARG},
      {"eps NaN", [](moe_layer_config_t& x) { x.rms_eps = 0.f / 0.f; }, MOE_ERR_INVALID_ARG},
      {"eps < 0", [](moe_layer_config_t& x) { x.rms_eps = -1.f; }, MOE_ERR_INVALID_ARG},
      {"E > 64", [](moe_layer_config_t& x) { x.n_experts = 65; }, MOE_ERR_UNSUPPORTED},
      {"k > 8", [](moe_layer_config_t& x) { x.n_experts = 16; x.top_k = 9; }, MOE_ERR_UNSUPPORTED},
      {"max_tokens > 2^20", [](moe_layer_config_t& x) { x.max_tokens = (1 << 20) + 1; },
       MOE_ERR_UNSUPPORTED},
      {"bf16 d % 256", [](moe_layer_config_t& x) { x.d_model = 384; }, MOE_ERR_UNSUPPORTED},
      {"bf16 F % 128", [](moe_layer_config_t& x) { x.d_ff = 192; }, MOE_ERR_UNSUPPORTED},
      {"f32 d % 4", [](moe_layer_config_t& x) { x.dtype = MOE_DTYPE_F32; x.d_model = 6; },
       MOE_ERR_UNSUPPORTED},
  };
  for (const Bad& b : bads) {
    moe_layer_config_t x = good_cfg();
    b.edit(x);
    L = reinterpret_cast<moe_layer_t*>(&buf[1]);
    if (!expect(moe_layer_create(&x, &w, nullptr, &L) == b.want && L == nullptr, b.what)) return 1;
  }
  moe_layer_weights_t wn = w;
  wn.w_gate = nullptr;
  EXPECT(moe_layer_create(&c, &wn, nullptr, &L) == MOE_ERR_INVALID_ARG);
  moe_layer_weights_t wm = w;
  wm.w_up = &buf[2];  // misaligned
  EXPECT(moe_layer_create(&c, &wm, nullptr, &L) == MOE_ERR_INVALID_ARG);
  moe_layer_weights_t wb = w;
  wb.b_router = nullptr;
  EXPECT(moe_layer_create(&c, &wb, nullptr, &L) == MOE_ERR_INVALID_ARG);
  // a valid request on a machine without a usable device fails cleanly
  {
    const moe_status_t st = moe_layer_create(&c, &w, nullptr, &L);
    EXPECT(st != MOE_OK || L != nullptr);
    if (st == MOE_OK) moe_layer_destroy(L);  // a device was there after all
    else EXPECT(L == nullptr && std::strlen(moe_last_error()) > 0);
  }

  // fp8 creates
  moe_fp8_scales_t sc{reinterpret_cast<const float*>(p), reinterpret_cast<const float*>(p),
                      reinterpret_cast<const float*>(p)};
  EXPECT(moe_layer_create_fp8(&c, &w, nullptr, nullptr, &L) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_layer_create_w8a8(&c, &w, nullptr, nullptr, &L) == MOE_ERR_INVALID_ARG);
  moe_fp8_scales_t scn = sc;
  scn.down = nullptr;
  EXPECT(moe_layer_create_fp8(&c, &w, &scn, nullptr, &L) == MOE_ERR_INVALID_ARG);
  moe_fp8_scales_t scm = sc;
  scm.up = reinterpret_cast<const float*>(&buf[2]);
  EXPECT(moe_layer_create_w8a8(&c, &w, &scm, nullptr, &L) == MOE_ERR_INVALID_ARG);
  moe_layer_config_t c32 = c;
  c32.dtype = MOE_DTYPE_F32;
  EXPECT(moe_layer_create_w8a8(&c32, &w, &sc, nullptr, &L) == MOE_ERR_INVALID_ARG);
  moe_layer_config_t cf = c;
  cf.d_ff = 384;
  EXPECT(moe_layer_create_fp8(&cf, &w, &sc, nullptr, &L) == MOE_ERR_UNSUPPORTED);

  // calls on a missing handle
  EXPECT(moe_layer_forward(nullptr, p, 4, p, nullptr, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_layer_forward_static(nullptr, p, 4, p, nullptr, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_layer_set_bias(nullptr, reinterpret_cast<const float*>(p), nullptr) ==
         MOE_ERR_INVALID_ARG);
  EXPECT(moe_layer_get_bias(nullptr, reinterpret_cast<float*>(p), nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_layer_update_bias(nullptr, nullptr, 0.1f, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_layer_timing_start(nullptr, 4) == MOE_ERR_INVALID_ARG);
  float ms[MOE_TIMED_SLOTS];
  int32_t nf = 0;
  EXPECT(moe_layer_timing_stop(nullptr, ms, &nf) == MOE_ERR_INVALID_ARG);
  moe_layer_destroy(nullptr);

  // stacks
  moe_stack_t* S = reinterpret_cast<moe_stack_t*>(&buf[3]);
  EXPECT(moe_stack_create(0, nullptr, 4, &S) == MOE_ERR_INVALID_ARG);
  moe_layer_t* none[2] = {nullptr, nullptr};
  EXPECT(moe_stack_create(2, none, 4, &S) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_stack_create(2, none, 4, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_stack_forward(nullptr, p, 4, p, nullptr) == MOE_ERR_INVALID_ARG);
  moe_routing_out_t ro{};
  EXPECT(moe_stack_forward_routing(nullptr, p, 4, p, nullptr, &ro) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_stack_set_eda(nullptr, 1, 0.5f) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_stack_capture(nullptr, p, 4, p, p) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_stack_replay(nullptr, nullptr) == MOE_ERR_INVALID_ARG);
  moe_stack_destroy(nullptr);

  // the quantisation entry point
  EXPECT(moe_fp8_quantize_rows(p, 4, 12, p, reinterpret_cast<float*>(p), nullptr) ==
         MOE_ERR_INVALID_ARG);
  EXPECT(moe_fp8_quantize_rows(p, -1, 8, p, reinterpret_cast<float*>(p), nullptr) ==
         MOE_ERR_INVALID_ARG);
  EXPECT(moe_fp8_quantize_rows(nullptr, 4, 8, p, reinterpret_cast<float*>(p), nullptr) ==
         MOE_ERR_INVALID_ARG);
  EXPECT(moe_fp8_quantize_rows(&buf[8], 4, 8, p, reinterpret_cast<float*>(p), nullptr) ==
         MOE_ERR_INVALID_ARG);
  EXPECT(moe_fp8_quantize_rows(nullptr, 0, 8, nullptr, nullptr, nullptr) == MOE_OK);
  EXPECT(std::strcmp(moe_last_error(), "") == 0);

  std::printf("ok %d checks\n", g_checks);
  return 0;
}
