// Drives every entry point of the C ABI through its validation and planning code with the kernel
// launchers stubbed out (launch_stubs.cpp), for the AddressSanitizer / UndefinedBehaviorSanitizer
// build that test_host_sanitizers.py makes.  Device buffers are fake addresses: the host code only
// carves and forwards them.  Exits 0 when every call returns the expected status.
#include "gmlp.h"

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

static int failures = 0;

#define EXPECT(call, want)                                                                          \
  do {                                                                                              \
    const int got_ = (int)(call);                                                                   \
    if (got_ != (int)(want)) {                                                                      \
      std::fprintf(stderr, "%s:%d: %s returned %d, expected %d (%s)\n", __FILE__, __LINE__, #call, got_, \
                   (int)(want), gmlp_last_error());                                                 \
      ++failures;                                                                                   \
    }                                                                                               \
  } while (0)

static void* fake(uintptr_t a) { return reinterpret_cast<void*>(a); }

static gmlp_grouped_q mx_q(uintptr_t base) {
  gmlp_grouped_q q;
  std::memset(&q, 0, sizeof(q));
  q.row_data = fake(base);
  q.row_scale_mfma = fake(base + 0x1000000);
  q.col_data = fake(base + 0x2000000);
  q.col_scale_mfma = fake(base + 0x3000000);
  return q;
}

static gmlp_grouped_q nv_q(uintptr_t base) {
  gmlp_grouped_q q = mx_q(base);
  q.row_scale = fake(base + 0x4000000);
  q.col_scale = fake(base + 0x5000000);
  q.amax_pre = static_cast<float*>(fake(base + 0x6000000));
  q.amax_post = static_cast<float*>(fake(base + 0x7000000));
  return q;
}

int main() {
  const gmlp_recipe mx{GMLP_MXFP8, 0}, nv{GMLP_NVFP4_RHT, 0xB5E3};
  // ---------------------------------------------------------------- queries
  EXPECT(gmlp_check_support("gfx950", 8, 4096, 1536, GMLP_SWIGLU, mx), GMLP_OK);
  EXPECT(gmlp_check_support("gfx942", 8, 4096, 1536, GMLP_SWIGLU, mx), GMLP_UNSUPPORTED);
  EXPECT(gmlp_check_support("gfx950", 8, 4096, 1500, GMLP_SWIGLU, mx), GMLP_UNSUPPORTED);
  EXPECT(gmlp_check_support("gfx950", 8, 4096, 1536, 9, mx), GMLP_UNSUPPORTED);
  EXPECT(gmlp_check_support("gfx950", 8, 4096, 1536, GMLP_SWIGLU, gmlp_recipe{7, 0}), GMLP_UNSUPPORTED);
  EXPECT(gmlp_check_support("gfx950", 0, 4096, 1536, GMLP_SRELU, nv), GMLP_INVALID_ARG);
  std::vector<char> longname(1000, 'x');
  longname.back() = 0;
  EXPECT(gmlp_check_support(longname.data(), 8, 4096, 1536, GMLP_SWIGLU, mx), GMLP_UNSUPPORTED);
  gmlp_sizes sz;
  EXPECT(gmlp_query_sizes(65536, 128, 7168, 2048, GMLP_SWIGLU, mx, 0, &sz), GMLP_OK);
  EXPECT(gmlp_query_sizes(24576, 8, 5120, 2048, GMLP_SRELU, nv, 1, &sz), GMLP_OK);
  EXPECT(gmlp_query_sizes(0, 2, 128, 128, GMLP_SWIGLU, mx, 0, &sz), GMLP_OK);
  EXPECT(gmlp_query_sizes(64, 2, 128, 128, GMLP_SWIGLU, mx, 0, nullptr), GMLP_INVALID_ARG);
  EXPECT(gmlp_read_device_flags(nullptr, nullptr, nullptr), GMLP_INVALID_ARG);
  int32_t counts[8];
  EXPECT(gmlp_last_launch_counts(counts, 8), GMLP_OK);
  EXPECT(gmlp_last_launch_counts(nullptr, 8), GMLP_INVALID_ARG);
  if (!gmlp_last_error()) ++failures;

  // ---------------------------------------------------------------- group quantize family
  gmlp_grouped_q qm = mx_q(0x10000000), qn = nv_q(0x20000000);
  void* x = fake(0x30000000);
  void* splits = fake(0x31000000);
  EXPECT(gmlp_query_sizes(0, 300, 128, 128, GMLP_SWIGLU, mx, 0, &sz), GMLP_OK);
  std::vector<char> host_ws_probe(1);      // the workspace is never dereferenced on the host
  void* ws = fake(0x40000000);
  const size_t qws = sz.quant_ws_bytes;
  EXPECT(gmlp_group_quantize(x, 1000, 256, static_cast<const int32_t*>(splits), 300, mx, 1, 1, &qm, ws, qws,
                             nullptr), GMLP_OK);
  EXPECT(gmlp_group_quantize(x, 1000, 256, static_cast<const int32_t*>(splits), 300, nv, 1, 1, &qn, ws, qws,
                             nullptr), GMLP_OK);
  EXPECT(gmlp_group_quantize(x, 1000, 256, static_cast<const int32_t*>(splits), 300, mx, 1, 1, &qm, ws, 16,
                             nullptr), GMLP_WORKSPACE);
  EXPECT(gmlp_group_quantize(x, 1000, 100, static_cast<const int32_t*>(splits), 3, mx, 1, 1, &qm, ws, qws,
                             nullptr), GMLP_UNSUPPORTED);
  EXPECT(gmlp_group_quantize(nullptr, 1000, 128, static_cast<const int32_t*>(splits), 3, mx, 1, 1, &qm, ws, qws,
                             nullptr), GMLP_INVALID_ARG);
  EXPECT(gmlp_group_quantize(x, 128LL * 33000, 128, static_cast<const int32_t*>(splits), 1, mx, 1, 1, &qm, ws, qws,
                             nullptr), GMLP_UNSUPPORTED);
  EXPECT(gmlp_group_quantize(x, 1000, 128, static_cast<const int32_t*>(splits), 0, mx, 1, 1, &qm, ws, qws, nullptr),
         GMLP_INVALID_ARG);
  EXPECT(gmlp_group_quantize(x, 1000, 128, static_cast<const int32_t*>(splits), 2, mx, 0, 0, &qm, ws, qws, nullptr),
         GMLP_INVALID_ARG);
  EXPECT(gmlp_group_hadamard_amax(x, 1000, 128, static_cast<const int32_t*>(splits), 4, 0x1234, qn.amax_pre,
                                  qn.amax_post, ws, qws, nullptr), GMLP_OK);
  EXPECT(gmlp_group_quantize_with_amax(x, 1000, 128, static_cast<const int32_t*>(splits), 4, nv, 1, 1, &qn, ws, qws,
                                       nullptr), GMLP_OK);
  EXPECT(gmlp_group_quantize_with_amax(x, 1000, 128, static_cast<const int32_t*>(splits), 4, mx, 1, 1, &qm, ws, qws,
                                       nullptr), GMLP_UNSUPPORTED);

  // ---------------------------------------------------------------- weights
  gmlp_weight_q wm = mx_q(0x50000000), wn = nv_q(0x60000000);
  EXPECT(gmlp_weight_quantize(fake(0x70000000), nullptr, 8, 3072, 4096, mx, &wm, ws, qws, nullptr), GMLP_OK);
  std::vector<const void*> ptrs(8, fake(0x70000000));
  EXPECT(gmlp_weight_quantize(nullptr, ptrs.data(), 8, 2048, 5120, nv, &wn, ws, qws, nullptr), GMLP_OK);
  ptrs[3] = nullptr;
  EXPECT(gmlp_weight_quantize(nullptr, ptrs.data(), 8, 2048, 5120, nv, &wn, ws, qws, nullptr), GMLP_INVALID_ARG);
  EXPECT(gmlp_weight_quantize(fake(0x70000000), nullptr, 8, 3000, 4096, mx, &wm, ws, qws, nullptr), GMLP_UNSUPPORTED);

  // ---------------------------------------------------------------- grouped GEMM
  size_t gws = 0;
  EXPECT(gmlp_grouped_gemm_ws_bytes(GMLP_GEMM_FPROP, nv, 8, 32768, 4096, 3072, &gws), GMLP_OK);
  EXPECT(gmlp_grouped_gemm_ws_bytes(7, mx, 8, 32768, 4096, 3072, &gws), GMLP_INVALID_ARG);
  EXPECT(gmlp_grouped_gemm(GMLP_GEMM_FPROP, mx, &qm, &wm, static_cast<const int32_t*>(splits), 8, 32768, 4096, 3072,
                           fake(0x80000000), GMLP_OUT_BF16, ws, 1 << 20, nullptr), GMLP_OK);
  EXPECT(gmlp_grouped_gemm(GMLP_GEMM_WGRAD, nv, &qn, &qn, static_cast<const int32_t*>(splits), 8, 32768, 4096, 1536,
                           fake(0x80000000), GMLP_OUT_FP32_ACCUMULATE, ws, gws * 4, nullptr), GMLP_OK);
  EXPECT(gmlp_grouped_gemm(GMLP_GEMM_FPROP, mx, &qm, &wm, static_cast<const int32_t*>(splits), 8, 32768, 4096, 3072,
                           fake(0x80000000), GMLP_OUT_FP32_ACCUMULATE, ws, 1 << 20, nullptr), GMLP_UNSUPPORTED);
  EXPECT(gmlp_grouped_gemm(GMLP_GEMM_FPROP, mx, &qm, &wm, static_cast<const int32_t*>(splits), 8, 32768, 4096, 3000,
                           fake(0x80000000), GMLP_OUT_BF16, ws, 1 << 20, nullptr), GMLP_UNSUPPORTED);
  // DGRAD: the weight's dgrad operand as B (n = the weight's K, k = its N)
  EXPECT(gmlp_grouped_gemm_ws_bytes(GMLP_GEMM_DGRAD, nv, 8, 32768, 4096, 3072, &gws), GMLP_OK);
  EXPECT(gmlp_grouped_gemm(GMLP_GEMM_DGRAD, mx, &qm, &wm, static_cast<const int32_t*>(splits), 8, 32768, 4096, 3072,
                           fake(0x80000000), GMLP_OUT_BF16, ws, 1 << 20, nullptr), GMLP_OK);
  EXPECT(gmlp_grouped_gemm(GMLP_GEMM_DGRAD, mx, &qm, &wm, static_cast<const int32_t*>(splits), 8, 32768, 4096, 3000,
                           fake(0x80000000), GMLP_OUT_BF16, ws, 1 << 20, nullptr), GMLP_UNSUPPORTED);
  EXPECT(gmlp_grouped_gemm(GMLP_GEMM_DGRAD, mx, &qm, &wm, static_cast<const int32_t*>(splits), 8, 32768, 4096, 3072,
                           fake(0x80000000), GMLP_OUT_FP32_ACCUMULATE, ws, 1 << 20, nullptr), GMLP_UNSUPPORTED);
  EXPECT(gmlp_grouped_gemm(3, mx, &qm, &wm, static_cast<const int32_t*>(splits), 8, 32768, 4096, 3072,
                           fake(0x80000000), GMLP_OUT_BF16, ws, 1 << 20, nullptr), GMLP_INVALID_ARG);

  // ---------------------------------------------------------------- fused MLP
  for (int kind = 0; kind < 2; ++kind) {
    for (int act = 0; act < 4; ++act) {
      for (int rec = 0; rec < 2; ++rec) {
        const gmlp_recipe r = kind ? nv : mx;
        const int64_t M = 3000, H = 512, ffn = 384;
        const int32_t E = 6;
        EXPECT(gmlp_query_sizes(M, E, H, ffn, act, r, rec, &sz), GMLP_OK);
        gmlp_weight_q w1 = kind ? nv_q(0x90000000) : mx_q(0x90000000);
        gmlp_weight_q w2 = kind ? nv_q(0xA0000000) : mx_q(0xA0000000);
        gmlp_fwd_args f;
        std::memset(&f, 0, sizeof(f));
        f.x = x;
        f.m_splits = static_cast<const int32_t*>(splits);
        f.M = M;
        f.E = E;
        f.H = H;
        f.ffn = ffn;
        f.w1 = &w1;
        f.w2 = &w2;
        f.probs = static_cast<const float*>(fake(0xB0000000));
        f.activation = act;
        f.tanh_clamp_scale = act == GMLP_TANH_SRELU ? 8.0f : 0.0f;
        f.recipe = r;
        f.recompute = rec;
        f.input_requires_grad = f.weight_requires_grad = 1;
        f.y = fake(0xC0000000);
        f.ctx = fake(0x100000000ULL);
        f.ctx_bytes = sz.ctx_bytes;
        f.ws = fake(0x200000000ULL);
        f.ws_bytes = sz.ws_bytes;
        EXPECT(gmlp_grouped_mlp_forward(&f, nullptr), GMLP_OK);
        f.fc2_amax_in_fc1 = 1;
        EXPECT(gmlp_grouped_mlp_forward(&f, nullptr),
               (kind == 1 && (act == GMLP_SRELU || act == GMLP_TANH_SRELU)) ? GMLP_OK : GMLP_UNSUPPORTED);
        f.fc2_amax_in_fc1 = 0;
        if (act == GMLP_TANH_SRELU) {        // the clamp scale must be positive and finite
          f.tanh_clamp_scale = 0.0f;
          EXPECT(gmlp_grouped_mlp_forward(&f, nullptr), GMLP_INVALID_ARG);
          f.tanh_clamp_scale = -1.0f;
          EXPECT(gmlp_grouped_mlp_forward(&f, nullptr), GMLP_INVALID_ARG);
          f.tanh_clamp_scale = 8.0f;
        }
        void* h = nullptr;
        float *pre = nullptr, *post = nullptr;
        EXPECT(gmlp_forward_saved(&f, &h, &pre, &post), GMLP_OK);
        if (h != f.ctx || (kind == 1) != (pre != nullptr)) ++failures;
        f.ctx_bytes = 100;
        EXPECT(gmlp_grouped_mlp_forward(&f, nullptr), GMLP_WORKSPACE);
        EXPECT(gmlp_forward_saved(&f, &h, &pre, &post), GMLP_WORKSPACE);
        f.ctx_bytes = sz.ctx_bytes;
        gmlp_bwd_args b;
        std::memset(&b, 0, sizeof(b));
        b.dy = fake(0xD0000000);
        b.m_splits = f.m_splits;
        b.M = M;
        b.E = E;
        b.H = H;
        b.ffn = ffn;
        b.w1 = &w1;
        b.w2 = &w2;
        b.probs = f.probs;
        b.activation = act;
        b.tanh_clamp_scale = f.tanh_clamp_scale;
        b.recipe = r;
        b.recompute = rec;
        b.input_requires_grad = b.weight_requires_grad = 1;
        b.dx = fake(0xE0000000);
        b.dprobs = static_cast<float*>(fake(0xE8000000));
        b.dw1 = fake(0xF0000000);
        b.dw2 = fake(0xF8000000);
        b.wgrad_dtype = GMLP_OUT_FP32_ACCUMULATE;
        b.ctx = f.ctx;
        b.ctx_bytes = sz.ctx_bytes;
        b.ws = f.ws;
        b.ws_bytes = sz.ws_bytes;
        EXPECT(gmlp_grouped_mlp_backward(&b, nullptr), GMLP_OK);
        // a deferred wgrad on a workspace whose last backward did not defer, and a backward whose
        // settings differ from the forward that wrote ctx, are rejected
        EXPECT(gmlp_grouped_mlp_wgrad(&b, nullptr), GMLP_INVALID_ARG);
        if (!rec) {                          // (the recompute plan needs a larger workspace)
          b.recompute = 1;
          b.ws_bytes = 4 * sz.ws_bytes;
          EXPECT(gmlp_grouped_mlp_backward(&b, nullptr), GMLP_INVALID_ARG);
          b.recompute = 0;
          b.ws_bytes = sz.ws_bytes;
        }
        if (act == GMLP_TANH_SRELU) {
          b.tanh_clamp_scale = 4.0f;
          EXPECT(gmlp_grouped_mlp_backward(&b, nullptr), GMLP_INVALID_ARG);
          b.tanh_clamp_scale = f.tanh_clamp_scale;
        }
        if (act == GMLP_TANH_SRELU) {
          b.tanh_clamp_scale = 0.0f;
          EXPECT(gmlp_grouped_mlp_backward(&b, nullptr), GMLP_INVALID_ARG);
          b.tanh_clamp_scale = f.tanh_clamp_scale;
        }
        b.defer_wgrad = 1;
        EXPECT(gmlp_grouped_mlp_backward(&b, nullptr), GMLP_OK);
        EXPECT(gmlp_grouped_mlp_wgrad(&b, nullptr), GMLP_OK);
        b.ws_bytes = 64;
        EXPECT(gmlp_grouped_mlp_backward(&b, nullptr), GMLP_WORKSPACE);
        b.ws_bytes = sz.ws_bytes;
        b.wgrad_dtype = 9;
        b.defer_wgrad = 0;
        EXPECT(gmlp_grouped_mlp_backward(&b, nullptr), GMLP_INVALID_ARG);
      }
    }
  }
  gmlp_fwd_args bad;
  std::memset(&bad, 0, sizeof(bad));
  EXPECT(gmlp_grouped_mlp_forward(nullptr, nullptr), GMLP_INVALID_ARG);
  bad.E = 2;
  bad.M = 64;
  bad.H = 128;
  bad.ffn = 100;
  bad.recipe = mx;
  EXPECT(gmlp_grouped_mlp_forward(&bad, nullptr), GMLP_UNSUPPORTED);
  (void)host_ws_probe;
  if (failures) std::fprintf(stderr, "%d unexpected statuses\n", failures);
  else std::printf("all statuses as expected\n");
  return failures ? 1 : 0;
}
