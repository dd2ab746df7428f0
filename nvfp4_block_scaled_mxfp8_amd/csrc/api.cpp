// C ABI of libgmlp: validation, workspace carving and the launch plan of the fused grouped MLP.
//
// The launch plan follows "GEMM + Swiglu fused Grouped MLP for MXFP8" (sequence
// diagram) for MXFP8 and "Reduce NVFP4 quantization work for the fused
// GroupedMLP fc2 input with activation recompute" (Description, Changes) for
// NVFP4: the recompute decision is taken before the fc2-input cast, so the
// forward casts fc2_x row-wise only when the backward rebuilds it; the forward
// keeps the fc2_x (pre, post) amax; the backward casts the rebuilt fc2_x with
// that amax and runs no second Hadamard-amax pass.
#include "gmlp.h"
#include "kernels.h"
#include "planner.h"

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

using namespace gmlp;

namespace {

thread_local std::string g_err;
thread_local int32_t g_counts[8];

enum { CNT_SCAN = 0, CNT_MXQ = 1, CNT_HAMAX = 2, CNT_NVQ = 3, CNT_GEMM = 4, CNT_DPROB = 5, CNT_FILL = 6 };

gmlp_status fail(gmlp_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}
gmlp_status ok() {
  g_err.clear();
  return GMLP_OK;
}

#define HIP_TRY(expr)                                                                  \
  do {                                                                                 \
    hipError_t e_ = (expr);                                                            \
    if (e_ != hipSuccess) return fail(GMLP_HIP_ERROR, "system: %s failed: %s", #expr, \
                                      hipGetErrorString(e_));                          \
  } while (0)

// Bump allocator over a caller buffer (base == nullptr: sizing pass).
struct Bump {
  uint8_t* base;
  size_t off = 0;
  explicit Bump(void* b) : base(static_cast<uint8_t*>(b)) {}
  template <class T>
  T* take(size_t count) {
    off = (off + 255) & ~size_t(255);
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
};

SplitTables carve_tables(Bump& b, int G) {
  SplitTables T;
  T.flags = b.take<uint32_t>(1);
  T.row_off = b.take<int32_t>(G + 1);
  T.col_off = b.take<int32_t>(G + 1);
  T.colw_off = b.take<int32_t>(G + 1);
  T.t128_off = b.take<int32_t>(G + 1);
  T.t256_off = b.take<int32_t>(G + 1);
  T.amax_slots = b.take<uint32_t>(2 * (size_t)G * kAmaxSlots);
  return T;
}

bool is_mx(const gmlp_recipe& r) { return r.kind == GMLP_MXFP8; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
// Upper bounds of the padded column-wise extents for M rows in G groups.
int64_t pad_rows_bound(int64_t M, int G) { return M + 127LL * G; }
int64_t pad_words_bound(int64_t M, int G) { return ceil_div(M, 128) + G; }

// Buffers of one group-quantized activation tensor [M, K].
struct QBuf {
  gmlp_grouped_q q{};
};

QBuf carve_q(Bump& b, const gmlp_recipe& r, int64_t M, int64_t K, int G, bool row, bool col, bool amax) {
  QBuf o;
  const int64_t PR = pad_rows_bound(M, G);
  if (is_mx(r)) {
    if (row) {
      o.q.row_data = b.take<uint8_t>(M * K);
      o.q.row_scale_mfma = b.take<uint32_t>(ceil_div(K, 128) * M);
    }
    if (col) {
      o.q.col_data = b.take<uint8_t>(K * PR);
      o.q.col_scale_mfma = b.take<uint32_t>(K * pad_words_bound(M, G));
    }
  } else {
    // NVFP4 inside the fused MLP: only the GEMMs read these casts, so they are kept as the
    // bf16 panels the GEMMs take (the packed E2M1 / E4M3 form is not written)
    if (row) o.q.row_bf16 = b.take<uint8_t>(2 * M * K);
    if (col) o.q.col_bf16 = b.take<uint8_t>(2 * K * PR);
    if (amax) {
      o.q.amax_pre = b.take<float>(G);
      o.q.amax_post = b.take<float>(G);
    }
  }
  return o;
}

// NVFP4 cast outputs of q (direction not wanted: null).
NvOut nv_out(const gmlp_grouped_q& q, bool row, bool col) {
  NvOut o{row ? static_cast<uint8_t*>(q.row_data) : nullptr, row ? static_cast<uint8_t*>(q.row_scale) : nullptr,
          col ? static_cast<uint8_t*>(q.col_data) : nullptr, col ? static_cast<uint8_t*>(q.col_scale) : nullptr};
  o.row_bf16 = row ? static_cast<uint8_t*>(q.row_bf16) : nullptr;
  o.col_bf16 = col ? static_cast<uint8_t*>(q.col_bf16) : nullptr;
  return o;
}

struct Launcher {
  hipStream_t s;
  gmlp_status st = GMLP_OK;
  bool check(hipError_t e, const char* what) {
    if (e != hipSuccess) {
      fail(GMLP_HIP_ERROR, "system: launching %s failed: %s", what, hipGetErrorString(e));
      st = GMLP_HIP_ERROR;
      return false;
    }
    return true;
  }
};

// ----------------------------------------------------------------------------- validation
gmlp_status check_recipe(const gmlp_recipe& r) {
  if (r.kind != GMLP_MXFP8 && r.kind != GMLP_NVFP4_RHT)
    return fail(GMLP_UNSUPPORTED, "recipe: requires an MXFP8 or NVFP4 (with RHT) recipe, got kind %d", r.kind);
  return GMLP_OK;
}

gmlp_status check_dims(int64_t M, int64_t K, int G) {
  if (G < 1) return fail(GMLP_INVALID_ARG, "dims: number of groups must be >= 1, got %d", G);
  if (M < 0) return fail(GMLP_INVALID_ARG, "dims: M must be >= 0, got %lld", (long long)M);
  if (K <= 0 || K % 32 != 0) return fail(GMLP_UNSUPPORTED, "dims: K must be a positive multiple of 32, got %lld", (long long)K);
  if (M + 127LL * G > (1LL << 30)) return fail(GMLP_UNSUPPORTED, "dims: M = %lld rows is too large", (long long)M);
  // one launch covers both 64-row halves of every 128-row tile of every group along the grid's
  // y dimension (at most 65535)
  if (2 * ((M + 127) / 128 + G) > 65535)
    return fail(GMLP_UNSUPPORTED, "dims: M = %lld rows in %d groups exceeds one launch's tile range", (long long)M, G);
  return GMLP_OK;
}

gmlp_status quant_core(const void* x, int64_t M, int64_t K, const int32_t* m_splits, int G, const gmlp_recipe& r,
                       bool row, bool col, const gmlp_grouped_q* out, void* ws, size_t ws_bytes,
                       hipStream_t stream, bool compute_amax) {
  gmlp_status st;
  if ((st = check_recipe(r)) != GMLP_OK) return st;
  if ((st = check_dims(M, K, G)) != GMLP_OK) return st;
  if (!out || (M > 0 && !x) || !m_splits) return fail(GMLP_INVALID_ARG, "null pointer argument");
  if (!row && !col && !compute_amax) return fail(GMLP_INVALID_ARG, "nothing requested (want_row = want_col = 0)");
  const bool rows_exist = M > 0;   // an empty tensor has no row-wise buffers to check
  if (is_mx(r)) {
    if (rows_exist && row && (!out->row_data || (!out->row_scale && !out->row_scale_mfma)))
      return fail(GMLP_INVALID_ARG, "row-wise output buffers missing");
    if (col && (!out->col_data || (!out->col_scale && !out->col_scale_mfma)))
      return fail(GMLP_INVALID_ARG, "column-wise output buffers missing");
  } else {
    // packed data needs its scales; the bf16 panels may stand alone
    if (rows_exist && row && ((!out->row_data && !out->row_bf16) || (out->row_data && !out->row_scale)))
      return fail(GMLP_INVALID_ARG, "row-wise output buffers missing");
    if (col && ((!out->col_data && !out->col_bf16) || (out->col_data && !out->col_scale)))
      return fail(GMLP_INVALID_ARG, "column-wise output buffers missing");
    if (!out->amax_pre || !out->amax_post) return fail(GMLP_INVALID_ARG, "NVFP4 needs amax_pre and amax_post");
  }
  Bump b(ws);
  SplitTables T = carve_tables(b, G);
  if (!ws || ws_bytes < b.off) return fail(GMLP_WORKSPACE, "workspace too small: need %zu bytes", b.off);
  Launcher L{stream};
  if (!L.check(launch_scan(m_splits, G, M, T, stream), "scan")) return L.st;
  g_counts[CNT_SCAN]++;
  const uint16_t* xx = static_cast<const uint16_t*>(x);
  if (is_mx(r)) {
    MxOut o{static_cast<uint8_t*>(row ? out->row_data : nullptr), static_cast<uint8_t*>(row ? out->row_scale : nullptr),
            static_cast<uint32_t*>(row ? out->row_scale_mfma : nullptr),
            static_cast<uint8_t*>(col ? out->col_data : nullptr), static_cast<uint8_t*>(col ? out->col_scale : nullptr),
            static_cast<uint32_t*>(col ? out->col_scale_mfma : nullptr)};
    if (!L.check(launch_mxfp8_quant(xx, M, K, T, G, row, col, o, stream), "mxfp8 quantize")) return L.st;
    g_counts[CNT_MXQ]++;
    return ok();
  }
  if (compute_amax) {
    if (!L.check(launch_hadamard_amax(xx, M, K, T, G, r.rht_sign_mask & 0xFFFFu, out->amax_pre, out->amax_post,
                                      stream), "hadamard amax"))
      return L.st;
    g_counts[CNT_HAMAX]++;
  }
  if (row || col) {
    const NvOut o = nv_out(*out, row, col);
    if (!L.check(launch_nvfp4_quant(xx, M, K, T, G, r.rht_sign_mask & 0xFFFFu, true, row, col, out->amax_pre,
                                    out->amax_post, o, stream), "nvfp4 quantize"))
      return L.st;
    g_counts[CNT_NVQ]++;
  }
  return ok();
}

// Operand of the GEMM kernels from a quantized tensor.
GemmOperand op_row(const gmlp_grouped_q& q, const float* amax) {
  GemmOperand o;
  o.data = static_cast<const uint8_t*>(q.row_data);
  o.scale_mfma = static_cast<const uint32_t*>(q.row_scale_mfma);
  o.scale = static_cast<const uint8_t*>(q.row_scale);
  o.amax = amax;
  o.bf16 = static_cast<const uint8_t*>(q.row_bf16);
  return o;
}
GemmOperand op_col(const gmlp_grouped_q& q, const float* amax) {
  GemmOperand o;
  o.data = static_cast<const uint8_t*>(q.col_data);
  o.scale_mfma = static_cast<const uint32_t*>(q.col_scale_mfma);
  o.scale = static_cast<const uint8_t*>(q.col_scale);
  o.amax = amax;
  o.bf16 = static_cast<const uint8_t*>(q.col_bf16);
  return o;
}

GemmArgs gemm_base(int mode, const gmlp_recipe& r, int epi, SplitTables T, int G) {
  GemmArgs g;
  memset(&g, 0, sizeof(g));
  g.mode = mode;
  g.fmt = is_mx(r) ? FMT_MXFP8 : FMT_NVFP4;
  g.epi = epi;
  g.T = T;
  g.G = G;
  return g;
}

gmlp_status weight_ok(const gmlp_weight_q* w, const gmlp_recipe& r, bool fprop, bool dgrad) {
  if (!w) return fail(GMLP_INVALID_ARG, "null weight descriptor");
  const bool f_ok = is_mx(r) ? (w->row_data && w->row_scale_mfma) : (w->row_bf16 || (w->row_data && w->row_scale));
  const bool d_ok = is_mx(r) ? (w->col_data && w->col_scale_mfma) : (w->col_bf16 || (w->col_data && w->col_scale));
  if (fprop && !f_ok) return fail(GMLP_INVALID_ARG, "weight fprop operand (row-wise data and scales) missing");
  if (dgrad && !d_ok) return fail(GMLP_INVALID_ARG, "weight dgrad operand (column-wise data and scales) missing");
  if (!is_mx(r) && !w->amax_pre) return fail(GMLP_INVALID_ARG, "NVFP4 weights need their per-expert amax (amax_pre)");
  return GMLP_OK;
}

// ----------------------------------------------------------------------------- saved-plan records
// What a forward wrote into a ctx buffer, and what a backward left in its workspace, keyed by the
// buffer's address (an address only: never dereferenced).  The backward and the deferred wgrad
// call check their own settings against the record and reject a mismatch, with which they would
// read the buffer in another layout (different offsets, or operands never written).  The records
// are process-wide and bounded (the oldest is dropped); a buffer with no record (written by
// another process, or dropped) is taken as it is.
struct SavedPlan {
  const void* key = nullptr;
  uint64_t stamp = 0;
  int64_t M = 0, H = 0, ffn = 0;
  int E = 0, act = 0, kind = 0, recompute = 0, wgrad = 0, deferred = 0;
  uint32_t mask = 0;
  float clamp = 0.0f;
};
constexpr int kSavedPlans = 512;
std::mutex g_plans_mu;
SavedPlan g_plans[kSavedPlans];
uint64_t g_plan_stamp = 0;

SavedPlan plan_of(const void* key, int64_t M, int E, int64_t H, int64_t ffn, int act, float clamp,
                  const gmlp_recipe& r, int recompute, int wgrad, int deferred) {
  SavedPlan p;
  p.key = key;
  p.M = M;
  p.E = E;
  p.H = H;
  p.ffn = ffn;
  p.act = act;
  p.clamp = act == GMLP_TANH_SRELU ? clamp : 0.0f;
  p.kind = r.kind;
  p.mask = r.kind == GMLP_NVFP4_RHT ? (r.rht_sign_mask & 0xFFFF) : 0u;
  p.recompute = recompute != 0;
  p.wgrad = wgrad != 0;
  p.deferred = deferred != 0;
  return p;
}
void remember_plan(const SavedPlan& p) {
  std::lock_guard<std::mutex> lock(g_plans_mu);
  int slot = 0;
  for (int i = 0; i < kSavedPlans; ++i) {
    if (g_plans[i].key == p.key) { slot = i; break; }
    if (g_plans[i].stamp < g_plans[slot].stamp) slot = i;
  }
  g_plans[slot] = p;
  g_plans[slot].stamp = ++g_plan_stamp;
}
bool recall_plan(const void* key, SavedPlan* out) {
  std::lock_guard<std::mutex> lock(g_plans_mu);
  for (int i = 0; i < kSavedPlans; ++i)
    if (g_plans[i].key == key && g_plans[i].stamp) {
      *out = g_plans[i];
      return true;
    }
  return false;
}
// The first setting in which `want` differs from the record (nullptr: none).
const char* plan_mismatch(const SavedPlan& have, const SavedPlan& want) {
  if (have.M != want.M) return "M";
  if (have.E != want.E) return "E";
  if (have.H != want.H) return "hidden";
  if (have.ffn != want.ffn) return "ffn";
  if (have.act != want.act) return "activation";
  if (have.clamp != want.clamp) return "tanh_clamp_scale";
  if (have.kind != want.kind) return "recipe";
  if (have.mask != want.mask) return "rht_sign_mask";
  if (have.recompute != want.recompute) return "recompute";
  return nullptr;
}
// ctx: written by a forward with these settings (and, when the caller needs the weight-gradient
// operands, one that saved them).
gmlp_status check_ctx_plan(const SavedPlan& want) {
  SavedPlan have;
  if (!recall_plan(want.key, &have)) return GMLP_OK;
  if (const char* f = plan_mismatch(have, want))
    return fail(GMLP_INVALID_ARG, "ctx: written by a forward with a different %s", f);
  if (want.wgrad && !have.wgrad)
    return fail(GMLP_INVALID_ARG, "ctx: the forward saved no weight-gradient operands (weight_requires_grad 0)");
  return GMLP_OK;
}

// ----------------------------------------------------------------------------- MLP plan
// Width of h: the gated activations (SwiGLU, QGeGLU) read [gate | up].
int64_t f1_of(int act, int64_t ffn) { return (act == GMLP_SWIGLU || act == GMLP_QGEGLU) ? 2 * ffn : ffn; }
// The activation as the kernels take it; its parameter is checked by check_act.
Act act_of(int act, float tanh_clamp_scale) {
  Act a;
  a.kind = act;
  a.c = act == GMLP_TANH_SRELU ? tanh_clamp_scale : 0.0f;
  return a;
}
gmlp_status check_act(int act, float tanh_clamp_scale) {
  if (act == GMLP_TANH_SRELU && !(tanh_clamp_scale > 0.0f && tanh_clamp_scale <= 3.0e38f))
    return fail(GMLP_INVALID_ARG, "activation: the tanh clamp scale must be a positive finite number, got %g",
                (double)tanh_clamp_scale);
  return GMLP_OK;
}

struct FwdCtx {     // saved tensors (in ctx)
  uint16_t* h;
  QBuf xq_col;      // column-wise x (+ NVFP4 amax)
  QBuf aq_col;      // column-wise fc2 input when not recomputing
  float* a_pre;     // NVFP4 fc2-input amax (kept for the recompute cast)
  float* a_post;
};

FwdCtx carve_ctx(Bump& b, int64_t M, int E, int64_t H, int64_t ffn, int act, const gmlp_recipe& r, bool recompute) {
  const int64_t F1 = f1_of(act, ffn);
  FwdCtx c{};
  c.h = b.take<uint16_t>(M * F1);
  c.xq_col = carve_q(b, r, M, H, E, false, true, true);
  if (!recompute) c.aq_col = carve_q(b, r, M, ffn, E, false, true, false);
  if (!is_mx(r)) {
    c.a_pre = b.take<float>(E);
    c.a_post = b.take<float>(E);
  }
  return c;
}

// NVFP4 GEMM scratch: the two operands of one GEMM expanded to bf16 (see GemmArgs::xa, xb).
struct NvScratch {
  uint8_t* xa = nullptr;
  uint8_t* xb = nullptr;
};
NvScratch carve_nv(Bump& b, const gmlp_recipe& r, int64_t a_elems, int64_t b_elems) {
  NvScratch n;
  if (is_mx(r)) return n;
  n.xa = b.take<uint8_t>(2 * a_elems);
  n.xb = b.take<uint8_t>(2 * b_elems);
  return n;
}
void set_nv(GemmArgs& g, const NvScratch& n) {
  g.xa = n.xa;
  g.xb = n.xb;
}

struct FwdWs {
  SplitTables T;
  QBuf xq_row;
  QBuf aq_row;
  NvScratch nv;
};
FwdWs carve_fwd_ws(Bump& b, int64_t M, int E, int64_t H, int64_t ffn, int act, const gmlp_recipe& r) {
  const int64_t F1 = f1_of(act, ffn);
  FwdWs w;
  w.T = carve_tables(b, E);
  w.xq_row = carve_q(b, r, M, H, E, true, false, false);
  w.aq_row = carve_q(b, r, M, ffn, E, true, false, false);
  // fc1: x [M, H] and W1 [E, F1, H]; fc2: a [M, ffn] and W2 [E, H, ffn]
  w.nv = carve_nv(b, r, M * std::max(H, ffn), (int64_t)E * H * std::max(F1, ffn));
  return w;
}

struct BwdWs {
  SplitTables T;
  QBuf dyq;
  uint16_t* dh;
  QBuf dhq;
  uint16_t* a2;
  QBuf a2q;
  float* dprob_part;
  NvScratch nv;
  uint16_t* da;       // NVFP4: bf16 da between the fc2 dgrad and the activation gradient
};
int dact_ntiles(int64_t ffn) { return (int)ceil_div(ffn, 256); }
BwdWs carve_bwd_ws(Bump& b, int64_t M, int E, int64_t H, int64_t ffn, int act, const gmlp_recipe& r, bool recompute) {
  const int64_t F1 = f1_of(act, ffn);
  BwdWs w{};
  w.T = carve_tables(b, E);
  w.dyq = carve_q(b, r, M, H, E, true, true, true);
  w.dh = b.take<uint16_t>(M * F1);
  w.dhq = carve_q(b, r, M, F1, E, true, true, true);
  if (recompute) {
    w.a2 = b.take<uint16_t>(M * ffn);
    w.a2q = carve_q(b, r, M, ffn, E, false, true, false);
  }
  // dL/dp partials: per 256-feature tile of the NVFP4 activation-gradient pass, per 64 features
  // of the MXFP8 activation-gradient cast
  w.dprob_part = b.take<float>((size_t)ceil_div(ffn, 64) * M);
  // NVFP4 GEMM operands: A up to [padded tokens, max(H, F1)] (dy, dh row- or column-wise), B up to
  // the larger of the weights [E, H, F1] and a column-wise [max(H, ffn), padded tokens]
  const int64_t Pt = M + 127LL * E;
  w.nv = carve_nv(b, r, Pt * std::max(H, F1), std::max((int64_t)E * H * F1, std::max(H, ffn) * Pt));
  if (!is_mx(r)) w.da = b.take<uint16_t>(M * ffn);
  return w;
}

gmlp_status mlp_common_checks(int64_t M, int E, int64_t H, int64_t ffn, int act, const gmlp_recipe& r) {
  gmlp_status st;
  if ((st = check_recipe(r)) != GMLP_OK) return st;
  if (act != GMLP_SWIGLU && act != GMLP_SRELU && act != GMLP_TANH_SRELU && act != GMLP_QGEGLU)
    return fail(GMLP_UNSUPPORTED, "activation: unsupported activation %d", act);
  if ((st = check_dims(M, H, E)) != GMLP_OK) return st;
  if (ffn <= 0 || ffn % 128 != 0) return fail(GMLP_UNSUPPORTED, "dims: ffn must be a positive multiple of 128, got %lld", (long long)ffn);
  if (H % 128 != 0) return fail(GMLP_UNSUPPORTED, "dims: hidden must be a multiple of 128, got %lld", (long long)H);
  // the NVFP4 activation-gradient pass covers 8 rows per workgroup along the grid's y dimension
  if (!is_mx(r) && (M + 7) / 8 > 65535)
    return fail(GMLP_UNSUPPORTED, "dims: M = %lld rows exceeds one launch's row range", (long long)M);
  // the GEMMs address every quantized operand with 32-bit offsets
  const int64_t F1 = f1_of(act, ffn);
  const int64_t eb = is_mx(r) ? 1 : 2;             // NVFP4 operands run expanded to bf16
  if (eb * (M + 127LL * E) * std::max(H, F1) >= (1LL << 32) || eb * (int64_t)E * F1 * H >= (1LL << 32))
    return fail(GMLP_UNSUPPORTED, "dims: a quantized operand would reach 4 GB (M = %lld, hidden %lld, ffn %lld)",
                (long long)M, (long long)H, (long long)ffn);
  return GMLP_OK;
}

}  // namespace

namespace gmlp {

gmlp_status set_error(gmlp_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

size_t group_quantize_ws_need(int G) {
  Bump b(nullptr);
  carve_tables(b, G);
  return b.off;
}

gmlp_status group_quantize_on(const void* x, int64_t M, int64_t K, const int32_t* m_splits, int32_t G,
                              gmlp_recipe recipe, int32_t want_row, int32_t want_col, const gmlp_grouped_q* out,
                              void* ws, size_t ws_bytes, hipStream_t stream) {
  memset(g_counts, 0, sizeof(g_counts));
  return quant_core(x, M, K, m_splits, G, recipe, want_row != 0, want_col != 0, out, ws, ws_bytes, stream,
                    !is_mx(recipe));
}

}  // namespace gmlp

// =============================================================================== C ABI
extern "C" {

const char* gmlp_last_error(void) { return g_err.c_str(); }

gmlp_status gmlp_check_support(const char* arch, int32_t experts, int64_t hidden, int64_t ffn, int32_t activation,
                               gmlp_recipe recipe) {
  char name[256] = {0};
  if (arch) {
    strncpy(name, arch, sizeof(name) - 1);
  } else {
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n == 0) return fail(GMLP_UNSUPPORTED, "system: no HIP device available");
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, 0) != hipSuccess) return fail(GMLP_UNSUPPORTED, "system: cannot query device 0");
    strncpy(name, p.gcnArchName, sizeof(name) - 1);
  }
  if (strncmp(name, "gfx950", 6) != 0)
    return fail(GMLP_UNSUPPORTED, "system: unsupported device architecture %s (this library is built for gfx950)", name);
  gmlp_status st = mlp_common_checks(0, experts, hidden, ffn, activation, recipe);
  if (st != GMLP_OK) return st;
  return ok();
}

gmlp_status gmlp_query_sizes(int64_t M, int32_t experts, int64_t hidden, int64_t ffn, int32_t activation,
                             gmlp_recipe recipe, int32_t recompute, gmlp_sizes* out) {
  if (!out) return fail(GMLP_INVALID_ARG, "null output");
  gmlp_status st = mlp_common_checks(M, experts, hidden, ffn, activation, recipe);
  if (st != GMLP_OK) return st;
  Bump c(nullptr);
  carve_ctx(c, M, experts, hidden, ffn, activation, recipe, recompute != 0);
  Bump f(nullptr);
  carve_fwd_ws(f, M, experts, hidden, ffn, activation, recipe);
  Bump b(nullptr);
  carve_bwd_ws(b, M, experts, hidden, ffn, activation, recipe, recompute != 0);
  Bump q(nullptr);
  carve_tables(q, experts);
  out->ctx_bytes = c.off + 256;
  out->ws_bytes = std::max(f.off, b.off) + 256;
  out->quant_ws_bytes = q.off + 256;
  return ok();
}

gmlp_status gmlp_read_device_flags(const void* ws, uint32_t* flags, hipStream_t stream) {
  if (!ws || !flags) return fail(GMLP_INVALID_ARG, "null pointer argument");
  HIP_TRY(hipMemcpyAsync(flags, ws, sizeof(uint32_t), hipMemcpyDeviceToHost, stream));
  HIP_TRY(hipStreamSynchronize(stream));
  return ok();
}

gmlp_status gmlp_last_launch_counts(int32_t* counts, int32_t n) {
  if (!counts) return fail(GMLP_INVALID_ARG, "null pointer argument");
  for (int i = 0; i < n && i < 8; ++i) counts[i] = g_counts[i];
  return ok();
}

gmlp_status gmlp_group_quantize(const void* x, int64_t M, int64_t K, const int32_t* m_splits, int32_t G,
                                gmlp_recipe recipe, int32_t want_row, int32_t want_col, const gmlp_grouped_q* out,
                                void* ws, size_t ws_bytes, hipStream_t stream) {
  return gmlp::group_quantize_on(x, M, K, m_splits, G, recipe, want_row, want_col, out, ws, ws_bytes, stream);
}

gmlp_status gmlp_group_hadamard_amax(const void* x, int64_t M, int64_t K, const int32_t* m_splits, int32_t G,
                                     uint32_t rht_sign_mask, float* amax_pre, float* amax_post, void* ws,
                                     size_t ws_bytes, hipStream_t stream) {
  memset(g_counts, 0, sizeof(g_counts));
  gmlp_grouped_q q{};
  q.amax_pre = amax_pre;
  q.amax_post = amax_post;
  gmlp_recipe r{GMLP_NVFP4_RHT, rht_sign_mask};
  return quant_core(x, M, K, m_splits, G, r, false, false, &q, ws, ws_bytes, stream, true);
}

gmlp_status gmlp_group_quantize_with_amax(const void* x, int64_t M, int64_t K, const int32_t* m_splits, int32_t G,
                                          gmlp_recipe recipe, int32_t want_row, int32_t want_col,
                                          const gmlp_grouped_q* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  memset(g_counts, 0, sizeof(g_counts));
  if (recipe.kind != GMLP_NVFP4_RHT)
    return fail(GMLP_UNSUPPORTED, "recipe: quantize_with_amax applies to the NVFP4 recipe only");
  if (!want_row && !want_col) return fail(GMLP_INVALID_ARG, "nothing requested (want_row = want_col = 0)");
  return quant_core(x, M, K, m_splits, G, recipe, want_row != 0, want_col != 0, out, ws, ws_bytes, stream, false);
}

gmlp_status gmlp_weight_quantize(const void* w, const void* const* w_ptrs, int32_t E, int64_t N, int64_t K,
                                 gmlp_recipe recipe, const gmlp_weight_q* out, void* ws, size_t ws_bytes,
                                 hipStream_t stream) {
  memset(g_counts, 0, sizeof(g_counts));
  gmlp_status st;
  if ((st = check_recipe(recipe)) != GMLP_OK) return st;
  if (E < 1 || N <= 0 || N % 128 != 0 || K <= 0 || K % 128 != 0)
    return fail(GMLP_UNSUPPORTED, "dims: weights need E >= 1 and N, K positive multiples of 128");
  if (!out || (!w && !w_ptrs)) return fail(GMLP_INVALID_ARG, "null pointer argument");
  if (!out->row_data || !out->col_data) return fail(GMLP_INVALID_ARG, "weight output data buffers missing");
  if (is_mx(recipe) ? (!out->row_scale_mfma || !out->col_scale_mfma) : (!out->row_scale || !out->col_scale || !out->amax_pre))
    return fail(GMLP_INVALID_ARG, "weight output scale buffers missing");
  if (is_mx(recipe) && (out->row_bf16 || out->col_bf16))
    return fail(GMLP_INVALID_ARG, "bf16 operand panels apply to the NVFP4 recipe only");
  Bump b(ws);
  SplitTables T = carve_tables(b, 1);
  int32_t* split = b.take<int32_t>(1);
  if (!ws || ws_bytes < b.off) return fail(GMLP_WORKSPACE, "workspace too small: need %zu bytes", b.off);
  Launcher L{stream};
  if (!L.check(launch_fill_u32(reinterpret_cast<uint32_t*>(split), (uint32_t)N, 1, stream), "fill")) return L.st;
  if (!L.check(launch_scan(split, 1, N, T, stream), "scan")) return L.st;
  const int64_t nkt = ceil_div(K, 128), nkt_t = ceil_div(N, 128);
  for (int e = 0; e < E; ++e) {
    const uint16_t* src = w ? static_cast<const uint16_t*>(w) + (int64_t)e * N * K : static_cast<const uint16_t*>(w_ptrs[e]);
    if (!src) return fail(GMLP_INVALID_ARG, "null expert weight pointer %d", e);
    if (is_mx(recipe)) {
      MxOut o{static_cast<uint8_t*>(out->row_data) + (int64_t)e * N * K,
              out->row_scale ? static_cast<uint8_t*>(out->row_scale) + (int64_t)e * N * (K / 32) : nullptr,
              static_cast<uint32_t*>(out->row_scale_mfma) + (int64_t)e * nkt * N,
              static_cast<uint8_t*>(out->col_data) + (int64_t)e * N * K,
              out->col_scale ? static_cast<uint8_t*>(out->col_scale) + (int64_t)e * N * (K / 32) : nullptr,
              static_cast<uint32_t*>(out->col_scale_mfma) + (int64_t)e * nkt_t * K};
      if (!L.check(launch_mxfp8_quant(src, N, K, T, 1, true, true, o, stream), "mxfp8 weight quantize")) return L.st;
      g_counts[CNT_MXQ]++;
    } else {
      float* amax = out->amax_pre + e;
      if (!L.check(launch_weight_amax(src, nullptr, 1, N, K, amax, stream), "weight amax")) return L.st;
      NvOut o{static_cast<uint8_t*>(out->row_data) + (int64_t)e * N * K / 2,
              static_cast<uint8_t*>(out->row_scale) + (int64_t)e * N * K / 16,
              static_cast<uint8_t*>(out->col_data) + (int64_t)e * N * K / 2,
              static_cast<uint8_t*>(out->col_scale) + (int64_t)e * N * K / 16};
      // expert e's panels: fprop [N rows, K], dgrad [K rows, N] (the one group's column-wise cast)
      o.row_bf16 = out->row_bf16 ? static_cast<uint8_t*>(out->row_bf16) + 2 * (int64_t)e * N * K : nullptr;
      o.col_bf16 = out->col_bf16 ? static_cast<uint8_t*>(out->col_bf16) + 2 * (int64_t)e * N * K : nullptr;
      if (!L.check(launch_nvfp4_quant(src, N, K, T, 1, 0u, false, true, true, amax, amax, o, stream),
                   "nvfp4 weight quantize"))
        return L.st;
      g_counts[CNT_NVQ]++;
    }
  }
  return ok();
}

gmlp_status gmlp_grouped_gemm_ws_bytes(int32_t layout, gmlp_recipe recipe, int32_t G, int64_t M, int64_t n, int64_t k,
                                       size_t* bytes) {
  if (!bytes) return fail(GMLP_INVALID_ARG, "null output");
  gmlp_status st;
  if ((st = check_recipe(recipe)) != GMLP_OK) return st;
  if (layout != GMLP_GEMM_FPROP && layout != GMLP_GEMM_WGRAD && layout != GMLP_GEMM_DGRAD)
    return fail(GMLP_INVALID_ARG, "unknown GEMM layout %d", layout);
  if (G < 1 || M < 0 || n <= 0 || k <= 0) return fail(GMLP_INVALID_ARG, "dims: G, n, k must be positive and M >= 0");
  Bump bb(nullptr);
  carve_tables(bb, G);
  const int64_t Pt = M + 127LL * G;
  if (layout != GMLP_GEMM_WGRAD) carve_nv(bb, recipe, M * k, (int64_t)G * n * k);
  else carve_nv(bb, recipe, n * Pt, k * Pt);
  *bytes = bb.off + 256;
  return ok();
}

gmlp_status gmlp_grouped_gemm(int32_t layout, gmlp_recipe recipe, const gmlp_grouped_q* a, const gmlp_grouped_q* b,
                              const int32_t* m_splits, int32_t G, int64_t M, int64_t n, int64_t k, void* c,
                              int32_t out_dtype, void* ws, size_t ws_bytes, hipStream_t stream) {
  memset(g_counts, 0, sizeof(g_counts));
  gmlp_status st;
  if ((st = check_recipe(recipe)) != GMLP_OK) return st;
  if (layout != GMLP_GEMM_FPROP && layout != GMLP_GEMM_WGRAD && layout != GMLP_GEMM_DGRAD)
    return fail(GMLP_INVALID_ARG, "unknown GEMM layout %d", layout);
  if (!a || !b || !m_splits || !c) return fail(GMLP_INVALID_ARG, "null pointer argument");
  if (G < 1 || M < 0 || n <= 0 || k <= 0 || n % 32 || k % 32) return fail(GMLP_UNSUPPORTED, "dims: n, k must be positive multiples of 32");
  // DGRAD is FPROP on the weight's dgrad operand (W^T per expert, blocks along the weight's N)
  const bool fp = layout != GMLP_GEMM_WGRAD;
  if (fp && k % 128) return fail(GMLP_UNSUPPORTED, "dims: the FPROP / DGRAD contraction k must be a multiple of 128");
  if (out_dtype != GMLP_OUT_BF16 && out_dtype != GMLP_OUT_FP32 && out_dtype != GMLP_OUT_FP32_ACCUMULATE)
    return fail(GMLP_INVALID_ARG, "unknown output dtype %d", out_dtype);
  if (out_dtype == GMLP_OUT_FP32_ACCUMULATE && layout != GMLP_GEMM_WGRAD)
    return fail(GMLP_UNSUPPORTED, "accumulating output: WGRAD layout only");
  const GemmOperand oa = fp ? op_row(*a, a->amax_pre) : op_col(*a, a->amax_post);
  const GemmOperand ob = layout == GMLP_GEMM_FPROP ? op_row(*b, b->amax_pre)
                         : layout == GMLP_GEMM_DGRAD ? op_col(*b, b->amax_pre)
                                                     : op_col(*b, b->amax_post);
  {
    const bool nv_a = oa.bf16 || (oa.data && oa.scale), nv_b = ob.bf16 || (ob.data && ob.scale);
    if (is_mx(recipe) ? (!oa.data || !ob.data || !oa.scale_mfma || !ob.scale_mfma)
                      : (!nv_a || !nv_b || !oa.amax || !ob.amax))
      return fail(GMLP_INVALID_ARG, "operand data, scales%s missing", is_mx(recipe) ? "" : " or amax");
    // a packed NVFP4 row-wise operand is expanded 16 rows per workgroup along the grid's y dimension
    if (!is_mx(recipe) && fp && !oa.bf16 && (M + 15) / 16 > 65535)
      return fail(GMLP_UNSUPPORTED, "dims: a packed NVFP4 operand of %lld rows exceeds one expansion launch",
                  (long long)M);
  }
  Bump bb(ws);
  SplitTables T = carve_tables(bb, G);
  const int64_t Pt = M + 127LL * G;
  const NvScratch nv = fp ? carve_nv(bb, recipe, M * k, (int64_t)G * n * k) : carve_nv(bb, recipe, n * Pt, k * Pt);
  if (!ws || ws_bytes < bb.off) return fail(GMLP_WORKSPACE, "workspace too small: need %zu bytes", bb.off);
  Launcher L{stream};
  if (!L.check(launch_scan(m_splits, G, M, T, stream), "scan")) return L.st;
  GemmArgs g = gemm_base(fp ? MODE_FPROP : MODE_WGRAD, recipe, EPI_STORE, T, G);
  set_nv(g, nv);
  g.M = M;
  g.N = n;
  g.K = k;
  g.c = c;
  g.out_fp32 = out_dtype;   // 0 bf16, 1 fp32, 2 fp32 added to c
  g.a = oa;
  g.b = ob;

  if (!L.check(launch_gemm(g, stream), "grouped gemm")) return L.st;
  g_counts[CNT_GEMM]++;
  return ok();
}

gmlp_status gmlp_grouped_mlp_forward(const gmlp_fwd_args* A, hipStream_t stream) {
  memset(g_counts, 0, sizeof(g_counts));
  if (!A) return fail(GMLP_INVALID_ARG, "null args");
  gmlp_status st = mlp_common_checks(A->M, A->E, A->H, A->ffn, A->activation, A->recipe);
  if (st != GMLP_OK) return st;
  if ((A->M > 0 && (!A->x || !A->probs || !A->y)) || !A->m_splits) return fail(GMLP_INVALID_ARG, "null pointer argument");
  if ((st = weight_ok(A->w1, A->recipe, true, false)) != GMLP_OK) return st;
  if ((st = weight_ok(A->w2, A->recipe, true, false)) != GMLP_OK) return st;
  if ((st = check_act(A->activation, A->tanh_clamp_scale)) != GMLP_OK) return st;
  if (A->fc2_amax_in_fc1 &&
      !(A->recipe.kind == GMLP_NVFP4_RHT && (A->activation == GMLP_SRELU || A->activation == GMLP_TANH_SRELU)))
    return fail(GMLP_UNSUPPORTED,
                "%s: the fc2-input amax in the fc1 epilogue needs the NVFP4 recipe and a squared-ReLU activation",
                A->recipe.kind == GMLP_NVFP4_RHT ? "activation" : "recipe");
  const Act act = act_of(A->activation, A->tanh_clamp_scale);
  const bool mx = is_mx(A->recipe);
  const bool wgrad = A->weight_requires_grad != 0;
  const bool rec = A->recompute != 0;
  const int E = A->E;
  const int64_t M = A->M, H = A->H, ffn = A->ffn;
  const gmlp_recipe& r = A->recipe;
  Bump cb(A->ctx);
  FwdCtx C = carve_ctx(cb, M, E, H, ffn, A->activation, r, rec);
  if (!A->ctx || A->ctx_bytes < cb.off) return fail(GMLP_WORKSPACE, "ctx too small: need %zu bytes", cb.off);
  Bump wb(A->ws);
  FwdWs W = carve_fwd_ws(wb, M, E, H, ffn, A->activation, r);
  if (!A->ws || A->ws_bytes < wb.off) return fail(GMLP_WORKSPACE, "workspace too small: need %zu bytes", wb.off);

  Launcher L{stream};
  if (!L.check(launch_scan(A->m_splits, E, M, W.T, stream), "scan")) return L.st;
  g_counts[CNT_SCAN]++;
  const uint16_t* x = static_cast<const uint16_t*>(A->x);

  // 1. group-quantize x: row-wise for fc1, column-wise for the fc1 wgrad
  const float* x_pre = nullptr;
  if (mx) {
    MxOut o{static_cast<uint8_t*>(W.xq_row.q.row_data), nullptr, static_cast<uint32_t*>(W.xq_row.q.row_scale_mfma),
            static_cast<uint8_t*>(C.xq_col.q.col_data), nullptr, static_cast<uint32_t*>(C.xq_col.q.col_scale_mfma)};
    if (!L.check(launch_mxfp8_quant(x, M, H, W.T, E, true, wgrad, o, stream), "mxfp8 quantize x")) return L.st;
    g_counts[CNT_MXQ]++;
  } else {
    float* pre = C.xq_col.q.amax_pre;
    float* post = C.xq_col.q.amax_post;
    if (!L.check(launch_hadamard_amax(x, M, H, W.T, E, r.rht_sign_mask & 0xFFFF, pre, post, stream), "amax x")) return L.st;
    g_counts[CNT_HAMAX]++;
    NvOut o = nv_out(W.xq_row.q, true, false);
    o.col_bf16 = wgrad ? static_cast<uint8_t*>(C.xq_col.q.col_bf16) : nullptr;
    if (!L.check(launch_nvfp4_quant(x, M, H, W.T, E, r.rht_sign_mask & 0xFFFF, true, true, wgrad, pre, post, o, stream),
                 "nvfp4 quantize x"))
      return L.st;
    g_counts[CNT_NVQ]++;
    x_pre = pre;
  }
  // 2. fc1 grouped GEMM: it stores h (saved); the fc2 input a = bf16(act(h) p) is formed from h by
  // the pass that casts it (MXFP8) or by the amax pass and the cast that read it (NVFP4), so a
  // itself is never written.  With fc2_amax_in_fc1 (NVFP4, squared ReLU) the GEMM's epilogue forms
  // a for its tile and takes the fc2 input's pre- and post-RHT amax there ([NV] Changes: the
  // Hadamard-fused fc1 kernel returns both amax values), and no amax pass reads h.
  const bool fused_amax = A->fc2_amax_in_fc1 != 0;
  {
    GemmArgs g = gemm_base(MODE_FPROP, r, fused_amax ? EPI_STORE_AMAX : EPI_STORE, W.T, E);
    g.M = M;
    g.N = f1_of(A->activation, ffn);
    g.K = H;
    g.a = op_row(W.xq_row.q, x_pre);
    g.b = op_row(*A->w1, A->w1->amax_pre);
    g.c = C.h;
    if (fused_amax) {
      g.act = act;
      g.ffn = ffn;
      g.probs = A->probs;
      g.rht_mask = r.rht_sign_mask & 0xFFFF;
      g.amax_pre_out = C.a_pre;
      g.amax_post_out = C.a_post;
    }
    set_nv(g, W.nv);
    if (!L.check(launch_gemm(g, stream), "fc1 gemm")) return L.st;
    g_counts[CNT_GEMM]++;
  }
  // 3. fc2-input cast: row-wise always; column-wise only when the backward will not rebuild it
  const bool a_col = wgrad && !rec;
  const float* a_pre = nullptr;
  if (mx) {
    MxOut o{static_cast<uint8_t*>(W.aq_row.q.row_data), nullptr, static_cast<uint32_t*>(W.aq_row.q.row_scale_mfma),
            a_col ? static_cast<uint8_t*>(C.aq_col.q.col_data) : nullptr, nullptr,
            a_col ? static_cast<uint32_t*>(C.aq_col.q.col_scale_mfma) : nullptr};
    if (!L.check(launch_act_quant(C.h, A->probs, act, ffn, W.T, E, M, o, stream), "fc2 input cast"))
      return L.st;
    g_counts[CNT_MXQ]++;
  } else {
    ActSrc src;
    src.h = C.h;
    src.probs = A->probs;
    src.act = act;
    src.ffn = ffn;
    if (!fused_amax) {
      if (!L.check(launch_hadamard_amax(C.h, M, ffn, W.T, E, r.rht_sign_mask & 0xFFFF, C.a_pre, C.a_post, stream,
                                        src), "amax fc2 input"))
        return L.st;
      g_counts[CNT_HAMAX]++;
    }
    NvOut o = nv_out(W.aq_row.q, true, false);
    o.col_bf16 = a_col ? static_cast<uint8_t*>(C.aq_col.q.col_bf16) : nullptr;
    if (!L.check(launch_nvfp4_quant(C.h, M, ffn, W.T, E, r.rht_sign_mask & 0xFFFF, true, true, a_col, C.a_pre,
                                    C.a_post, o, stream, src), "nvfp4 quantize fc2 input"))
      return L.st;
    g_counts[CNT_NVQ]++;
    a_pre = C.a_pre;
  }
  // 4. fc2 grouped GEMM
  {
    GemmArgs g = gemm_base(MODE_FPROP, r, EPI_STORE, W.T, E);
    g.M = M;
    g.N = H;
    g.K = ffn;
    g.a = op_row(W.aq_row.q, a_pre);
    g.b = op_row(*A->w2, A->w2->amax_pre);
    g.c = A->y;
    set_nv(g, W.nv);
    if (!L.check(launch_gemm(g, stream), "fc2 gemm")) return L.st;
    g_counts[CNT_GEMM]++;
  }
  remember_plan(plan_of(A->ctx, M, E, H, ffn, A->activation, A->tanh_clamp_scale, r, rec, wgrad, 0));
  // the forward's workspace holds no deferred weight-gradient operands any more
  remember_plan(plan_of(A->ws, M, E, H, ffn, A->activation, A->tanh_clamp_scale, r, rec, wgrad, 0));
  return ok();
}

gmlp_status gmlp_forward_saved(const gmlp_fwd_args* A, void** h, float** fc2_amax_pre, float** fc2_amax_post) {
  if (!A || !h || !fc2_amax_pre || !fc2_amax_post) return fail(GMLP_INVALID_ARG, "null pointer argument");
  gmlp_status st = mlp_common_checks(A->M, A->E, A->H, A->ffn, A->activation, A->recipe);
  if (st != GMLP_OK) return st;
  Bump cb(A->ctx);
  FwdCtx C = carve_ctx(cb, A->M, A->E, A->H, A->ffn, A->activation, A->recipe, A->recompute != 0);
  if (!A->ctx || A->ctx_bytes < cb.off) return fail(GMLP_WORKSPACE, "ctx too small: need %zu bytes", cb.off);
  *h = C.h;
  *fc2_amax_pre = C.a_pre;
  *fc2_amax_post = C.a_post;
  return ok();
}

}  // extern "C"

namespace {

gmlp_status check_wgrad_dtype(int32_t d) {
  if (d != GMLP_OUT_BF16 && d != GMLP_OUT_FP32 && d != GMLP_OUT_FP32_ACCUMULATE)
    return fail(GMLP_INVALID_ARG, "unknown wgrad dtype %d", d);
  return GMLP_OK;
}

// fc2 wgrad: dW2_g = Qc(dy_g)^T Qc(a_g), with the fc2 input rebuilt and cast in the backward when
// recomputing (its column-wise cast then lives in the backward's workspace, cast with the saved
// amax), else the forward's column-wise cast in ctx.
bool fc2_wgrad(const gmlp_bwd_args* A, const FwdCtx& C, const BwdWs& W, Launcher& L, hipStream_t stream) {
  const bool rec = A->recompute != 0;
  GemmArgs g = gemm_base(MODE_WGRAD, A->recipe, EPI_STORE, W.T, A->E);
  g.M = A->M;
  g.N = A->H;
  g.K = A->ffn;
  g.a = op_col(W.dyq.q, W.dyq.q.amax_post);
  g.b = rec ? op_col(W.a2q.q, C.a_post) : op_col(C.aq_col.q, C.a_post);
  g.c = A->dw2;
  g.out_fp32 = A->wgrad_dtype;
  set_nv(g, W.nv);
  if (!L.check(launch_gemm(g, stream), "fc2 wgrad gemm")) return false;
  g_counts[CNT_GEMM]++;
  return true;
}

// fc1 wgrad: dW1_g = Qc(dh_g)^T Qc(x_g).
bool fc1_wgrad(const gmlp_bwd_args* A, const FwdCtx& C, const BwdWs& W, Launcher& L, hipStream_t stream) {
  const int64_t F1 = f1_of(A->activation, A->ffn);
  GemmArgs g = gemm_base(MODE_WGRAD, A->recipe, EPI_STORE, W.T, A->E);
  g.M = A->M;
  g.N = F1;
  g.K = A->H;
  g.a = op_col(W.dhq.q, W.dhq.q.amax_post);
  g.b = op_col(C.xq_col.q, C.xq_col.q.amax_post);
  g.c = A->dw1;
  g.out_fp32 = A->wgrad_dtype;
  set_nv(g, W.nv);
  if (!L.check(launch_gemm(g, stream), "fc1 wgrad gemm")) return false;
  g_counts[CNT_GEMM]++;
  return true;
}

}  // namespace

extern "C" {

gmlp_status gmlp_grouped_mlp_backward(const gmlp_bwd_args* A, hipStream_t stream) {
  memset(g_counts, 0, sizeof(g_counts));
  if (!A) return fail(GMLP_INVALID_ARG, "null args");
  gmlp_status st = mlp_common_checks(A->M, A->E, A->H, A->ffn, A->activation, A->recipe);
  if (st != GMLP_OK) return st;
  if ((st = check_act(A->activation, A->tanh_clamp_scale)) != GMLP_OK) return st;
  const bool dgrad = A->input_requires_grad != 0;
  const bool wgrad = A->weight_requires_grad != 0;
  const bool defer = wgrad && A->defer_wgrad != 0;
  if (!A->m_splits || (A->M > 0 && (!A->dy || !A->probs || !A->dprobs)) || (dgrad && A->M > 0 && !A->dx) ||
      (wgrad && !defer && (!A->dw1 || !A->dw2)))
    return fail(GMLP_INVALID_ARG, "null pointer argument");
  if (wgrad && !defer && (st = check_wgrad_dtype(A->wgrad_dtype)) != GMLP_OK) return st;
  if ((st = weight_ok(A->w2, A->recipe, false, true)) != GMLP_OK) return st;
  if (dgrad && (st = weight_ok(A->w1, A->recipe, false, true)) != GMLP_OK) return st;
  const bool mx = is_mx(A->recipe);
  const bool rec = A->recompute != 0;
  const int E = A->E;
  const int64_t M = A->M, H = A->H, ffn = A->ffn;
  const int64_t F1 = f1_of(A->activation, ffn);
  const gmlp_recipe& r = A->recipe;
  const uint32_t mask = r.rht_sign_mask & 0xFFFF;
  Bump cb(const_cast<void*>(A->ctx));
  FwdCtx C = carve_ctx(cb, M, E, H, ffn, A->activation, r, rec);
  if (!A->ctx || A->ctx_bytes < cb.off) return fail(GMLP_WORKSPACE, "ctx too small: need %zu bytes", cb.off);
  Bump wb(A->ws);
  BwdWs W = carve_bwd_ws(wb, M, E, H, ffn, A->activation, r, rec);
  if (!A->ws || A->ws_bytes < wb.off) return fail(GMLP_WORKSPACE, "workspace too small: need %zu bytes", wb.off);
  const SavedPlan plan = plan_of(A->ctx, M, E, H, ffn, A->activation, A->tanh_clamp_scale, r, rec, wgrad, defer);
  if ((st = check_ctx_plan(plan)) != GMLP_OK) return st;

  Launcher L{stream};
  if (!L.check(launch_scan(A->m_splits, E, M, W.T, stream), "scan")) return L.st;
  g_counts[CNT_SCAN]++;

  // quantize a bf16 tensor into q (NVFP4: its own amax pass first)
  auto quant = [&](const uint16_t* t, int64_t K, QBuf& q, bool row, bool col) -> bool {
    if (mx) {
      MxOut o{static_cast<uint8_t*>(q.q.row_data), nullptr, static_cast<uint32_t*>(q.q.row_scale_mfma),
              static_cast<uint8_t*>(q.q.col_data), nullptr, static_cast<uint32_t*>(q.q.col_scale_mfma)};
      if (!L.check(launch_mxfp8_quant(t, M, K, W.T, E, row, col, o, stream), "mxfp8 quantize")) return false;
      g_counts[CNT_MXQ]++;
      return true;
    }
    if (!L.check(launch_hadamard_amax(t, M, K, W.T, E, mask, q.q.amax_pre, q.q.amax_post, stream), "amax")) return false;
    g_counts[CNT_HAMAX]++;
    const NvOut o = nv_out(q.q, row, col);
    if (!L.check(launch_nvfp4_quant(t, M, K, W.T, E, mask, true, row, col, q.q.amax_pre, q.q.amax_post, o, stream),
                 "nvfp4 quantize"))
      return false;
    g_counts[CNT_NVQ]++;
    return true;
  };

  // 1. dy: row-wise for the fc2 dgrad, column-wise for the fc2 wgrad
  if (!quant(static_cast<const uint16_t*>(A->dy), H, W.dyq, true, wgrad)) return L.st;
  // 2-3. MXFP8: fc2 dgrad da = dy W2 (bf16, in the dh buffer), then one pass that forms dh from
  // da and h, casts it row- and column-wise, sums the dL/dp partials and (recomputing) rebuilds
  // and casts the fc2 input.  NVFP4: the dgrad GEMM stores bf16 da, the activation-gradient
  // pass writes bf16 dh (and the rebuilt fc2 input), then dh is cast like any tensor.
  if (mx) {
    uint16_t* da = W.dh;
    GemmArgs g = gemm_base(MODE_FPROP, r, EPI_STORE, W.T, E);
    g.M = M;
    g.N = ffn;
    g.K = H;
    g.a = op_row(W.dyq.q, W.dyq.q.amax_pre);
    g.b = op_col(*A->w2, A->w2->amax_pre);
    g.c = da;
    if (!L.check(launch_gemm(g, stream), "fc2 dgrad gemm")) return L.st;
    g_counts[CNT_GEMM]++;
    DactArgs d{};
    d.da = da;
    d.h = C.h;
    d.probs = A->probs;
    d.act = act_of(A->activation, A->tanh_clamp_scale);
    d.ffn = ffn;
    d.dh = MxOut{dgrad ? static_cast<uint8_t*>(W.dhq.q.row_data) : nullptr, nullptr,
                 dgrad ? static_cast<uint32_t*>(W.dhq.q.row_scale_mfma) : nullptr,
                 wgrad ? static_cast<uint8_t*>(W.dhq.q.col_data) : nullptr, nullptr,
                 wgrad ? static_cast<uint32_t*>(W.dhq.q.col_scale_mfma) : nullptr};
    d.a2 = (rec && wgrad) ? MxOut{nullptr, nullptr, nullptr, static_cast<uint8_t*>(W.a2q.q.col_data), nullptr,
                                  static_cast<uint32_t*>(W.a2q.q.col_scale_mfma)}
                          : MxOut{};
    d.dprob_part = W.dprob_part;
    if (!L.check(launch_dact_quant(d, W.T, E, M, stream), "activation gradient cast")) return L.st;
    g_counts[CNT_MXQ]++;
    if (!L.check(launch_dprob_reduce(W.dprob_part, (int)ceil_div(ffn, 64), M, A->dprobs, stream), "dprob reduce"))
      return L.st;
    g_counts[CNT_DPROB]++;
  }
  const int ntn = dact_ntiles(ffn);
  if (!mx) {
    GemmArgs g = gemm_base(MODE_FPROP, r, EPI_DACT, W.T, E);
    g.M = M;
    g.N = ffn;
    g.K = H;
    g.a = op_row(W.dyq.q, W.dyq.q.amax_pre);
    g.b = op_col(*A->w2, A->w2->amax_pre);
    g.act = act_of(A->activation, A->tanh_clamp_scale);
    g.ffn = ffn;
    g.probs = A->probs;
    g.h = C.h;
    g.a_out = (rec && wgrad) ? W.a2 : nullptr;
    g.dh = W.dh;
    g.dprob_part = W.dprob_part;
    set_nv(g, W.nv);
    g.da_tmp = W.da;
    if (!L.check(launch_gemm(g, stream), "fc2 dgrad gemm")) return L.st;
    g_counts[CNT_GEMM]++;
  }
  if (!mx) {
    if (!L.check(launch_dprob_reduce(W.dprob_part, ntn, M, A->dprobs, stream), "dprob reduce")) return L.st;
    g_counts[CNT_DPROB]++;
    // 3. dh: row-wise for the fc1 dgrad, column-wise for the fc1 wgrad
    if (dgrad || wgrad)
      if (!quant(W.dh, F1, W.dhq, dgrad, wgrad)) return L.st;
  }
  // 4. fc2 wgrad: column-wise dy and fc2 input (rebuilt and cast with the saved amax when
  // recomputing; the MXFP8 rebuild was cast by the activation-gradient pass above).  Deferred:
  // the operands stay in the workspace for gmlp_grouped_mlp_wgrad.
  if (wgrad) {
    if (rec && !mx) {
      const NvOut o = nv_out(W.a2q.q, false, true);
      if (!L.check(launch_nvfp4_quant(W.a2, M, ffn, W.T, E, mask, true, false, true, C.a_pre, C.a_post, o, stream),
                   "nvfp4 quantize rebuilt fc2 input"))
        return L.st;
      g_counts[CNT_NVQ]++;
    }
    if (!defer && !fc2_wgrad(A, C, W, L, stream)) return L.st;
  }
  // 5. fc1 dgrad
  if (dgrad) {
    GemmArgs g = gemm_base(MODE_FPROP, r, EPI_STORE, W.T, E);
    g.M = M;
    g.N = H;
    g.K = F1;
    g.a = op_row(W.dhq.q, W.dhq.q.amax_pre);
    g.b = op_col(*A->w1, A->w1->amax_pre);
    g.c = A->dx;
    set_nv(g, W.nv);
    if (!L.check(launch_gemm(g, stream), "fc1 dgrad gemm")) return L.st;
    g_counts[CNT_GEMM]++;
  }
  // 6. fc1 wgrad
  if (wgrad && !defer && !fc1_wgrad(A, C, W, L, stream)) return L.st;
  SavedPlan ws_plan = plan;
  ws_plan.key = A->ws;
  remember_plan(ws_plan);
  return ok();
}

gmlp_status gmlp_grouped_mlp_wgrad(const gmlp_bwd_args* A, hipStream_t stream) {
  memset(g_counts, 0, sizeof(g_counts));
  if (!A) return fail(GMLP_INVALID_ARG, "null args");
  gmlp_status st = mlp_common_checks(A->M, A->E, A->H, A->ffn, A->activation, A->recipe);
  if (st != GMLP_OK) return st;
  if (!A->weight_requires_grad) return fail(GMLP_INVALID_ARG, "the deferred weight gradients need weight_requires_grad");
  if (!A->m_splits || !A->dw1 || !A->dw2) return fail(GMLP_INVALID_ARG, "null pointer argument");
  if ((st = check_wgrad_dtype(A->wgrad_dtype)) != GMLP_OK) return st;
  Bump cb(const_cast<void*>(A->ctx));
  FwdCtx C = carve_ctx(cb, A->M, A->E, A->H, A->ffn, A->activation, A->recipe, A->recompute != 0);
  if (!A->ctx || A->ctx_bytes < cb.off) return fail(GMLP_WORKSPACE, "ctx too small: need %zu bytes", cb.off);
  Bump wb(A->ws);
  BwdWs W = carve_bwd_ws(wb, A->M, A->E, A->H, A->ffn, A->activation, A->recipe, A->recompute != 0);
  if (!A->ws || A->ws_bytes < wb.off) return fail(GMLP_WORKSPACE, "workspace too small: need %zu bytes", wb.off);
  SavedPlan want = plan_of(A->ctx, A->M, A->E, A->H, A->ffn, A->activation, A->tanh_clamp_scale, A->recipe,
                           A->recompute, 1, 1);
  if ((st = check_ctx_plan(want)) != GMLP_OK) return st;
  {
    // ws: left by a backward with the same settings that deferred its weight gradients
    SavedPlan have;
    want.key = A->ws;
    if (recall_plan(A->ws, &have)) {
      if (const char* f = plan_mismatch(have, want))
        return fail(GMLP_INVALID_ARG, "ws: written by a backward with a different %s", f);
      if (!have.deferred)
        return fail(GMLP_INVALID_ARG, "ws: last written by a call that left no deferred weight-gradient operands");
    }
  }
  Launcher L{stream};
  // the split tables are rebuilt from m_splits: only the operands come from the deferring call
  if (!L.check(launch_scan(A->m_splits, A->E, A->M, W.T, stream), "scan")) return L.st;
  g_counts[CNT_SCAN]++;
  if (!fc2_wgrad(A, C, W, L, stream) || !fc1_wgrad(A, C, W, L, stream)) return L.st;
  return ok();
}

}  // extern "C"
