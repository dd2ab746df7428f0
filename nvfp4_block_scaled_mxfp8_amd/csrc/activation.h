// Activations of the grouped MLP and their gradients, shared by the passes that form the fc2
// input from h (forward casts and amax), the activation-gradient passes and the fc2-input
// rebuild of the backward, so that all of them produce the same bits.
//
// Sources: "GEMM + Swiglu fused Grouped MLP for MXFP8" (SwiGLU: silu(gate) * up over the
// [gate | up] halves of the fc1 output, scaled by the token's routing probability);
// "Reduce NVFP4 quantization work for the fused GroupedMLP fc2 input with activation
// recompute" (squared ReLU with the probability scale, the rebuilt fc2 input, and the
// tanh soft clamp of the squared ReLU with its tanh_clamp_scale: Changes and commits);
// "Add NVTE_CUTEDSL_FUSED_GROUPED_MLP_WARN_FALLBACK ..." (review: the QGeGLU activation).
// The pages name the last two without formulas; the forms below are this library's readings:
//   tanh-clamped squared ReLU: c tanh(relu(h)^2 / c), a soft clamp of relu(h)^2 to (0, c);
//   QGeGLU: the GLU with the quick GELU gate g sigmoid(1.702 g) (Hendrycks and Gimpel,
//   "Gaussian Error Linear Units", section 2: the sigmoid approximation of GELU) times up.
#pragma once
#include "device_common.h"
#include "kernels.h"

namespace gmlp {

// Activation kinds (the C ABI's gmlp_activation values).
enum ActKind { ACT_SWIGLU = 0, ACT_SRELU = 1, ACT_TANH_SRELU = 2, ACT_QGEGLU = 3 };
constexpr float kQuickGeluK = 1.702f;

// Gated kinds read h = [gate | up] (F1 = 2 ffn).
__host__ __device__ constexpr bool act_is_glu(int kind) { return kind == ACT_SWIGLU || kind == ACT_QGEGLU; }

// sigmoid(g) = 1 / (1 + 2^(-g log2 e)) on the hardware exp2 and reciprocal (each within about
// one ulp of fp32); fp32 products below are explicitly rounded (no contraction).
__device__ __forceinline__ float sigmoid_f(float g) {
  const float e = __builtin_amdgcn_exp2f(__fmul_rn(-g, 1.4426950408889634f));
  return __builtin_amdgcn_rcpf(__fadd_rn(1.0f, e));
}

// Gated kinds: the gate's value gs = g s(g) and its derivative (SwiGLU: s = sigmoid(g);
// QGeGLU: s = sigmoid(k g), d/dg [g s(k g)] = s (1 + k g (1 - s))).
template <int KIND>
__device__ __forceinline__ void gate_fn(float g, float& gs, float& dgs) {
  const float kg = KIND == ACT_QGEGLU ? __fmul_rn(kQuickGeluK, g) : g;
  const float sg = sigmoid_f(kg);
  gs = __fmul_rn(g, sg);
  dgs = __fmul_rn(sg, __fadd_rn(1.0f, __fmul_rn(kg, __fsub_rn(1.0f, sg))));
}
// Squared-ReLU kinds: the value of s = relu(h)^2 after the kind's clamp, and the factor that
// multiplies d(relu(h)^2)/dh = 2 relu(h) in its derivative.
template <int KIND>
__device__ __forceinline__ void srelu_fn(float r2, float c, float& v, float& dv) {
  if constexpr (KIND == ACT_TANH_SRELU) {
    const float t = tanhf(__fdiv_rn(r2, c));
    v = __fmul_rn(c, t);
    dv = __fmul_rn(__fsub_rn(1.0f, t), __fadd_rn(1.0f, t));    // 1 - t^2
  } else {
    v = r2;
    dv = 1.0f;
  }
}

template <int KIND>
__device__ __forceinline__ float act_value(float g, float u, float c) {
  if constexpr (act_is_glu(KIND)) {
    float gs, dgs;
    gate_fn<KIND>(g, gs, dgs);
    return __fmul_rn(gs, u);
  } else {
    const float r = fmaxf(g, 0.0f);
    float v, dv;
    srelu_fn<KIND>(__fmul_rn(r, r), c, v, dv);
    return v;
  }
}
// bf16 fc2 input a = act(h) * p
template <int KIND>
__device__ __forceinline__ float act_out(float g, float u, float p, float c) {
  return round_bf16(__fmul_rn(act_value<KIND>(g, u, c), p));
}
// d(act * p)/dh for upstream da: d0 = d/dgate (or d/dh), d1 = d/dup; dp = da * act (dL/dp); with
// the rebuilt fc2 input a = bf16(act p) next to them.
template <int KIND>
__device__ __forceinline__ void act_grad_out(float g, float u, float da, float p, float c, float& d0, float& d1,
                                             float& dp, float& a) {
  const float dap = __fmul_rn(da, p);
  if constexpr (act_is_glu(KIND)) {
    float gs, dgs;
    gate_fn<KIND>(g, gs, dgs);
    const float v = __fmul_rn(gs, u);
    d0 = __fmul_rn(__fmul_rn(dap, u), dgs);
    d1 = __fmul_rn(dap, gs);
    dp = __fmul_rn(da, v);
    a = round_bf16(__fmul_rn(v, p));
  } else {
    const float r = fmaxf(g, 0.0f);
    float v, dv;
    srelu_fn<KIND>(__fmul_rn(r, r), c, v, dv);
    d0 = KIND == ACT_TANH_SRELU ? __fmul_rn(__fmul_rn(__fmul_rn(dap, dv), 2.0f), r)
                                : __fmul_rn(__fmul_rn(dap, 2.0f), r);
    d1 = 0.0f;
    dp = __fmul_rn(da, v);
    a = round_bf16(__fmul_rn(v, p));
  }
}
template <int KIND>
__device__ __forceinline__ void act_grad(float g, float u, float da, float p, float c, float& d0, float& d1,
                                         float& dp) {
  float a;
  act_grad_out<KIND>(g, u, da, p, c, d0, d1, dp, a);
}

// Runtime-kind forms for the passes that take the activation as an argument (one uniform
// branch per call).
__device__ __forceinline__ float act_out_rt(const Act& A, float g, float u, float p) {
  switch (A.kind) {
    case ACT_SWIGLU: return act_out<ACT_SWIGLU>(g, u, p, A.c);
    case ACT_SRELU: return act_out<ACT_SRELU>(g, u, p, A.c);
    case ACT_TANH_SRELU: return act_out<ACT_TANH_SRELU>(g, u, p, A.c);
    default: return act_out<ACT_QGEGLU>(g, u, p, A.c);
  }
}
__device__ __forceinline__ void act_grad_out_rt(const Act& A, float g, float u, float da, float p, float& d0,
                                                float& d1, float& dp, float& a) {
  switch (A.kind) {
    case ACT_SWIGLU: act_grad_out<ACT_SWIGLU>(g, u, da, p, A.c, d0, d1, dp, a); break;
    case ACT_SRELU: act_grad_out<ACT_SRELU>(g, u, da, p, A.c, d0, d1, dp, a); break;
    case ACT_TANH_SRELU: act_grad_out<ACT_TANH_SRELU>(g, u, da, p, A.c, d0, d1, dp, a); break;
    default: act_grad_out<ACT_QGEGLU>(g, u, da, p, A.c, d0, d1, dp, a); break;
  }
}

}  // namespace gmlp
