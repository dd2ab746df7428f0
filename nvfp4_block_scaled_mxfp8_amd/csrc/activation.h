// Activations of the grouped MLP and their gradients, shared by the passes that form the fc2
// input from h (forward casts and amax), the activation-gradient passes and the fc2-input
// rebuild of the backward, so that all of them produce the same bits.
//
// Sources: "GEMM + Swiglu fused Grouped MLP for MXFP8" (SwiGLU: silu(gate) * up over the
// [gate | up] halves of the fc1 output, scaled by the token's routing probability);
// "Reduce NVFP4 quantization work for the fused GroupedMLP fc2 input with activation
// recompute" (squared ReLU with the probability scale, and the rebuilt fc2 input).
#pragma once
#include "device_common.h"

namespace gmlp {

// sigmoid(g) = 1 / (1 + 2^(-g log2 e)) on the hardware exp2 and reciprocal (each within about
// one ulp of fp32); fp32 products below are explicitly rounded (no contraction).
__device__ __forceinline__ float sigmoid_f(float g) {
  const float e = __builtin_amdgcn_exp2f(__fmul_rn(-g, 1.4426950408889634f));
  return __builtin_amdgcn_rcpf(__fadd_rn(1.0f, e));
}

__device__ __forceinline__ float act_value(int act, float g, float u) {
  if (act == 0) return __fmul_rn(__fmul_rn(g, sigmoid_f(g)), u);   // silu(gate) * up
  const float r = fmaxf(g, 0.0f);
  return __fmul_rn(r, r);                                            // relu(h)^2
}
// bf16 fc2 input a = act(h) * p
__device__ __forceinline__ float act_out(int act, float g, float u, float p) {
  return round_bf16(__fmul_rn(act_value(act, g, u), p));
}
// d(act * p)/dh for upstream da: d0 = d/dgate (or d/dh), d1 = d/dup; dp = da * act (dL/dp).
__device__ __forceinline__ void act_grad(int act, float g, float u, float da, float p, float& d0, float& d1,
                                         float& dp) {
  if (act == 0) {
    const float sg = sigmoid_f(g);
    const float silu = __fmul_rn(g, sg);
    const float dap = __fmul_rn(da, p);
    const float dsilu = __fmul_rn(sg, __fadd_rn(1.0f, __fmul_rn(g, __fsub_rn(1.0f, sg))));
    d0 = __fmul_rn(__fmul_rn(dap, u), dsilu);
    d1 = __fmul_rn(dap, silu);
    dp = __fmul_rn(da, __fmul_rn(silu, u));
  } else {
    const float r = fmaxf(g, 0.0f);
    d0 = __fmul_rn(__fmul_rn(__fmul_rn(da, p), 2.0f), r);
    d1 = 0.0f;
    dp = __fmul_rn(da, __fmul_rn(r, r));
  }
}
// Both at once (the rebuilt fc2 input next to the gradient): one sigmoid.
__device__ __forceinline__ void act_grad_out(int act, float g, float u, float da, float p, float& d0, float& d1,
                                             float& dp, float& a) {
  if (act == 0) {
    const float sg = sigmoid_f(g);
    const float silu = __fmul_rn(g, sg);
    const float dap = __fmul_rn(da, p);
    const float dsilu = __fmul_rn(sg, __fadd_rn(1.0f, __fmul_rn(g, __fsub_rn(1.0f, sg))));
    const float su = __fmul_rn(silu, u);
    d0 = __fmul_rn(__fmul_rn(dap, u), dsilu);
    d1 = __fmul_rn(dap, silu);
    dp = __fmul_rn(da, su);
    a = round_bf16(__fmul_rn(su, p));
  } else {
    const float r = fmaxf(g, 0.0f);
    const float r2 = __fmul_rn(r, r);
    d0 = __fmul_rn(__fmul_rn(__fmul_rn(da, p), 2.0f), r);
    d1 = 0.0f;
    dp = __fmul_rn(da, r2);
    a = round_bf16(__fmul_rn(r2, p));
  }
}

}  // namespace gmlp
