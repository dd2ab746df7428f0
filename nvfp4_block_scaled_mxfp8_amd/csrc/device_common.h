// Device helpers shared by the gmlp kernels (gfx950 only).
//
// Number formats follow the OCP 8-bit Floating Point spec v1.0 (E4M3) and the
// OCP Microscaling Formats spec v1.0 (E8M0 scales, E2M1 elements); the pages
// name the formats ("GEMM + Swiglu fused Grouped MLP for MXFP8": 32-element
// MXFP8 blocks with E4M3 data and E8M0 scales; "Reduce NVFP4 quantization work
// ...": NVFP4 with E4M3 block scales and a per-group fp32 global scale).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gmlp {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr float kE4M3Max = 448.0f;
constexpr float kE2M1Max = 6.0f;
constexpr float kFltMax = 3.40282346638528859811704183484516925e+38f;

// --------------------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// Round to nearest even (the hardware conversion, v_cvt_pk_bf16_f32; NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}
// Two values at once: lo in bits [0, 16), hi in [16, 32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){lo, hi}, v2bf));
}
__device__ __forceinline__ float round_bf16(float f) { return __uint_as_float(f32_to_bf16_bits(f) << 16); }

// --------------------------------------------------------------------------- E8M0 (MXFP8 scale)
// Scale code of a block with amax a (a is a bf16 value, hence an fp32 normal, subnormal or 0):
// X = clamp(floor(log2 a) - 8, -127, 127), code = X + 127; an all-zero block gets code 127.
// For a normal fp32 a, floor(log2 a) = exponent field - 127, so code = max(field - 8, 0);
// every subnormal a has floor(log2 a) - 8 < -127, so its code is 0.
__device__ __forceinline__ uint32_t e8m0_code(float amax) {
  uint32_t field = __float_as_uint(amax) >> 23;
  if (amax == 0.0f) return 127u;
  return field > 8u ? field - 8u : 0u;
}
// 2^-X for scale code c = X + 127 (c <= 246 for finite bf16 inputs, so the result is a normal fp32).
__device__ __forceinline__ float e8m0_inv_scale(uint32_t code) { return __uint_as_float((254u - code) << 23); }

// --------------------------------------------------------------------------- E4M3 / E2M1 encode
// The gfx950 converters round to nearest even; clamping to the largest finite
// magnitude first gives the saturating (satfinite) encode.  Both were checked
// against an exhaustive round-to-nearest-even reference on every finite bf16
// input times a spread of power-of-two scales.
__device__ __forceinline__ uint32_t cvt_e4m3x2(float a, float b) {
  a = fminf(fmaxf(a, -kE4M3Max), kE4M3Max);
  b = fminf(fmaxf(b, -kE4M3Max), kE4M3Max);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}
// Four values -> four E4M3 bytes (little endian).
__device__ __forceinline__ uint32_t cvt_e4m3x4(float a, float b, float c, float d) {
  return cvt_e4m3x2(a, b) | (cvt_e4m3x2(c, d) << 16);
}
__device__ __forceinline__ uint32_t cvt_e4m3(float a) { return cvt_e4m3x2(a, 0.0f) & 0xFFu; }

// Eight values -> eight E2M1 nibbles packed in a u32 (value 2i in the low nibble of byte i).
__device__ __forceinline__ float clamp_e2m1(float a) { return fminf(fmaxf(a, -kE2M1Max), kE2M1Max); }
__device__ __forceinline__ uint32_t cvt_e2m1x8(const float* v) {
  uint32_t out = 0;
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, clamp_e2m1(v[0]), clamp_e2m1(v[1]), 1.0f, 0);
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, clamp_e2m1(v[2]), clamp_e2m1(v[3]), 1.0f, 1);
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, clamp_e2m1(v[4]), clamp_e2m1(v[5]), 1.0f, 2);
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, clamp_e2m1(v[6]), clamp_e2m1(v[7]), 1.0f, 3);
  return out;
}

// --------------------------------------------------------------------------- decode
// E4M3 code (sign ignored: block scales are non-negative) -> fp32, exact.
__device__ __forceinline__ float e4m3_decode_pos(uint32_t c) {
  uint32_t e = (c >> 3) & 15u, m = c & 7u;
  if (e == 0) return (float)m * 0.001953125f;          // m * 2^-9
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// The two E2M1 values of byte I of w (low nibble first) times sc, as one bf16 pair (the low
// nibble's value in bits [0, 16)).  The hardware converter gives each E2M1 value exactly
// (magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}, the sign from bit 3); a product with an E4M3 block
// scale has at most 6 significant bits, so its bf16 bits are the high half of its fp32 bits.
template <int I>
__device__ __forceinline__ uint32_t e2m1x2_scaled_bf16(uint32_t w, float sc) {
  const v2f p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, I);
  return (__float_as_uint(p.x * sc) >> 16) | (__float_as_uint(p.y * sc) & 0xFFFF0000u);
}

// --------------------------------------------------------------------------- NVFP4 global scale
// S = fp32(2688 / amax), clipped to FLT_MAX; 1 when amax == 0 (2688 = 6 * 448).
__device__ __forceinline__ float nvfp4_global_scale(float amax) {
  if (amax == 0.0f) return 1.0f;
  float s = __fdiv_rn(2688.0f, amax);
  return fminf(s, kFltMax);
}

// --------------------------------------------------------------------------- signed Hadamard
// The NVFP4 recipe's 16x16 randomized Hadamard transform ("Reduce NVFP4 quantization work ...",
// Changes: the quantizer's rht_sign_mask): y = H16 (s * x) with s_j = -1 where bit j of the mask
// is set and H16[i][j] = (-1)^popcount(i & j), as the fp32 butterfly over strides 1, 2, 4, 8
// (each stage maps (v[i], v[i+h]) -> (v[i] + v[i+h], v[i] - v[i+h])); the caller applies the
// exact factor 1/4.  Every pass that transforms or takes the post-transform amax uses this one
// function, so that they agree bit for bit.
__device__ __forceinline__ void signed_fwht16(float* v, uint32_t mask) {
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = ((mask >> j) & 1u) ? -v[j] : v[j];
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i & h) continue;
      const float a = v[i], b = v[i + h];
      v[i] = a + b;
      v[i + h] = a - b;
    }
  }
}

// --------------------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Group lookup: largest g in [0, G) with off[g] <= t (off is an exclusive prefix of length G+1).
__device__ __forceinline__ int find_group(const int32_t* off, int G, int t) {
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace gmlp
