/*
 * gmlp -- fused MoE grouped MLP with MXFP8 / NVFP4 group quantization on MI355X (gfx950).
 *
 * C ABI of libgmlp.so.  Every entry point is stream-ordered on the caller's
 * hipStream_t, performs no host synchronisation and no device allocation, and
 * dereferences no pointer beyond the call (the MLP calls remember the addresses of
 * their ctx and ws buffers, with the settings they were written with, so that a
 * backward or a deferred wgrad call whose settings differ from those of the call
 * that wrote the buffer fails with GMLP_INVALID_ARG instead of reading it in
 * another layout; a buffer with no record is taken as it is).  All tensors are caller-owned device
 * buffers passed as plain pointers; sizes are host integers.
 *
 * Errors: every argument is validated before anything is enqueued.  On error
 * nothing is enqueued, a status is returned and gmlp_last_error() (thread-local)
 * names the reason.  A failure of the launch itself returns GMLP_HIP_ERROR.
 * Device-side split sizes that do not add up to the host row count M are
 * clamped on the device so that no kernel reads or writes out of bounds; the
 * condition is recorded in the workspace and reported by gmlp_read_device_flags().
 *
 * Sources (the pages this library implements):
 *  [MX]  "GEMM + Swiglu fused Grouped MLP for MXFP8" (TransformerEngine PR 2769):
 *        Greptile summary and sequence diagram.
 *  [NV]  "Reduce NVFP4 quantization work for the fused GroupedMLP fc2 input with
 *        activation recompute" (TransformerEngine PR 3837): Description, Changes,
 *        commit messages.
 *  [FB]  "Add NVTE_CUTEDSL_FUSED_GROUPED_MLP_WARN_FALLBACK ..." (TransformerEngine
 *        PR 3631): Changes (the reasons a grouped MLP cannot be fused).
 *
 * Notation: G groups (experts), group g owns m_g consecutive rows, M = sum m_g.
 * P_g = m_g rounded up to 128.  "row-wise" = blocks along the last dimension;
 * "column-wise" = each group's [m_g, K] slab transposed to [K, P_g] (zero
 * padded) with blocks along tokens; group g's column-wise data starts at element
 * K * sum_{h<g} P_h.
 *
 * MXFP8: 32-element blocks, E4M3 data (round to nearest even, saturating),
 *   E8M0 scale code = clamp(floor(log2 amax) - 8, -127, 127) + 127; an all-zero
 *   block gets code 127.
 * MXFP8 MFMA-ready scales: for a scale matrix [R, nkb] the u32 array
 *   [ceil(nkb/4), R] whose word (t, r) holds blocks 4t..4t+3 of row r in bytes
 *   0..3 (missing blocks = 127).  Column-wise: each group's [K, P_g/32] matrix
 *   converted on its own, at word offset K * sum_{h<g} P_h/128.
 * NVFP4: 16-element blocks, E2M1 data packed two per byte (element 2i in the low
 *   nibble), E4M3 block scales, fp32 global scale S = 2688 / amax per group
 *   (S = 1 if amax = 0; clipped to FLT_MAX).  Row-wise casts use the group's
 *   pre-RHT amax; column-wise casts apply the signed 16x16 Hadamard transform
 *   along tokens and use the post-RHT amax [NV, Changes].
 */
#ifndef GMLP_H
#define GMLP_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GMLP_OK = 0,
  GMLP_INVALID_ARG = 1,   /* a null pointer, a bad size or an inconsistent argument */
  GMLP_UNSUPPORTED = 2,   /* device, recipe, activation or dimensions the library does not handle [FB] */
  GMLP_WORKSPACE = 3,     /* workspace or context buffer smaller than gmlp_query_sizes() reports */
  GMLP_HIP_ERROR = 4      /* a HIP runtime call or kernel launch failed */
} gmlp_status;

typedef enum { GMLP_MXFP8 = 0, GMLP_NVFP4_RHT = 1 } gmlp_recipe_kind;
/* Activation of the fc2 input, scaled by the token's routing probability p:
 *   GMLP_SWIGLU      silu(gate) * up over h = [gate | up] (F1 = 2 ffn)        [MX, sequence diagram]
 *   GMLP_SRELU       relu(h)^2 (F1 = ffn)                                      [NV, Description]
 *   GMLP_TANH_SRELU  c * tanh(relu(h)^2 / c), c = tanh_clamp_scale > 0: the squared ReLU with the tanh
 *                    soft clamp [NV, Changes and commits: ScaledTanhSReLU, tanh_clamp_scale; the pages
 *                    give no formula, this is the library's reading]           (F1 = ffn)
 *   GMLP_QGEGLU      gate * sigmoid(1.702 gate) * up, the GLU with the quick-GELU gate [FB, review: QGeGLU,
 *                    named without a formula; the gate is the sigmoid approximation of GELU from
 *                    Hendrycks and Gimpel, "Gaussian Error Linear Units", section 2] (F1 = 2 ffn) */
typedef enum { GMLP_SWIGLU = 0, GMLP_SRELU = 1, GMLP_TANH_SRELU = 2, GMLP_QGEGLU = 3 } gmlp_activation;
/* Output of a GEMM: bf16 or fp32 (round to nearest even), or fp32 added to what the output
 * buffer holds: C = fp32(C + product), the weight gradient accumulated into a persistent fp32
 * main_grad [MX, review comments on overwrite_main_grad: the grouped wgrad either overwrites
 * main_grad or accumulates into it].  Accumulation
 * is for weight gradients only (WGRAD layout, the backward's dw1 / dw2); an empty expert
 * leaves its slice unchanged. */
typedef enum { GMLP_OUT_BF16 = 0, GMLP_OUT_FP32 = 1, GMLP_OUT_FP32_ACCUMULATE = 2 } gmlp_out_dtype;

/* Recipe [FB, Changes]: MXFP8 (E4M3 data for activations and gradients alike),
 * or NVFP4 with the randomized Hadamard transform (NVFP4 without RHT is not
 * supported).  rht_sign_mask: bit j set = token j of each 16-token block is
 * negated before the Hadamard [NV, Changes]; ignored for MXFP8. */
typedef struct {
  int32_t kind;            /* gmlp_recipe_kind */
  uint32_t rht_sign_mask;  /* low 16 bits used */
} gmlp_recipe;

/* A group-quantized tensor [MX, Greptile summary: flat 1-D data and scale
 * buffers with per-group offsets].  Every pointer is device memory owned by the
 * caller; a pointer the call does not need may be NULL.
 * MXFP8 data is stored in 64-byte K panels (the GEMM stages one panel of 256
 * rows as 16 KB of contiguous memory): for a matrix of R rows and K columns,
 * panel p holds columns [64p, 64p + w), w = min(64, K - 64p), as R rows of w
 * bytes starting at byte 64 p R.  Row-wise data is one such [M, K] matrix;
 * column-wise data is, per group g, the [K, P_g] matrix of the group's columns
 * (tokens along the panel), starting at byte K * sum_{h<g} P_h.
 * NVFP4 data is row-major with two E2M1 codes per byte (low nibble first).
 *   row_data       MXFP8 u8 [M, K] (panels);     NVFP4 u8 [M, K/2]
 *   row_scale      MXFP8 E8M0 u8 [M, K/32];      NVFP4 E4M3 u8 [M, K/16]
 *   row_scale_mfma MXFP8 u32 [ceil(K/128), M]    (unused for NVFP4)
 *   col_data       MXFP8 u8 [K * sum P_g] (panels); NVFP4 u8 [K * sum P_g / 2]
 *   col_scale      MXFP8 u8 [K * sum P_g / 32];  NVFP4 u8 [K * sum P_g / 16]
 *   col_scale_mfma MXFP8 u32 [K * sum P_g/128]
 *   amax_pre, amax_post  NVFP4 fp32 [G] (per-group pre-/post-RHT amax)
 *   row_bf16, col_bf16   NVFP4 only, optional: the same casts as the values
 *                  dec(E2M1) * dec(E4M3) (exact in bf16; the global scale is not
 *                  applied), laid out like MXFP8 data with 2-byte elements: element
 *                  (r, c) of an R x C matrix at byte ((c / 32) R + r) 64 + 2 (c % 32);
 *                  row-wise one [M, K] matrix (2 M K bytes), column-wise group g's
 *                  [K, P_g] at byte 2 K sum_{h<g} P_h.  The NVFP4 GEMMs run on the bf16
 *                  matrix cores: an operand given in this form is read directly,
 *                  otherwise the GEMM expands the packed form into its workspace.
 *                  Written by the quantize calls when non-NULL; either form (or
 *                  both) may be requested. */
typedef struct {
  void* row_data;
  void* row_scale;
  void* row_scale_mfma;
  void* col_data;
  void* col_scale;
  void* col_scale_mfma;
  float* amax_pre;
  float* amax_post;
  void* row_bf16;
  void* col_bf16;
} gmlp_grouped_q;

/* Quantized stacked weights for one GroupedLinear, W [E, N, K] (Linear layout
 * [out, in]) [MX, Greptile summary: stacked and discrete weights].
 *   fprop operand: blocks along K  -> row_data [E][N, K(/2)], row scales
 *   dgrad operand: blocks along N  -> col_data [E][K, N(/2)], col scales (W^T per expert)
 *   MXFP8 data of each expert is one matrix in 64-byte K panels, as above. 
 *   NVFP4: amax [E] (one global scale per expert for both casts; weights get no RHT);
 *   row_bf16 [E][N, K] and col_bf16 [E][K, N] panels (2 N K bytes per expert each),
 *   optional, written once here so that the GEMMs of every step read them directly. */
typedef gmlp_grouped_q gmlp_weight_q;

/* ------------------------------------------------------------------ queries */

/* Thread-local text of the last error (never NULL). */
const char* gmlp_last_error(void);

/* Host-only support check [FB, Changes: system / recipe / activation / dims].
 * arch: a gfx target name such as "gfx950", or NULL to query device 0.
 * Returns GMLP_OK or GMLP_UNSUPPORTED / GMLP_INVALID_ARG with the reason set. */
gmlp_status gmlp_check_support(const char* arch, int32_t experts, int64_t hidden, int64_t ffn,
                               int32_t activation, gmlp_recipe recipe);

/* Sizes (bytes) of the caller-owned buffers for one forward + backward:
 *   ctx_bytes: tensors the forward saves for the backward;
 *   ws_bytes:  scratch of one forward or backward call;
 *   quant_ws_bytes: scratch of the stand-alone quantize calls. */
typedef struct {
  size_t ctx_bytes;
  size_t ws_bytes;
  size_t quant_ws_bytes;
} gmlp_sizes;

gmlp_status gmlp_query_sizes(int64_t M, int32_t experts, int64_t hidden, int64_t ffn,
                             int32_t activation, gmlp_recipe recipe, int32_t recompute,
                             gmlp_sizes* out);

/* Reads (synchronously, on the given stream) the device flag word that kernels
 * set when the device split sizes were clamped (bit 0: negative split, bit 1:
 * splits sum past M, bit 2: splits sum short of M).  Diagnostic only. */
gmlp_status gmlp_read_device_flags(const void* ws, uint32_t* flags, hipStream_t stream);

/* ------------------------------------------------------------------ group quantization */

/* Group quantize a bf16 tensor x [M, K] whose rows are split into G groups by
 * the device int32 array m_splits [G] [MX, sequence diagram: MXFP8 quantize of
 * x and dy; NV, Description: the fc2-input group quantize].
 * MXFP8: one pass, row-wise and/or column-wise.  NVFP4: the Hadamard-amax pass
 * (writes out->amax_pre/post) followed by the cast, as two launches.
 * K % 32 == 0.  ws: >= quant_ws_bytes of gmlp_query_sizes. */
gmlp_status gmlp_group_quantize(const void* x, int64_t M, int64_t K, const int32_t* m_splits,
                                int32_t G, gmlp_recipe recipe, int32_t want_row, int32_t want_col,
                                const gmlp_grouped_q* out, void* ws, size_t ws_bytes,
                                hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): gmlp_group_quantize with no workspace argument.  Its
 * workspace (split tables, NVFP4 amax slots) is a fixed 288 KiB device array of the library, one
 * copy per GPU, held until the process ends; the call allocates nothing.  1 <= G <= 1024, else
 * GMLP_UNSUPPORTED and nothing is enqueued.  Every call rewrites that workspace from scratch
 * (no state carries over between calls); calls that overlap on one GPU (unordered streams)
 * share it and race.  The first call on a device looks up the array's address on that device
 * (hipGetSymbolAddress, with the device current); make it outside graph capture.  Arguments,
 * outputs and errors otherwise as gmlp_group_quantize. */
gmlp_status gmlp_group_quantize_noalloc(const void* x, int64_t M, int64_t K, const int32_t* m_splits,
                                        int32_t G, gmlp_recipe recipe, int32_t want_row, int32_t want_col,
                                        const gmlp_grouped_q* out, hipStream_t stream);

/* Per-group pre-RHT amax (max |x| over the group's rows) and post-RHT amax (max
 * |bf16(H S x)| over every 16-token block of every column of the group, padded
 * with zeros), both in one read of x [NV, Changes: nvfp4_group_hadamard_amax].
 * Outputs fp32 [G]. */
gmlp_status gmlp_group_hadamard_amax(const void* x, int64_t M, int64_t K, const int32_t* m_splits,
                                     int32_t G, uint32_t rht_sign_mask, float* amax_pre,
                                     float* amax_post, void* ws, size_t ws_bytes, hipStream_t stream);

/* NVFP4 cast from given per-group amax (out->amax_pre / amax_post are read, not
 * written) [NV, Changes: nvfp4_group_quantize_with_amax].  Row-wise with the
 * pre-RHT amax, column-wise (with the RHT) with the post-RHT amax. */
gmlp_status gmlp_group_quantize_with_amax(const void* x, int64_t M, int64_t K,
                                          const int32_t* m_splits, int32_t G, gmlp_recipe recipe,
                                          int32_t want_row, int32_t want_col,
                                          const gmlp_grouped_q* out, void* ws, size_t ws_bytes,
                                          hipStream_t stream);

/* Quantize weights W [E, N, K] bf16 for fprop (blocks along K) and dgrad (blocks
 * along N), no RHT.  w: stacked base pointer, or NULL with w_ptrs = a HOST array
 * of E device pointers to the experts' [N, K] matrices (discrete weights) [MX,
 * Greptile summary].  Output in the stacked layout of gmlp_weight_q.  N, K must be
 * multiples of 128.  Scale words are per expert: row_scale_mfma [E][K/128][N],
 * col_scale_mfma [E][N/128][K]. */
gmlp_status gmlp_weight_quantize(const void* w, const void* const* w_ptrs, int32_t E, int64_t N,
                                 int64_t K, gmlp_recipe recipe, const gmlp_weight_q* out,
                                 void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------ grouped GEMM (test / debug export) */

typedef enum {
  GMLP_GEMM_FPROP = 0,  /* C[rows of group g, N] = A_g [m_g, K] . B_g [N, K]^T   (A row-wise, B = weight) */
  GMLP_GEMM_WGRAD = 1,  /* C_g [N_a, N_b] = A_g [N_a, P_g] . B_g [N_b, P_g]^T       (both column-wise)   */
  GMLP_GEMM_DGRAD = 2   /* C[rows of group g, K_w] = A_g [m_g, N_w] . W_g [N_w, K_w] (A row-wise, B = the weight's
                         * dgrad operand b->col_*: FPROP on W^T)                                          */
} gmlp_gemm_layout;

/* One grouped GEMM on already-quantized operands, fp32 accumulation, output
 * bf16 or fp32 (round to nearest even) [MX, sequence diagram: the fc1, fc2,
 * dgrad and wgrad grouped GEMMs].
 * FPROP: a = row-wise quantized [M, K] tensor, b = weight fprop operand
 *        (b->row_*), n = N, k = K; C [M, N].
 * WGRAD: a, b = column-wise quantized tensors with rows N_a = n, N_b = k;
 *        C [G, n, k]; empty groups write zeros (accumulating: leave C_g as it is).
 * DGRAD: a = row-wise quantized [M, k] gradient (k = the weight's N), b = weight whose
 *        dgrad operand (b->col_*, blocks along N) is used, n = the weight's K; C [M, n].
 * out_dtype: gmlp_out_dtype; an unknown value is INVALID_ARG, accumulation with FPROP
 * UNSUPPORTED.
 * ws: >= gmlp_grouped_gemm_ws_bytes for the same arguments. */
/* Workspace bytes of one gmlp_grouped_gemm call with these sizes (host only).  MXFP8 needs
 * only the split tables; NVFP4 also holds both operands expanded exactly to bf16
 * (2 bytes per element of A and of B). */
gmlp_status gmlp_grouped_gemm_ws_bytes(int32_t layout, gmlp_recipe recipe, int32_t G, int64_t M,
                                       int64_t n, int64_t k, size_t* bytes);

gmlp_status gmlp_grouped_gemm(int32_t layout, gmlp_recipe recipe, const gmlp_grouped_q* a,
                              const gmlp_grouped_q* b, const int32_t* m_splits, int32_t G,
                              int64_t M, int64_t n, int64_t k, void* c, int32_t out_dtype,
                              void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------ fused grouped MLP */

/* Forward [MX, sequence diagram; NV, Description and Changes]:
 *   h = bf16(Q(x) Q(W1)^T)   a = bf16(act(h) * prob)   y = bf16(Q(a) Q(W2)^T)
 * act: one of gmlp_activation (F1 = 2 ffn for the gated kinds, ffn otherwise).
 * recompute != 0: the forward casts the fc2 input row-wise only and the
 * backward rebuilds it from h (NVFP4: with the amax saved here).
 * ctx must stay untouched between this call and the matching backward. */
typedef struct {
  const void* x;              /* bf16 [M, H] */
  const int32_t* m_splits;    /* device int32 [E] */
  int64_t M;                  /* host total rows */
  int32_t E;
  int64_t H, ffn;
  const gmlp_weight_q* w1;    /* quantized [E, F1, H] */
  const gmlp_weight_q* w2;    /* quantized [E, H, ffn] */
  const float* probs;         /* fp32 [M] */
  int32_t activation;         /* gmlp_activation */
  gmlp_recipe recipe;
  int32_t recompute;
  int32_t input_requires_grad;
  int32_t weight_requires_grad;
  void* y;                    /* bf16 [M, H] out */
  void* ctx; size_t ctx_bytes;
  void* ws;  size_t ws_bytes;
  int32_t fc2_amax_in_fc1;    /* NVFP4 with a squared-ReLU activation (GMLP_SRELU, GMLP_TANH_SRELU) only (else
                                 GMLP_UNSUPPORTED): != 0 takes the fc2 input's pre- and post-RHT amax in the
                                 fc1 GEMM's epilogue [NV, Changes: the Hadamard-fused fc1 kernel] instead of
                                 a pass over h after it; the same values either way (the separate pass is the
                                 faster one here) */
  float tanh_clamp_scale;     /* GMLP_TANH_SRELU: c > 0 and finite (else GMLP_INVALID_ARG); ignored otherwise */
} gmlp_fwd_args;

/* Backward [MX, sequence diagram; NV, commits]:
 *   da = bf16(Q(dy) Q(W2 along H))        (dh, dprob) = act'(h, da, prob), dh -> bf16
 *   dx = bf16(Q(dh) Q(W1 along F1))       dW2_g = Q_c(dy_g)^T Q_c(a_g)   dW1_g = Q_c(dh_g)^T Q_c(x_g)
 * dprobs[m] = sum_f da[m,f] act(h)[m,f], summed in a fixed order. */
typedef struct {
  const void* dy;             /* bf16 [M, H] */
  const int32_t* m_splits;
  int64_t M;
  int32_t E;
  int64_t H, ffn;
  const gmlp_weight_q* w1;    /* uses the dgrad operand (col_*) */
  const gmlp_weight_q* w2;
  const float* probs;
  int32_t activation;
  gmlp_recipe recipe;
  int32_t recompute;          /* must match the forward (checked, as are the sizes, activation and recipe) */
  int32_t input_requires_grad;
  int32_t weight_requires_grad;
  void* dx;                   /* bf16 [M, H] (may be NULL if !input_requires_grad) */
  float* dprobs;              /* fp32 [M] */
  void* dw1;                  /* [E, F1, H] in wgrad_dtype (NULL if !weight_requires_grad) */
  void* dw2;                  /* [E, H, ffn] */
  int32_t wgrad_dtype;        /* gmlp_out_dtype; FP32_ACCUMULATE: dw1, dw2 are fp32 main_grads, added to */
  const void* ctx; size_t ctx_bytes;
  void* ws; size_t ws_bytes;
  int32_t defer_wgrad;        /* != 0 (with weight_requires_grad): cast the weight-gradient operands into
                                 ws but leave dw1, dw2 to a later gmlp_grouped_mlp_wgrad */
  float tanh_clamp_scale;     /* GMLP_TANH_SRELU: the forward's c (else GMLP_INVALID_ARG); ignored otherwise */
} gmlp_bwd_args;

gmlp_status gmlp_grouped_mlp_forward(const gmlp_fwd_args* args, hipStream_t stream);

/* Device addresses, inside a forward's ctx, of two things it saves for the backward: h [M, F1]
 * bf16 (the fc1 output, the bf16 pre-activation of [MX, sequence diagram]) and, for NVFP4, the
 * fc2 input's per-group pre- and post-RHT amax (fp32 [E] each; the forward keeps them for the
 * recompute cast [NV, Changes]; NULL for MXFP8), whether the forward took them in a pass over h
 * or in the fc1 GEMM's epilogue (fc2_amax_in_fc1).  args: the forward's M, E, H, ffn, activation,
 * recipe, recompute, ctx and ctx_bytes (nothing else is read).  Host only: computes addresses,
 * enqueues nothing. */
gmlp_status gmlp_forward_saved(const gmlp_fwd_args* args, void** h, float** fc2_amax_pre, float** fc2_amax_post);
gmlp_status gmlp_grouped_mlp_backward(const gmlp_bwd_args* args, hipStream_t stream);

/* Deferred weight gradients [MX, Greptile summary, Important Files Changed: the grouped linear
 * op's delay_wgrad hooks]:
 * dW2_g and dW1_g from the operands a backward with defer_wgrad != 0 left in ws (and the
 * forward's ctx).  args: the same sizes, recipe, activation, recompute, m_splits, ctx and ws as
 * that backward, with dw1, dw2 and wgrad_dtype for this call (dy, dx, dprobs, w1, w2 are not
 * read).  Stream-ordered after that backward; ctx and ws must be untouched in between,
 * otherwise the gradients are unspecified (the split tables are rebuilt from m_splits, so
 * every address stays inside the buffers).  May be called once or several times (e.g.
 * accumulating into main_grad). */
gmlp_status gmlp_grouped_mlp_wgrad(const gmlp_bwd_args* args, hipStream_t stream);

/* Launch counts of the last forward / backward on this thread, by kernel kind
 * (0 scan, 1 mxfp8 quantize, 2 hadamard amax, 3 nvfp4 cast, 4 gemm, 5 dprob
 * reduce, 6 fill).  Lets a test check that a recompute backward issues no
 * second Hadamard-amax pass [NV, Description]. */
gmlp_status gmlp_last_launch_counts(int32_t* counts, int32_t n);

#ifdef __cplusplus
}
#endif
#endif /* GMLP_H */
