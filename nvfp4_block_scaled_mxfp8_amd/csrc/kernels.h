// Private interface between the host planner (api.cpp) and the kernel files.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace gmlp {

// Activation of the fc2 input: kind (0 SwiGLU, 1 squared ReLU, 2 tanh-clamped squared ReLU,
// 3 QGeGLU; the C ABI's gmlp_activation) and the clamp scale c of kind 2.
struct Act {
  int kind = 0;
  float c = 0.0f;
};

// Per-call split tables, computed on the device from m_splits (all int32, length G+1,
// exclusive prefix sums; row counts clamped so that row_off[G] <= M).
struct SplitTables {
  uint32_t* flags;     // bit 0 negative split, bit 1 sum past M, bit 2 sum short of M
  int32_t* row_off;    // rows
  int32_t* col_off;    // P_g = m_g rounded up to 128 (column-wise layout)
  int32_t* colw_off;   // P_g / 128 (MFMA-ready column-wise scale words)
  int32_t* t128_off;   // ceil(m_g / 128)  (128-row tiles)
  int32_t* t256_off;   // ceil(m_g / 256)  (256-row tiles)
  // NVFP4 amax partials [2 (pre, post)][G][kAmaxSlots] (non-negative floats as bits): the scan
  // clears them, the Hadamard-amax kernel maxes into them (a workgroup picks one slot, so that
  // few atomics meet on one address), and its finalize pass reduces and clears them again.
  uint32_t* amax_slots;
};
constexpr int kAmaxSlots = 32;

struct MxOut {
  uint8_t* row_data;
  uint8_t* row_scale;
  uint32_t* row_scale_mfma;
  uint8_t* col_data;
  uint8_t* col_scale;
  uint32_t* col_scale_mfma;
};

// Fused activation gradient + MXFP8 cast (backward, between the fc2 dgrad and the fc1 GEMMs).
struct DactArgs {
  const uint16_t* da;   // [M, ffn] bf16: dy W2
  const uint16_t* h;    // [M, F1] bf16: fc1 output ([gate | up] for SwiGLU)
  const float* probs;   // [M]
  Act act;
  int64_t ffn;
  MxOut dh;             // MXFP8 dh [M, F1], row- and/or column-wise (null pointers: not written)
  MxOut a2;             // column-wise MXFP8 of the rebuilt fc2 input [M, ffn], or all null
  float* dprob_part;    // [ffn / 64][M]
};

// NVFP4 cast outputs; any null pointer is not written.  row_bf16 / col_bf16: the quantized
// values dec(E2M1) dec(E4M3) (exact in bf16, no global scale) in the GEMMs' 64-byte panels:
// row-wise element (r, k) at byte ((k / 32) M + r) 64 + 2 (k % 32); column-wise group g's
// element (f, t) at 2 K col_off[g] + ((t / 32) K + f) 64 + 2 (t % 32).
struct NvOut {
  uint8_t* row_data;
  uint8_t* row_scale;
  uint8_t* col_data;
  uint8_t* col_scale;
  uint8_t* row_bf16 = nullptr;
  uint8_t* col_bf16 = nullptr;
};

hipError_t launch_scan(const int32_t* m_splits, int G, int64_t M, SplitTables T, hipStream_t s);
hipError_t launch_fill_u32(uint32_t* p, uint32_t v, int64_t n, hipStream_t s);
hipError_t launch_mxfp8_quant(const uint16_t* x, int64_t M, int64_t K, SplitTables T, int G,
                              bool row, bool col, MxOut o, hipStream_t s);
hipError_t launch_dact_quant(const DactArgs& d, SplitTables T, int G, int64_t M, hipStream_t s);
// MXFP8 forward: the fc2 input a = bf16(act(h) p) from the fc1 output h [M, F1], cast row-wise
// (and column-wise when o.col_data is set) without writing a.
hipError_t launch_act_quant(const uint16_t* h, const float* probs, Act act, int64_t ffn, SplitTables T, int G,
                            int64_t M, MxOut o, hipStream_t s);
// The input of an NVFP4 amax pass or cast: x itself (h == nullptr) or the fc2 input
// a = bf16(act(h) p) [M, ffn], formed on the fly from the fc1 output h [M, F1] (F1 = 2 ffn for
// SwiGLU: gate | up) with the same function as the backward's rebuild.
struct ActSrc {
  const uint16_t* h = nullptr;
  const float* probs = nullptr;
  Act act;
  int64_t ffn = 0;
};
hipError_t launch_hadamard_amax(const uint16_t* x, int64_t M, int64_t K, SplitTables T, int G,
                                uint32_t mask, float* pre, float* post, hipStream_t s, ActSrc act = ActSrc());
// pre[g] / post[g] = the max over group g's amax slots (T.amax_slots), which it clears again.
hipError_t launch_amax_finalize(SplitTables T, int G, float* pre, float* post, hipStream_t s);
hipError_t launch_nvfp4_quant(const uint16_t* x, int64_t M, int64_t K, SplitTables T, int G,
                              uint32_t mask, bool rht, bool row, bool col, const float* pre,
                              const float* post, NvOut o, hipStream_t s, ActSrc act = ActSrc());
// Per-expert amax of stacked weights [E, N, K] (one group per expert, no transform).
hipError_t launch_weight_amax(const uint16_t* w, const void* const* w_ptrs, int E, int64_t N,
                              int64_t K, float* amax, hipStream_t s);
// Copies discrete expert weights into a stacked bf16 buffer.
hipError_t launch_gather_weights(const void* const* w_ptrs, int E, int64_t N, int64_t K,
                                 uint16_t* out, hipStream_t s);

// NVFP4 operands expanded exactly to bf16 in 64-byte K panels (element (r, c) of an R x C matrix
// at byte ((c / 32) R + r) 64 + 2 (c % 32)): nmat stacked [R, C] matrices, or the column-wise
// groups [R, P_g] at element offsets R col_off[g] (cols_bound >= col_off[G]).
hipError_t launch_nv_expand(const uint8_t* data, const uint8_t* scale, uint8_t* out, int64_t R, int64_t C,
                            int nmat, hipStream_t s);
hipError_t launch_nv_expand_groups(const uint8_t* data, const uint8_t* scale, uint8_t* out, int64_t R,
                                   int64_t cols_bound, const int32_t* col_off, int G, hipStream_t s);
// NVFP4 backward: bf16 dh (and the rebuilt fc2 input a2 when non-null) from bf16 da and h, with
// the dL/dp partials of each 256-feature tile in dprob_part [ceil(ffn / 256)][M].
hipError_t launch_dact_bf16(const uint16_t* da, const uint16_t* h, const float* probs, Act act, int64_t ffn,
                            int64_t M, uint16_t* dh, uint16_t* a2, float* dprob_part, hipStream_t s);

// ----------------------------------------------------------------------------- GEMM
// FMT_NVFP4_BF16: NVFP4 operands expanded exactly to bf16 (dec(E2M1) dec(E4M3), no global scale) in
// the 64-byte panel layout of the MXFP8 operands, with the per-group amax for the global scales.
enum GemmFmt { FMT_MXFP8 = 0, FMT_NVFP4 = 1, FMT_NVFP4_BF16 = 2 };
enum GemmMode { MODE_FPROP = 0, MODE_WGRAD = 1 };
// STORE32: fp32 output.  ACC32: fp32 output added to what C holds (weight gradients into an fp32
// main_grad).  DACT (NVFP4 fc2 dgrad): da is stored, then the activation-gradient pass.
// STORE_AMAX (NVFP4 fc1 with squared ReLU): h is stored as by STORE, and the epilogue also forms
// the fc2 input a = bf16(relu(h)^2 p) of its tile and maxes the tile's pre- and post-RHT amax of a
// into the group's amax slots; a finalize pass after the GEMM writes amax_pre_out / amax_post_out.
enum GemmEpi { EPI_STORE = 0, EPI_DACT = 2, EPI_STORE32 = 3, EPI_ACC32 = 4, EPI_STORE_AMAX = 5 };

struct GemmOperand {
  const uint8_t* data;        // fp8 / packed fp4
  const uint32_t* scale_mfma; // MXFP8: MFMA-ready words
  const uint8_t* scale;       // NVFP4: E4M3 block scales (canonical)
  const float* amax;          // NVFP4: per-group (or per-expert) amax for the global scale
  const uint8_t* bf16 = nullptr;  // NVFP4: the operand already expanded to bf16 panels (else expanded here)
};

struct GemmArgs {
  int mode, fmt, epi;
  GemmOperand a, b;
  SplitTables T;
  int G;
  int64_t M;         // FPROP: total rows of A
  int64_t N;         // FPROP: output columns (B rows per expert); WGRAD: rows of A per group
  int64_t K;         // FPROP: contraction; WGRAD: rows of B per group
  // outputs
  void* c;           // EPI_STORE: C (bf16 or fp32)
  int out_fp32;      // 0 bf16, 1 fp32, 2 fp32 added to C (WGRAD)
  // EPI_DACT (NVFP4 fc2 dgrad): operands of the activation-gradient pass run after the GEMM
  Act act;
  int64_t ffn;       // EPI_DACT: ffn (width of da and a'); gated kinds F1 = 2 ffn
  const float* probs;
  uint16_t* h;       // EPI_DACT: in h [M, F1]
  uint16_t* a_out;   // EPI_DACT: out a' (recompute) or null
  uint16_t* dh;      // EPI_DACT: out dh [M, F1]
  float* dprob_part; // EPI_DACT: [n_tiles, M]
  int group_rows;    // tile rows per launch-order group (see tile_ctx); set by the launcher
  int expert_groups; // FPROP: 1 when the launch-order groups stay inside one expert; set by the launcher
  // NVFP4: scratch for the operands expanded to bf16 (A: 2 x rows x contraction bytes, B: the
  // same for the weight or column-wise operand) and, for EPI_DACT, da [M, ffn] bf16
  uint8_t* xa;
  uint8_t* xb;
  uint16_t* da_tmp;
  // EPI_STORE_AMAX: the recipe's sign mask (probs above) and the per-group fc2-input amax outputs
  uint32_t rht_mask;
  float* amax_pre_out;
  float* amax_post_out;
};

hipError_t launch_gemm(const GemmArgs& g, hipStream_t s);
int gemm_fprop_ntiles_n(const GemmArgs& g);   // N tiles of an FPROP launch (dprob partial count)
hipError_t launch_dprob_reduce(const float* part, int nparts, int64_t M, float* out, hipStream_t s);

}  // namespace gmlp
