// Group quantization kernels: split scan, MXFP8 row/column cast, NVFP4 Hadamard amax and cast.
//
// Sources: "GEMM + Swiglu fused Grouped MLP for MXFP8" (sequence diagram: MXFP8
// row-wise data for the GEMMs, column-wise data for wgrad); "Reduce NVFP4
// quantization work for the fused GroupedMLP fc2 input with activation
// recompute" (Changes: nvfp4_group_hadamard_amax returns the per-group pre- and
// post-RHT amax in one pass; nvfp4_group_quantize_with_amax casts from given
// amax; the RHT carries the quantizer's sign mask).
//
// Tiling: the split tables count 128-token tiles per group; tiles never straddle
// groups, so every 32-token (MXFP8) or 16-token (NVFP4) column block starts at a
// group-relative multiple of its size.  The casts run one 256-thread workgroup per
// 64-token half of such a tile and 128 features (64 for the activation passes), so
// 17 KB of LDS keeps eight workgroups per CU in flight; the NVFP4 amax pass keeps
// whole 128-token tiles, which measured faster for it.
// Each load instruction of a wave reads four whole 256-byte row segments (16 lanes
// per row, 8 bf16 each); the values are cast row-wise in registers (a block spans a
// lane pair or quad) and parked in LDS, from where the column pass reads one feature
// column per lane.
#include "activation.h"
#include "device_common.h"
#include "kernels.h"

#include <type_traits>

namespace gmlp {

constexpr int QT = 128;          // tokens per tile
constexpr int QF = 128;          // features per tile
constexpr int LDW = QF + 8;      // LDS row stride (bf16): +16 bytes keeps the 16-byte writes conflict-free

// Parked MXFP8 tiles: element (token r, feature c) at r LDW + (c ^ 32 ((r / 16) % 4)).  The
// column pass reads 16-token runs of 16 features with four runs 16 tokens apart in one
// instruction; 16 rows are a whole number of bank lines, so without the XOR the four runs
// would share banks.  The XOR moves them to four different 64-byte windows and keeps every
// 8-feature group (one 16-byte store) contiguous.
__device__ __forceinline__ int tile_off(int r, int c) { return r * LDW + (c ^ (((r >> 4) & 3) << 5)); }

// ----------------------------------------------------------------------------- split scan
__global__ __launch_bounds__(256) void scan_kernel(const int32_t* __restrict__ m_splits, int G, int64_t M,
                                                   SplitTables T) {
  __shared__ long long s_rows[256];
  __shared__ int s_d[4][256];
  __shared__ long long carry_raw;
  __shared__ int carry[5];
  __shared__ uint32_t s_flags;
  const int t = threadIdx.x;
  if (t == 0) {
    carry_raw = 0;
    s_flags = 0;
    for (int i = 0; i < 5; ++i) carry[i] = 0;
    T.row_off[0] = T.col_off[0] = T.colw_off[0] = T.t128_off[0] = T.t256_off[0] = 0;
  }
  uint32_t flags = 0;
  for (int i = t; i < 2 * G * kAmaxSlots; i += 256) T.amax_slots[i] = 0u;
  __syncthreads();
  for (int base = 0; base < G; base += 256) {
    const int g = base + t;
    long long m = (g < G) ? (long long)m_splits[g] : 0;
    if (m < 0) { flags |= 1u; m = 0; }
    // inclusive scan of the raw counts
    s_rows[t] = m;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
      long long v = (t >= o) ? s_rows[t - o] : 0;
      __syncthreads();
      s_rows[t] += v;
      __syncthreads();
    }
    const long long incl = carry_raw + s_rows[t];
    const long long start = min(incl - m, (long long)M);
    const long long end = min(incl, (long long)M);
    const int mc = (int)(end - start);
    if (g < G) T.row_off[g + 1] = (int)end;
    const int p = (mc + 127) & ~127;
    int d[4] = {p, (p + 127) / 128, (mc + 127) / 128, (mc + 255) / 256};
    for (int i = 0; i < 4; ++i) s_d[i][t] = d[i];
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
      int v[4];
      for (int i = 0; i < 4; ++i) v[i] = (t >= o) ? s_d[i][t - o] : 0;
      __syncthreads();
      for (int i = 0; i < 4; ++i) s_d[i][t] += v[i];
      __syncthreads();
    }
    if (g < G) {
      T.col_off[g + 1] = carry[1] + s_d[0][t];
      T.colw_off[g + 1] = carry[2] + s_d[1][t];
      T.t128_off[g + 1] = carry[3] + s_d[2][t];
      T.t256_off[g + 1] = carry[4] + s_d[3][t];
    }
    __syncthreads();
    if (t == 255) {
      carry_raw = incl;
      for (int i = 0; i < 4; ++i) carry[i + 1] += s_d[i][255];
    }
    __syncthreads();
  }
  if (t == 0) {
    if (carry_raw > M) flags |= 2u;
    if (carry_raw < M) flags |= 4u;
  }
  if (flags) atomicOr(&s_flags, flags);
  __syncthreads();
  if (t == 0) *T.flags = s_flags;        // the whole word: no clearing launch needed before the scan
}

__global__ void fill_u32_kernel(uint32_t* p, uint32_t v, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = v;
}

// ----------------------------------------------------------------------------- tile bookkeeping
struct TileInfo {
  int g;          // group
  int64_t gstart; // first row of the group
  int m;          // rows of the group
  int t0;         // first group-relative token of the tile
  int rows;       // valid rows in the tile
  int64_t k0;     // first feature of the tile
  int kcols;      // valid features in the tile (multiple of 32)
};

__device__ __forceinline__ bool tile_info(const SplitTables& T, int G, int64_t K, TileInfo& ti) {
  const int tt = blockIdx.y;
  if (G <= 0 || tt >= T.t128_off[G]) return false;
  ti.g = find_group(T.t128_off, G, tt);
  ti.gstart = T.row_off[ti.g];
  ti.m = T.row_off[ti.g + 1] - (int)ti.gstart;
  ti.t0 = (tt - T.t128_off[ti.g]) * QT;
  ti.rows = min(QT, ti.m - ti.t0);
  ti.k0 = (int64_t)blockIdx.x * QF;
  ti.kcols = (int)min((int64_t)QF, K - ti.k0);
  return ti.rows > 0;
}

__device__ __forceinline__ void unpack8(const uint4& q, float* v);

// 8 bf16 of rows row[i], features k .. k + 7, of an NVFP4 pass's input (zeros where !ok[i]):
// x itself, or the fc2 input a = bf16(act(h) p) formed from the fc1 output with the same
// function as every other producer of a, so the bits agree.  Every read is issued before any
// activation, so that the reads of the N rows are in flight together.
template <int KIND, int N>
__device__ __forceinline__ void load_act8(const ActSrc& A, const int64_t (&row)[N], const bool (&ok)[N], int64_t k,
                                          uint4 (&q)[N]) {
  constexpr bool GLU = act_is_glu(KIND);
  const int64_t F1 = GLU ? 2 * A.ffn : A.ffn;
  uint4 gq[N], uq[N];
  float p[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const uint16_t* h = A.h + row[i] * F1 + k;
    gq[i] = ok[i] ? *reinterpret_cast<const uint4*>(h) : make_uint4(0, 0, 0, 0);
    uq[i] = (GLU && ok[i]) ? *reinterpret_cast<const uint4*>(h + A.ffn) : make_uint4(0, 0, 0, 0);
    p[i] = ok[i] ? A.probs[row[i]] : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < N; ++i) {
    float g[8], u[8];
    unpack8(gq[i], g);
    unpack8(uq[i], u);
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = act_out<KIND>(g[2 * j], u[2 * j], p[i], A.act.c);
      const float hi = act_out<KIND>(g[2 * j + 1], u[2 * j + 1], p[i], A.act.c);
      w[j] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
    }
    q[i] = ok[i] ? make_uint4(w[0], w[1], w[2], w[3]) : make_uint4(0, 0, 0, 0);
  }
}
// IN: the input the pass reads, fixed per kernel instantiation so that each keeps its own register
// budget: kInX for x itself, else the activation kind of the fc2 input formed from h.
constexpr int kInX = -1;
template <int IN, int N>
__device__ __forceinline__ void load_in8(const uint16_t* __restrict__ x, int64_t K, const ActSrc& A,
                                         const int64_t (&row)[N], const bool (&ok)[N], int64_t k, uint4 (&q)[N]) {
  if constexpr (IN == kInX) {
#pragma unroll
    for (int i = 0; i < N; ++i) q[i] = ok[i] ? *reinterpret_cast<const uint4*>(x + row[i] * K + k) : make_uint4(0, 0, 0, 0);
  } else {
    load_act8<IN, N>(A, row, ok, k, q);
  }
}
// The input kind of a pass: kInX, or the activation kind when it reads h.
inline int input_kind(const ActSrc& A) { return A.h ? A.act.kind : kInX; }

// Load i of a thread covers tile row r = 32 wave + 4 i + lane / 16 and features 8 (lane % 16)
// .. + 7, so that every load instruction reads four whole 256-byte row segments.  Values
// outside the tile's valid rows / features are zero; with lds set they are also parked in the
// unswizzled LDS tile [QT][LDW].
__device__ __forceinline__ int chunk_row(int tid, int i) { return 32 * (tid >> 6) + 4 * i + ((tid & 63) >> 4); }
template <int IN>
__device__ __forceinline__ void load_row_chunk(const uint16_t* __restrict__ x, int64_t K, const TileInfo& ti,
                                               int tid, uint4 (&q)[8], uint16_t* lds, const ActSrc& A = ActSrc()) {
  const int kc = 8 * (tid & 15);
  int64_t row[8];
  bool ok[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = chunk_row(tid, i);
    ok[i] = (r < ti.rows) && (kc < ti.kcols);
    row[i] = ti.gstart + ti.t0 + r;
  }
  load_in8<IN>(x, K, A, row, ok, ti.k0 + kc, q);
  if (lds) {
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<uint4*>(lds + chunk_row(tid, i) * LDW + kc) = q[i];
  }
}

__device__ __forceinline__ void unpack8(const uint4& q, float* v) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
    v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
}

// MXFP8 cast of 32 values: returns the scale code, writes 8 words of E4M3 bytes.
__device__ __forceinline__ uint32_t mx_block(const float* v, uint32_t* w) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const uint32_t code = e8m0_code(amax);
  const float inv = e8m0_inv_scale(code);
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = cvt_e4m3x4(v[4 * i] * inv, v[4 * i + 1] * inv, v[4 * i + 2] * inv, v[4 * i + 3] * inv);
  return code;
}

// MXFP8 group quantize works on half tiles: 64 tokens (one column-wise token panel) x 128
// features (one row-wise MFMA scale word), parked in 17 KB of LDS so that eight workgroups per
// CU keep loads, row casts and column casts of different tiles overlapping.
constexpr int MQT = 64;

// Token half-tile blockIdx.y (the halves of the groups' 128-row tiles) and feature tile
// blockIdx.x.  A half past the group's rows but inside its 128-token padding is valid: its
// column-wise output is the padding (zero data, code 127).
__device__ __forceinline__ bool half_tile_info(const SplitTables& T, int G, int64_t K, TileInfo& ti) {
  const int tt = blockIdx.y >> 1;
  if (G <= 0 || tt >= T.t128_off[G]) return false;
  ti.g = find_group(T.t128_off, G, tt);
  ti.gstart = T.row_off[ti.g];
  ti.m = T.row_off[ti.g + 1] - (int)ti.gstart;
  ti.t0 = (tt - T.t128_off[ti.g]) * QT + MQT * (int)(blockIdx.y & 1);
  ti.rows = max(0, min(MQT, ti.m - ti.t0));
  ti.k0 = (int64_t)blockIdx.x * QF;
  ti.kcols = (int)min((int64_t)QF, K - ti.k0);
  return ti.m > 0;
}

// Column-wise MXFP8 cast of a parked half tile [64 tokens][LDW] whose features are kf0 ..
// kf0 + kcols of a K-feature tensor.  The group's [K, P_g] column-wise tensor is stored in
// 64-byte token panels: byte (f, t) at ((t / 64) K + f) 64 + t % 64, so the half tile is one
// panel row per feature.  Task u = 256 k + tid (k = 0, 1) -> feature c = u / 4, 16-token part
// p = u % 4: a 32-token block spans the lane pair p = 0, 1 or 2, 3 (amax by one shuffle), and
// the 64 lanes of a wave store 16 whole panel rows = 1 KB of contiguous memory per instruction.
// The half tile owns bytes 2 h and 2 h + 1 (h = its half of the 128-token tile) of each
// feature's MFMA scale word.
__device__ __forceinline__ void col_cast_half(const uint16_t* tile, const TileInfo& ti, int64_t K, int64_t kf0,
                                              int kcols, const SplitTables& T, const MxOut& o, int tid) {
  const int p = tid & 3;
  const int P = (ti.m + 127) & ~127;
  const int64_t colbase = K * (int64_t)T.col_off[ti.g];
  const int h = (ti.t0 / MQT) & 1;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = 64 * k + (tid >> 2);
    const int tok0 = 16 * p;
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = bf16_to_f32(tile[tile_off(tok0 + i, c)]);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    const uint32_t code = e8m0_code(amax);
    const float inv = e8m0_inv_scale(code);
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = cvt_e4m3x4(v[4 * i] * inv, v[4 * i + 1] * inv, v[4 * i + 2] * inv, v[4 * i + 3] * inv);
    if (c < kcols) {
      // every token of the half tile lies inside the group's padded range P
      __builtin_nontemporal_store(v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]},
                                  reinterpret_cast<v4i*>(o.col_data + colbase + ((ti.t0 / 64) * K + kf0 + c) * 64 + 16 * p));
      if (o.col_scale && (p & 1) == 0)
        o.col_scale[colbase / 32 + (kf0 + c) * (P / 32) + ti.t0 / 32 + (p >> 1)] = (uint8_t)code;
    }
    // bytes 2 h + (p >> 1) of the word: the lane pair p = 0 and 2 holds both
    const uint32_t pair = (code << (8 * (p >> 1))) | ((uint32_t)__shfl_xor((int)code, 2, 64) << (8 * (1 - (p >> 1))));
    if (o.col_scale_mfma && p == 0 && c < kcols)
      reinterpret_cast<uint16_t*>(o.col_scale_mfma)[2 * (K * (int64_t)T.colw_off[ti.g] + (int64_t)(ti.t0 / 128) * K +
                                                          kf0 + c) + h] = (uint16_t)pair;
  }
}

// ----------------------------------------------------------------------------- MXFP8 cast
// Loads and the row-wise cast: wave w, load i (0..3), lane l -> tile row 16 w + 4 i + l / 16,
// features 8 (l % 16) .. + 7, so every load instruction reads four whole 256-byte row segments.
// A 32-feature block is the lane quad l % 16 in {4b .. 4b + 3} (amax by two shuffles); each
// lane stores its 8 codes into the row's panel, and the 16 lanes of a row assemble its MFMA
// scale word.
template <bool ROW, bool COL>
__global__ __launch_bounds__(256) void mxfp8_quant_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                          SplitTables T, int G, MxOut o) {
  __shared__ __align__(16) uint16_t tile[COL ? MQT * LDW : 8];
  TileInfo ti;
  if (!half_tile_info(T, G, K, ti)) return;
  if (!COL && ti.rows == 0) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int ch = lane & 15;
  const int kc = 8 * ch;
  const bool kok = kc < ti.kcols;
  uint4 q[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * wave + 4 * i + (lane >> 4);
    const bool ok = r < ti.rows && kok;
    q[i] = ok ? *reinterpret_cast<const uint4*>(x + (ti.gstart + ti.t0 + r) * K + ti.k0 + kc) : make_uint4(0, 0, 0, 0);
  }
  if (COL) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * wave + 4 * i + (lane >> 4);
      *reinterpret_cast<uint4*>(tile + tile_off(r, kc)) = q[i];
    }
  }
  if (ROW) {
    const int64_t f = ti.k0 + kc;
    const int64_t pn = f / 64;
    const int64_t pw = min((int64_t)64, K - 64 * pn);    // width of the (last, maybe narrower) panel
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * wave + 4 * i + (lane >> 4);
      const int64_t grow = ti.gstart + ti.t0 + r;
      float v[8];
      unpack8(q[i], v);
      float amax = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
      amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
      amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
      const uint32_t code = e8m0_code(amax);
      const float inv = e8m0_inv_scale(code);
      const uint32_t w0 = cvt_e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
      const uint32_t w1 = cvt_e4m3x4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
      const bool ok = r < ti.rows && kok;
      if (ok) {
        __builtin_nontemporal_store((uint64_t)w0 | ((uint64_t)w1 << 32),
                                    reinterpret_cast<uint64_t*>(o.row_data + 64 * pn * M + grow * pw + (f - 64 * pn)));
        if (o.row_scale && (ch & 3) == 0) o.row_scale[grow * (K / 32) + f / 32] = (uint8_t)code;
      }
      if (o.row_scale_mfma) {
        // byte b of the row's word = block b of its 128 features (127 for blocks past K)
        uint32_t word = (kok ? code : 127u) << (8 * (ch >> 2));
        word |= (uint32_t)__shfl_xor((int)word, 4, 64);
        word |= (uint32_t)__shfl_xor((int)word, 8, 64);
        if (ch == 0 && r < ti.rows) o.row_scale_mfma[(ti.k0 / 128) * M + grow] = word;
      }
    }
  }
  if (!COL) return;
  __syncthreads();
  col_cast_half(tile, ti, K, ti.k0, ti.kcols, T, o, tid);
}

// ----------------------------------------------------------------------------- fused activation gradient + MXFP8 cast
// One pass of the backward between the fc2 dgrad and the fc1 GEMMs: from da = dy W2 (bf16
// [M, ffn]), h = fc1 output (bf16 [M, F1]) and the routing probabilities, it forms
// dh = bf16(d(act(h) p)/dh . da) and casts it row-wise (fc1 dgrad) and column-wise (fc1
// wgrad) to MXFP8 without writing dh itself; the per-row dL/dp partial sums of the tile's 64
// features go to dprob_part[feature tile][row]; with a2 set it also rebuilds the fc2 input
// a = bf16(act(h) p) and casts it column-wise (fc2 wgrad with activation recompute).
//
// Tile = 64 tokens x 64 of the ffn features (one 64-byte K panel of each output; for SwiGLU
// the gate and up gradients of those features are dh columns f and ffn + f).  Thread -> rows
// 32 j + tid / 8 (j = 0, 1), features 8 (tid % 8) .. + 7: every load instruction reads 32 whole
// 128-byte row segments of each input, the 8 lanes of a row reduce its dL/dp partial, a
// 32-feature block is a lane quad, and the lanes of a row store one whole 64-byte panel row.
// Parked tiles (bf16 [64 tokens][DLW]) feed the column pass; the small tiles (18 KB of LDS
// without the rebuild) keep eight workgroups per CU in flight.
constexpr int DF = 64;                // features per tile
constexpr int DLW = DF + 8;           // parked row stride (bf16): 144 bytes, 16-byte aligned
// Element (token r, feature c) of a parked tile: the column pass reads 16 features of four
// 16-token runs 16 tokens apart in one instruction; 16 rows are a whole number of bank lines,
// so the XOR moves the four runs to four different 32-byte windows.
__device__ __forceinline__ int dtile_off(int r, int c) { return r * DLW + (c ^ (((r >> 4) & 3) << 4)); }

// Column-wise MXFP8 cast of a parked [64 tokens][64 features] half tile whose features are
// kf0 .. kf0 + 63 of a K-feature tensor (token panels, as in col_cast_half): thread -> feature
// c = tid / 4, 16-token part p = tid % 4, so the tile is one panel row per feature; the half
// tile owns bytes 2 h, 2 h + 1 of each feature's 128-token MFMA scale word.
__device__ __forceinline__ void col_cast_tile64(const uint16_t* tile, const TileInfo& ti, int64_t K, int64_t kf0,
                                                const SplitTables& T, const MxOut& o, int tid) {
  const int p = tid & 3;
  const int c = tid >> 2;
  const int P = (ti.m + 127) & ~127;
  const int64_t colbase = K * (int64_t)T.col_off[ti.g];
  const int h = (ti.t0 / MQT) & 1;
  {
    const int tok0 = 16 * p;
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = bf16_to_f32(tile[dtile_off(tok0 + i, c)]);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    const uint32_t code = e8m0_code(amax);
    const float inv = e8m0_inv_scale(code);
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = cvt_e4m3x4(v[4 * i] * inv, v[4 * i + 1] * inv, v[4 * i + 2] * inv, v[4 * i + 3] * inv);
    // a half tile lies inside the group's padded range P (a multiple of 128)
    __builtin_nontemporal_store(v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]},
                                reinterpret_cast<v4i*>(o.col_data + colbase + ((ti.t0 / 64) * K + kf0 + c) * 64 + 16 * p));
    if (o.col_scale && (p & 1) == 0)
      o.col_scale[colbase / 32 + (kf0 + c) * (P / 32) + ti.t0 / 32 + (p >> 1)] = (uint8_t)code;
    const uint32_t pair = (code << (8 * (p >> 1))) | ((uint32_t)__shfl_xor((int)code, 2, 64) << (8 * (1 - (p >> 1))));
    if (o.col_scale_mfma && p == 0)
      reinterpret_cast<uint16_t*>(o.col_scale_mfma)[2 * (K * (int64_t)T.colw_off[ti.g] + (int64_t)(ti.t0 / 128) * K +
                                                          kf0 + c) + h] = (uint16_t)pair;
  }
}

template <int KIND, bool WANT_A>
__global__ __launch_bounds__(256) void dact_quant_kernel(DactArgs D, SplitTables T, int G, int64_t M) {
  constexpr bool GLU = act_is_glu(KIND);      // [gate | up] layout (SwiGLU, QGeGLU)
  constexpr int NT = 1 + (GLU ? 1 : 0) + (WANT_A ? 1 : 0);   // parked tiles: dgate (dh), dup, a
  __shared__ __align__(16) uint16_t tiles[NT][MQT * DLW];
  const int64_t ffn = D.ffn;
  const int64_t F1 = GLU ? 2 * ffn : ffn;
  // 64-token half tiles (as the MXFP8 cast); a half past the group's rows still writes its
  // column-wise padding
  TileInfo ti;
  {
    const int tt = blockIdx.y >> 1;
    if (G <= 0 || tt >= T.t128_off[G]) return;
    ti.g = find_group(T.t128_off, G, tt);
    ti.gstart = T.row_off[ti.g];
    ti.m = T.row_off[ti.g + 1] - (int)ti.gstart;
    ti.t0 = (tt - T.t128_off[ti.g]) * QT + MQT * (int)(blockIdx.y & 1);
    ti.rows = max(0, min(MQT, ti.m - ti.t0));
    ti.k0 = (int64_t)blockIdx.x * DF;
    ti.kcols = DF;                                 // ffn is a multiple of 128
    if (ti.m <= 0) return;
  }
  const int tid = threadIdx.x;
  const int rl = tid >> 3, g = tid & 7;
  uint4 qd[2], qg[2], qu[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 32 * j + rl;
    const bool ok = r < ti.rows;
    const int64_t row = ti.gstart + ti.t0 + r;
    qd[j] = ok ? *reinterpret_cast<const uint4*>(D.da + row * ffn + ti.k0 + 8 * g) : make_uint4(0, 0, 0, 0);
    qg[j] = ok ? *reinterpret_cast<const uint4*>(D.h + row * F1 + ti.k0 + 8 * g) : make_uint4(0, 0, 0, 0);
    qu[j] = (GLU && ok) ? *reinterpret_cast<const uint4*>(D.h + row * F1 + ffn + ti.k0 + 8 * g)
                           : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 32 * j + rl;
    const bool ok = r < ti.rows;
    const int64_t grow = ti.gstart + ti.t0 + (ok ? r : 0);
    const float p = ok ? D.probs[grow] : 0.0f;
    float vd[8], vg[8], vu[8];
    unpack8(qd[j], vd);
    unpack8(qg[j], vg);
    unpack8(qu[j], vu);
    // bf16 results, two per word: dgate (or dh), dup, rebuilt a
    uint32_t p0[4], p1[4], pa[4];
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      float r0[2], r1[2], ra[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        float dp, av = 0.0f;
        const float u = GLU ? vu[i + k] : 0.0f;
        if (WANT_A) act_grad_out<KIND>(vg[i + k], u, vd[i + k], p, D.act.c, r0[k], r1[k], dp, av);
        else act_grad<KIND>(vg[i + k], u, vd[i + k], p, D.act.c, r0[k], r1[k], dp);
        psum += dp;
        ra[k] = av;
      }
      p0[i / 2] = pack_bf16x2(r0[0], r0[1]);
      p1[i / 2] = pack_bf16x2(r1[0], r1[1]);
      pa[i / 2] = (__float_as_uint(ra[0]) >> 16) | (__float_as_uint(ra[1]) & 0xFFFF0000u);
    }
    // dL/dp partial of the row over the tile's 64 features (fixed order: the thread's 8, then
    // pairs, quads, halves)
    psum += __shfl_xor(psum, 1, 64);
    psum += __shfl_xor(psum, 2, 64);
    psum += __shfl_xor(psum, 4, 64);
    if (g == 0 && ok) D.dprob_part[(int64_t)blockIdx.x * M + grow] = psum;
    // row-wise cast of the thread's 8 values of one 32-block (gate / plain gradient at feature
    // f, up at ffn + f), and the values parked for the column pass
    auto row_cast = [&](const uint32_t* pk, int64_t f, uint16_t* tile) {
      if (D.dh.row_data) {
        float v[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[2 * i] = bf16_to_f32(pk[i] & 0xFFFFu);
          v[2 * i + 1] = bf16_to_f32(pk[i] >> 16);
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
        amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
        amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
        const uint32_t code = e8m0_code(amax);
        const float inv = e8m0_inv_scale(code);
        const uint32_t w0 = cvt_e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
        const uint32_t w1 = cvt_e4m3x4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
        // the tile's two blocks are bytes b, b + 1 of the row's 128-feature MFMA word
        const uint32_t pair = code | ((uint32_t)__shfl_xor((int)code, 4, 64) << 8);
        if (ok) {
          __builtin_nontemporal_store((uint64_t)w0 | ((uint64_t)w1 << 32),
                                      reinterpret_cast<uint64_t*>(D.dh.row_data + (f / 64) * 64 * M + grow * 64 + (f & 63)));
          if (D.dh.row_scale && (g & 3) == 0) D.dh.row_scale[grow * (F1 / 32) + f / 32] = (uint8_t)code;
          if (D.dh.row_scale_mfma && g == 0)
            *reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(D.dh.row_scale_mfma) +
                                         ((f / 128) * M + grow) * 4 + (f & 127) / 32) = (uint16_t)pair;
        }
      }
      *reinterpret_cast<uint4*>(tile + dtile_off(r, 8 * g)) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    };
    row_cast(p0, ti.k0 + 8 * g, tiles[0]);
    if (GLU) row_cast(p1, ffn + ti.k0 + 8 * g, tiles[1]);
    if (WANT_A) *reinterpret_cast<uint4*>(tiles[NT - 1] + dtile_off(r, 8 * g)) = make_uint4(pa[0], pa[1], pa[2], pa[3]);
  }
  __syncthreads();
  if (D.dh.col_data) {
    col_cast_tile64(tiles[0], ti, F1, ti.k0, T, D.dh, tid);
    if (GLU) col_cast_tile64(tiles[1], ti, F1, ffn + ti.k0, T, D.dh, tid);
  }
  if (WANT_A) col_cast_tile64(tiles[NT - 1], ti, ffn, ti.k0, T, D.a2, tid);
}

// ----------------------------------------------------------------------------- activation + MXFP8 cast (forward)
// The MXFP8 forward's fc2 input: from h = fc1 output (bf16 [M, F1]) and the routing
// probabilities, a = bf16(act(h) p) (the same function as the backward's rebuild, so the bits
// match) is cast row-wise for the fc2 GEMM and, when o.col_data is set, column-wise for the fc2
// wgrad; a itself is never written.  Half tiles and thread layout as in dact_quant_kernel:
// 64 tokens x 64 features of a (SwiGLU: gate feature f and up feature ffn + f of h).
template <int KIND>
__global__ __launch_bounds__(256) void act_quant_kernel(const uint16_t* __restrict__ h, const float* __restrict__ probs,
                                                        float act_c, int64_t ffn, SplitTables T, int G, int64_t M,
                                                        MxOut o) {
  constexpr bool GLU = act_is_glu(KIND);      // [gate | up] layout (SwiGLU, QGeGLU)
  __shared__ __align__(16) uint16_t tile[MQT * DLW];
  const int64_t F1 = GLU ? 2 * ffn : ffn;
  TileInfo ti;
  {
    const int tt = blockIdx.y >> 1;
    if (G <= 0 || tt >= T.t128_off[G]) return;
    ti.g = find_group(T.t128_off, G, tt);
    ti.gstart = T.row_off[ti.g];
    ti.m = T.row_off[ti.g + 1] - (int)ti.gstart;
    ti.t0 = (tt - T.t128_off[ti.g]) * QT + MQT * (int)(blockIdx.y & 1);
    ti.rows = max(0, min(MQT, ti.m - ti.t0));
    ti.k0 = (int64_t)blockIdx.x * DF;
    ti.kcols = DF;                                 // ffn is a multiple of 128
    if (ti.m <= 0) return;
  }
  const int tid = threadIdx.x;
  const int rl = tid >> 3, g = tid & 7;
  uint4 qg[2], qu[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 32 * j + rl;
    const bool ok = r < ti.rows;
    const int64_t row = ti.gstart + ti.t0 + r;
    qg[j] = ok ? *reinterpret_cast<const uint4*>(h + row * F1 + ti.k0 + 8 * g) : make_uint4(0, 0, 0, 0);
    qu[j] = (GLU && ok) ? *reinterpret_cast<const uint4*>(h + row * F1 + ffn + ti.k0 + 8 * g) : make_uint4(0, 0, 0, 0);
  }
  const int64_t f = ti.k0 + 8 * g;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 32 * j + rl;
    const bool ok = r < ti.rows;
    const int64_t grow = ti.gstart + ti.t0 + (ok ? r : 0);
    const float p = ok ? probs[grow] : 0.0f;
    float vg[8], vu[8], v[8];
    unpack8(qg[j], vg);
    unpack8(qu[j], vu);
    uint32_t pa[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = act_out<KIND>(vg[i], GLU ? vu[i] : 0.0f, p, act_c);
#pragma unroll
    for (int i = 0; i < 4; ++i) pa[i] = (__float_as_uint(v[2 * i]) >> 16) | (__float_as_uint(v[2 * i + 1]) & 0xFFFF0000u);
    // row-wise cast: a 32-feature block is a lane quad; the tile's two blocks are bytes b, b + 1
    // of the row's 128-feature MFMA word
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    const uint32_t code = e8m0_code(amax);
    const float inv = e8m0_inv_scale(code);
    const uint32_t w0 = cvt_e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
    const uint32_t w1 = cvt_e4m3x4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
    const uint32_t pair = code | ((uint32_t)__shfl_xor((int)code, 4, 64) << 8);
    if (ok) {
      __builtin_nontemporal_store((uint64_t)w0 | ((uint64_t)w1 << 32),
                                  reinterpret_cast<uint64_t*>(o.row_data + (f / 64) * 64 * M + grow * 64 + (f & 63)));
      if (o.row_scale && (g & 3) == 0) o.row_scale[grow * (ffn / 32) + f / 32] = (uint8_t)code;
      if (o.row_scale_mfma && g == 0)
        *reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(o.row_scale_mfma) + ((f / 128) * M + grow) * 4 +
                                     (f & 127) / 32) = (uint16_t)pair;
    }
    *reinterpret_cast<uint4*>(tile + dtile_off(r, 8 * g)) = make_uint4(pa[0], pa[1], pa[2], pa[3]);
  }
  if (!o.col_data) return;
  __syncthreads();
  col_cast_tile64(tile, ti, ffn, ti.k0, T, o, tid);
}

template <int IN>
__global__ __launch_bounds__(256) void hadamard_amax_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                            SplitTables T, int G, uint32_t mask, ActSrc A) {
  __shared__ __align__(16) uint16_t tile[QT * LDW];
  __shared__ float red[2][4];
  TileInfo ti;
  if (!tile_info(T, G, K, ti)) return;
  const int tid = threadIdx.x;
  uint4 q[8];
  load_row_chunk<IN>(x, K, ti, tid, q, tile, A);
  float amax_pre = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float v[8];
    unpack8(q[j], v);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax_pre = fmaxf(amax_pre, fabsf(v[i]));
  }
  __syncthreads();
  const int c = tid & (QF - 1);
  const int half = tid >> 7;
  float amax_post = 0.0f;
  if (c < ti.kcols) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tb = 4 * half + j;        // 16-token block; blocks past the rows read zeros
      float v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = bf16_to_f32(tile[(16 * tb + i) * LDW + c]);
      signed_fwht16(v, mask);
#pragma unroll
      for (int i = 0; i < 16; ++i) amax_post = fmaxf(amax_post, fabsf(v[i]));
    }
  }
  // max |bf16(y/4)| = bf16(max |y| / 4): the factor is exact and rounding is monotone
  amax_post = round_bf16(amax_post * 0.25f);
  amax_pre = wave_max(amax_pre);
  amax_post = wave_max(amax_post);
  const int wave = tid >> 6;
  if ((tid & 63) == 0) { red[0][wave] = amax_pre; red[1][wave] = amax_post; }
  __syncthreads();
  if (tid == 0) {
    float a = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
    float b = fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));
    // non-negative floats order like their bit patterns; one of the group's slots per workgroup
    const int slot = (int)((blockIdx.x + 7u * blockIdx.y) % (unsigned)kAmaxSlots);
    atomicMax(T.amax_slots + ((int64_t)ti.g * kAmaxSlots + slot), __float_as_uint(a));
    atomicMax(T.amax_slots + ((int64_t)(G + ti.g) * kAmaxSlots + slot), __float_as_uint(b));
  }
}

// pre[g] / post[g] = the max over the group's slots, which are cleared for the next amax pass.
__global__ __launch_bounds__(256) void amax_finalize_kernel(SplitTables T, int G, float* __restrict__ pre,
                                                            float* __restrict__ post) {
  const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);     // (direction, group)
  if (i >= 2 * G) return;
  uint32_t* s = T.amax_slots + (int64_t)i * kAmaxSlots;
  uint32_t m = 0;
#pragma unroll 8
  for (int j = 0; j < kAmaxSlots; ++j) {
    m = max(m, s[j]);
    s[j] = 0u;
  }
  (i < G ? pre : post)[i < G ? i : i - G] = __uint_as_float(m);
}

// ----------------------------------------------------------------------------- NVFP4 cast
// One 16-value block with global scale S: writes 8 packed bytes (two words), returns the E4M3 code.
//   s = fp32(fp32(b / 6) * S); q = E4M3(s); r = min(fp32(S / dec(q)), FLT_MAX) (0 if q == 0);
//   c_i = E2M1(fp32(v_i * r)).  r is clipped like S, so a zero element casts to zero even when S
//   itself was clipped (S / dec(q) would overflow and 0 * inf is no number).
__device__ __forceinline__ uint32_t nv_block(const float* v, float S, uint32_t& lo, uint32_t& hi) {
  float b = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) b = fmaxf(b, fabsf(v[i]));
  const float s = __fmul_rn(__fdiv_rn(b, 6.0f), S);
  const uint32_t code = cvt_e4m3(s);
  const float r = (code == 0) ? 0.0f : fminf(__fdiv_rn(S, e4m3_decode_pos(code)), kFltMax);
  float t[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) t[i] = __fmul_rn(v[i], r);
  lo = cvt_e2m1x8(t);
  hi = cvt_e2m1x8(t + 8);
  return code;
}

// Eight packed E2M1 codes (one word) with block scale sc as eight bf16 dec(E2M1) dec(E4M3).
__device__ __forceinline__ v4i nv_bf16x8(uint32_t w, float sc) {
  return v4i{(int)e2m1x2_scaled_bf16<0>(w, sc), (int)e2m1x2_scaled_bf16<1>(w, sc), (int)e2m1x2_scaled_bf16<2>(w, sc),
             (int)e2m1x2_scaled_bf16<3>(w, sc)};
}
// The 16 quantized values of a block as bf16 dec(E2M1) dec(E4M3) (exact: at most 6 significant
// bits), written as 32 contiguous bytes of a GEMM operand panel: half of a 64-byte panel row,
// whose other half the same lane writes for the neighbouring block.  Plain (write-back) stores,
// so that the two halves meet in L2 before the line goes to HBM.
__device__ __forceinline__ void nv_bf16_store(uint8_t* dst, uint32_t lo, uint32_t hi, uint32_t code) {
  const float sc = e4m3_decode_pos(code);
  *reinterpret_cast<v4i*>(dst) = nv_bf16x8(lo, sc);
  *reinterpret_cast<v4i*>(dst + 16) = nv_bf16x8(hi, sc);
}

// Half (8 values) of a 16-value block whose other half lane ^ 1 holds: the same steps as
// nv_block, with the block maximum taken across the lane pair.  Returns the E4M3 code and the
// 8 packed E2M1 codes (one word).
__device__ __forceinline__ uint32_t nv_half_block(const float* v, float S, uint32_t& word) {
  float b = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) b = fmaxf(b, fabsf(v[i]));
  b = fmaxf(b, __shfl_xor(b, 1, 64));
  const float s = __fmul_rn(__fdiv_rn(b, 6.0f), S);
  const uint32_t code = cvt_e4m3(s);
  const float r = (code == 0) ? 0.0f : fminf(__fdiv_rn(S, e4m3_decode_pos(code)), kFltMax);
  float t[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) t[i] = __fmul_rn(v[i], r);
  word = cvt_e2m1x8(t);
  return code;
}

// The 8 values of one lane's half block as bf16 dec(E2M1) dec(E4M3): 16 bytes of a panel row.
__device__ __forceinline__ uint4 nv_bf16_half(uint32_t w, uint32_t code) {
  const v4i o = nv_bf16x8(w, e4m3_decode_pos(code));
  return make_uint4((uint32_t)o[0], (uint32_t)o[1], (uint32_t)o[2], (uint32_t)o[3]);
}

template <bool ROW, bool COL, int IN>
__global__ __launch_bounds__(256) void nvfp4_quant_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                          SplitTables T, int G, uint32_t mask, int rht,
                                                          const float* __restrict__ pre,
                                                          const float* __restrict__ post, NvOut o, ActSrc A) {
  // 64-token half tiles, as the MXFP8 cast: load i of a thread covers half-tile row
  // 16 wave + 4 i + lane / 16, features 8 (lane % 16) .. + 7
  __shared__ __align__(16) uint16_t tile[COL ? MQT * LDW : 8];
  TileInfo ti;
  if (!half_tile_info(T, G, K, ti)) return;
  if (!COL && ti.rows == 0) return;
  const int tid = threadIdx.x;
  auto hrow = [&](int i) { return 16 * (tid >> 6) + 4 * i + ((tid & 63) >> 4); };
  uint4 q[4];
  {
    const int kc = 8 * (tid & 15);
    int64_t row[4];
    bool ok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = hrow(i);
      ok[i] = (r < ti.rows) && (kc < ti.kcols);
      row[i] = ti.gstart + ti.t0 + r;
    }
    load_in8<IN>(x, K, A, row, ok, ti.k0 + kc, q);
    if (COL) {
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(tile + hrow(i) * LDW + kc) = q[i];
    }
  }
  if (ROW) {
    // a 16-value block is a lane pair; the 16 lanes of a row write 64 contiguous packed bytes and
    // four whole 64-byte bf16 panel rows per instruction
    const float S = nvfp4_global_scale(pre[ti.g]);
    const int kc = 8 * (tid & 15);
    const int64_t k = ti.k0 + kc;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = hrow(i);
      const int64_t grow = ti.gstart + ti.t0 + r;
      float v[8];
      unpack8(q[i], v);
      uint32_t w;
      const uint32_t code = nv_half_block(v, S, w);
      if (r < ti.rows && kc < ti.kcols) {
        const int64_t e = grow * K + k;                          // element index
        if (o.row_data) {
          *reinterpret_cast<uint32_t*>(o.row_data + e / 2) = w;
          if ((tid & 1) == 0) o.row_scale[e / 16] = (uint8_t)code;
        }
        if (o.row_bf16)
          *reinterpret_cast<uint4*>(o.row_bf16 + ((k / 32) * M + grow) * 64 + 2 * (k % 32)) = nv_bf16_half(w, code);
      }
    }
  }
  if (!COL) return;
  __syncthreads();
  const float S = nvfp4_global_scale(rht ? post[ti.g] : pre[ti.g]);
  const int c = tid & (QF - 1);
  const int half = tid >> 7;
  const int P = (ti.m + 127) & ~127;
  const int64_t colbase = K * (int64_t)T.col_off[ti.g];
  if (c >= ti.kcols) return;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int tb = 2 * half + j;                               // a half tile lies inside the padding P
    if (ti.t0 + 16 * tb >= P) break;
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = bf16_to_f32(tile[(16 * tb + i) * LDW + c]);
    if (rht) {
      signed_fwht16(v, mask);
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = round_bf16(v[i] * 0.25f);
    }
    uint32_t lo, hi;
    const uint32_t code = nv_block(v, S, lo, hi);
    const int64_t t = ti.t0 + 16 * tb;                          // token within the group
    const int64_t e = colbase + (ti.k0 + c) * P + t;
    if (o.col_data) {
      *reinterpret_cast<uint2*>(o.col_data + e / 2) = make_uint2(lo, hi);
      o.col_scale[e / 16] = (uint8_t)code;
    }
    if (o.col_bf16)
      nv_bf16_store(o.col_bf16 + 2 * colbase + ((t / 32) * K + ti.k0 + c) * 64 + 2 * (t % 32), lo, hi, code);
  }
}

// ----------------------------------------------------------------------------- weights
// Per-expert amax of W [E, N, K] (stacked, or discrete via w_ptrs): grid (chunks, E).
__global__ __launch_bounds__(256) void weight_amax_kernel(const uint16_t* __restrict__ w, const void* const* w_ptrs,
                                                          int64_t NK, float* amax) {
  const int e = blockIdx.y;
  const uint16_t* base = w_ptrs ? static_cast<const uint16_t*>(w_ptrs[e]) : w + (int64_t)e * NK;
  float m = 0.0f;
  const int64_t nvec = NK / 8;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += (int64_t)gridDim.x * blockDim.x) {
    float v[8];
    unpack8(reinterpret_cast<const uint4*>(base)[i], v);
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) atomicMax(reinterpret_cast<unsigned int*>(amax + e), __float_as_uint(m));
}

__global__ __launch_bounds__(256) void gather_weights_kernel(const void* const* w_ptrs, int64_t NK, uint16_t* out) {
  const int e = blockIdx.y;
  const uint4* src = static_cast<const uint4*>(w_ptrs[e]);
  uint4* dst = reinterpret_cast<uint4*>(out + (int64_t)e * NK);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < NK / 8; i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

// ----------------------------------------------------------------------------- launchers
// x: feature tiles (consecutive workgroups write neighbouring panel rows of the column-wise
// output and read neighbouring 256-byte row segments), y: token tiles.
static dim3 tile_grid(int64_t M, int64_t K, int G) {
  return dim3((unsigned)((K + QF - 1) / QF), (unsigned)((M + QT - 1) / QT + G));
}

hipError_t launch_scan(const int32_t* m_splits, int G, int64_t M, SplitTables T, hipStream_t s) {
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(256), 0, s, m_splits, G, M, T);
  return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* p, uint32_t v, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}

hipError_t launch_mxfp8_quant(const uint16_t* x, int64_t M, int64_t K, SplitTables T, int G, bool row, bool col,
                              MxOut o, hipStream_t s) {
  if (M == 0 || (!row && !col)) return hipSuccess;
  const dim3 grid((unsigned)((K + QF - 1) / QF), (unsigned)(2 * ((M + QT - 1) / QT + G)));   // half tiles
  if (row && col) hipLaunchKernelGGL((mxfp8_quant_kernel<true, true>), grid, dim3(256), 0, s, x, M, K, T, G, o);
  else if (row) hipLaunchKernelGGL((mxfp8_quant_kernel<true, false>), grid, dim3(256), 0, s, x, M, K, T, G, o);
  else hipLaunchKernelGGL((mxfp8_quant_kernel<false, true>), grid, dim3(256), 0, s, x, M, K, T, G, o);
  return hipGetLastError();
}

hipError_t launch_dact_quant(const DactArgs& d, SplitTables T, int G, int64_t M, hipStream_t s) {
  if (M == 0) return hipSuccess;
  const dim3 grid((unsigned)(d.ffn / DF), (unsigned)(2 * ((M + QT - 1) / QT + G)));   // half tiles
  const bool a = d.a2.col_data != nullptr;
#define GMLP_DACT(K)                                                                                  \
  if (a) hipLaunchKernelGGL((dact_quant_kernel<K, true>), grid, dim3(256), 0, s, d, T, G, M);        \
  else hipLaunchKernelGGL((dact_quant_kernel<K, false>), grid, dim3(256), 0, s, d, T, G, M);
  switch (d.act.kind) {
    case ACT_SWIGLU: GMLP_DACT(ACT_SWIGLU) break;
    case ACT_SRELU: GMLP_DACT(ACT_SRELU) break;
    case ACT_TANH_SRELU: GMLP_DACT(ACT_TANH_SRELU) break;
    case ACT_QGEGLU: GMLP_DACT(ACT_QGEGLU) break;
    default: return hipErrorInvalidValue;
  }
#undef GMLP_DACT
  return hipGetLastError();
}

hipError_t launch_act_quant(const uint16_t* h, const float* probs, Act act, int64_t ffn, SplitTables T, int G,
                            int64_t M, MxOut o, hipStream_t s) {
  if (M == 0) return hipSuccess;
  const dim3 grid((unsigned)(ffn / DF), (unsigned)(2 * ((M + QT - 1) / QT + G)));   // half tiles
  switch (act.kind) {
    case ACT_SWIGLU:
      hipLaunchKernelGGL((act_quant_kernel<ACT_SWIGLU>), grid, dim3(256), 0, s, h, probs, act.c, ffn, T, G, M, o);
      break;
    case ACT_SRELU:
      hipLaunchKernelGGL((act_quant_kernel<ACT_SRELU>), grid, dim3(256), 0, s, h, probs, act.c, ffn, T, G, M, o);
      break;
    case ACT_TANH_SRELU:
      hipLaunchKernelGGL((act_quant_kernel<ACT_TANH_SRELU>), grid, dim3(256), 0, s, h, probs, act.c, ffn, T, G, M, o);
      break;
    case ACT_QGEGLU:
      hipLaunchKernelGGL((act_quant_kernel<ACT_QGEGLU>), grid, dim3(256), 0, s, h, probs, act.c, ffn, T, G, M, o);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_amax_finalize(SplitTables T, int G, float* pre, float* post, hipStream_t s) {
  hipLaunchKernelGGL(amax_finalize_kernel, dim3((unsigned)((2 * G + 255) / 256)), dim3(256), 0, s, T, G, pre, post);
  return hipGetLastError();
}

hipError_t launch_hadamard_amax(const uint16_t* x, int64_t M, int64_t K, SplitTables T, int G, uint32_t mask,
                                float* pre, float* post, hipStream_t s, ActSrc act) {
  // with no rows the finalize still writes the (zero) amax of every group
  if (M > 0) {
    const dim3 grid = tile_grid(M, K, G);
    switch (input_kind(act)) {
      case kInX: hipLaunchKernelGGL(hadamard_amax_kernel<kInX>, grid, dim3(256), 0, s, x, M, K, T, G, mask, act); break;
      case ACT_SWIGLU: hipLaunchKernelGGL(hadamard_amax_kernel<ACT_SWIGLU>, grid, dim3(256), 0, s, x, M, K, T, G, mask, act); break;
      case ACT_SRELU: hipLaunchKernelGGL(hadamard_amax_kernel<ACT_SRELU>, grid, dim3(256), 0, s, x, M, K, T, G, mask, act); break;
      case ACT_TANH_SRELU: hipLaunchKernelGGL(hadamard_amax_kernel<ACT_TANH_SRELU>, grid, dim3(256), 0, s, x, M, K, T, G, mask, act); break;
      default: hipLaunchKernelGGL(hadamard_amax_kernel<ACT_QGEGLU>, grid, dim3(256), 0, s, x, M, K, T, G, mask, act); break;
    }
  }
  hipLaunchKernelGGL(amax_finalize_kernel, dim3((unsigned)((2 * G + 255) / 256)), dim3(256), 0, s, T, G, pre, post);
  return hipGetLastError();
}

hipError_t launch_nvfp4_quant(const uint16_t* x, int64_t M, int64_t K, SplitTables T, int G, uint32_t mask,
                              bool rht, bool row, bool col, const float* pre, const float* post, NvOut o,
                              hipStream_t s, ActSrc act) {
  if (M == 0 || (!row && !col)) return hipSuccess;
  const dim3 grid((unsigned)((K + QF - 1) / QF), (unsigned)(2 * ((M + QT - 1) / QT + G)));   // half tiles
  const int r = rht ? 1 : 0;
  auto go = [&](auto in) {
    constexpr int IN = decltype(in)::value;
    if (row && col)
      hipLaunchKernelGGL((nvfp4_quant_kernel<true, true, IN>), grid, dim3(256), 0, s, x, M, K, T, G, mask, r, pre, post,
                         o, act);
    else if (row)
      hipLaunchKernelGGL((nvfp4_quant_kernel<true, false, IN>), grid, dim3(256), 0, s, x, M, K, T, G, mask, r, pre, post,
                         o, act);
    else
      hipLaunchKernelGGL((nvfp4_quant_kernel<false, true, IN>), grid, dim3(256), 0, s, x, M, K, T, G, mask, r, pre, post,
                         o, act);
  };
  switch (input_kind(act)) {
    case kInX: go(std::integral_constant<int, kInX>()); break;
    case ACT_SWIGLU: go(std::integral_constant<int, ACT_SWIGLU>()); break;
    case ACT_SRELU: go(std::integral_constant<int, ACT_SRELU>()); break;
    case ACT_TANH_SRELU: go(std::integral_constant<int, ACT_TANH_SRELU>()); break;
    default: go(std::integral_constant<int, ACT_QGEGLU>()); break;
  }
  return hipGetLastError();
}

hipError_t launch_weight_amax(const uint16_t* w, const void* const* w_ptrs, int E, int64_t N, int64_t K,
                              float* amax, hipStream_t s) {
  if (E == 0) return hipSuccess;
  hipError_t err = launch_fill_u32(reinterpret_cast<uint32_t*>(amax), 0u, E, s);
  if (err != hipSuccess) return err;
  const int64_t nvec = N * K / 8;
  const unsigned chunks = (unsigned)std::max<int64_t>(1, std::min<int64_t>((nvec + 255) / 256, 256));
  hipLaunchKernelGGL(weight_amax_kernel, dim3(chunks, E), dim3(256), 0, s, w, w_ptrs, N * K, amax);
  return hipGetLastError();
}

hipError_t launch_gather_weights(const void* const* w_ptrs, int E, int64_t N, int64_t K, uint16_t* out,
                                 hipStream_t s) {
  if (E == 0) return hipSuccess;
  const int64_t nvec = N * K / 8;
  const unsigned chunks = (unsigned)std::max<int64_t>(1, std::min<int64_t>((nvec + 255) / 256, 1024));
  hipLaunchKernelGGL(gather_weights_kernel, dim3(chunks, E), dim3(256), 0, s, w_ptrs, N * K, out);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------- NVFP4 -> bf16 panels
// The NVFP4 GEMMs run on the bf16 MFMA: each operand element becomes dec(E2M1) * dec(E4M3), which
// has at most 6 significant bits and a magnitude in [2^-10, 2688], so bf16 holds it exactly (the
// per-group global scales are applied to the fp32 result).  The expanded operand uses the MXFP8
// operands' 64-byte K panels with 2-byte elements: element (r, c) of an R x C matrix at byte
// ((c / 32) R + r) 64 + 2 (c % 32).
// A block covers 16 rows x 128 columns; thread -> row 16 by + tid / 16, 32-column chunk
// (tid / 4) % 4, 8 columns 8 (tid % 4) of it: it reads one packed word and writes 16 bytes, and
// the four lanes of a chunk-row write one whole 64-byte panel row.
// Dense batch (col_off == null): matrix blockIdx.z of nmat equal [R, C] matrices, stored one
// after the other.  Grouped (column-wise activations): the groups' [R, P_g] matrices at element
// offsets R * col_off[g]; blockIdx.x walks 128-column units of their concatenation (P_g is a
// multiple of 128, so a unit never straddles two groups).
__global__ __launch_bounds__(256) void nv_expand_kernel(const uint8_t* __restrict__ data,
                                                        const uint8_t* __restrict__ scale, uint8_t* __restrict__ out,
                                                        int64_t R, int64_t C, const int32_t* __restrict__ col_off,
                                                        int G) {
  const int tid = threadIdx.x;
  const int64_t r = (int64_t)blockIdx.y * 16 + (tid >> 4);
  if (r >= R) return;
  int64_t base, c0, cols;
  if (col_off) {
    const int u = (int)blockIdx.x * 128;
    if (u >= col_off[G]) return;
    const int g = find_group(col_off, G, u);
    base = R * (int64_t)col_off[g];
    cols = col_off[g + 1] - col_off[g];
    c0 = u - col_off[g];
  } else {
    base = (int64_t)blockIdx.z * R * C;
    cols = C;
    c0 = (int64_t)blockIdx.x * 128;
  }
  const int j = (tid >> 2) & 3, q = tid & 3;
  const int64_t c = c0 + 32 * j + 8 * q;
  if (c >= cols) return;
  const int64_t e = base + r * cols + c;                   // element index (a multiple of 8)
  const uint32_t w = *reinterpret_cast<const uint32_t*>(data + e / 2);
  uint8_t* dst = out + 2 * base + (((c / 32) * R + r) * 64 + 2 * (c % 32));
  __builtin_nontemporal_store(nv_bf16x8(w, e4m3_decode_pos(scale[e / 16])), reinterpret_cast<v4i*>(dst));
}

hipError_t launch_nv_expand(const uint8_t* data, const uint8_t* scale, uint8_t* out, int64_t R, int64_t C, int nmat,
                            hipStream_t s) {
  if (R == 0 || C == 0 || nmat == 0) return hipSuccess;
  hipLaunchKernelGGL(nv_expand_kernel, dim3((unsigned)((C + 127) / 128), (unsigned)((R + 15) / 16), (unsigned)nmat),
                     dim3(256), 0, s, data, scale, out, R, C, (const int32_t*)nullptr, 0);
  return hipGetLastError();
}

hipError_t launch_nv_expand_groups(const uint8_t* data, const uint8_t* scale, uint8_t* out, int64_t R,
                                   int64_t cols_bound, const int32_t* col_off, int G, hipStream_t s) {
  if (R == 0 || cols_bound == 0 || G == 0) return hipSuccess;
  hipLaunchKernelGGL(nv_expand_kernel, dim3((unsigned)((cols_bound + 127) / 128), (unsigned)((R + 15) / 16), 1u),
                     dim3(256), 0, s, data, scale, out, R, (int64_t)0, col_off, G);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------- activation gradient (bf16)
// NVFP4 backward between the fc2 dgrad (bf16 da [M, ffn]) and the dh casts: dh = bf16(d(act(h) p)/dh
// . da) written as bf16 [M, F1] (SwiGLU: the gate gradient at feature f, the up gradient at
// ffn + f), the rebuilt fc2 input a' = bf16(act(h) p) when a2 is set, and per-row dL/dp partials of
// each 256-feature tile (summed over its features in a fixed lane order) in dprob_part[tile][row].
// Block = 8 rows x 256 features; thread -> row 8 by + tid / 32, features 8 (tid % 32) .. + 7.
__global__ __launch_bounds__(256) void dact_bf16_kernel(const uint16_t* __restrict__ da, const uint16_t* __restrict__ h,
                                                        const float* __restrict__ probs, Act act, int64_t ffn,
                                                        int64_t M, uint16_t* __restrict__ dh, uint16_t* __restrict__ a2,
                                                        float* __restrict__ dprob_part) {
  const int tid = threadIdx.x;
  const int64_t row = (int64_t)blockIdx.y * 8 + (tid >> 5);
  if (row >= M) return;                                    // whole 32-lane row groups leave together
  const bool glu = act_is_glu(act.kind);
  const int64_t F1 = glu ? 2 * ffn : ffn;
  const int64_t f = (int64_t)blockIdx.x * 256 + 8 * (tid & 31);
  float psum = 0.0f;
  if (f < ffn) {
    const float p = probs[row];
    const uint4 dv = *reinterpret_cast<const uint4*>(da + row * ffn + f);
    const uint4 gv = *reinterpret_cast<const uint4*>(h + row * F1 + f);
    const uint4 uv = glu ? *reinterpret_cast<const uint4*>(h + row * F1 + ffn + f) : make_uint4(0, 0, 0, 0);
    const uint32_t dw[4] = {dv.x, dv.y, dv.z, dv.w}, gw[4] = {gv.x, gv.y, gv.z, gv.w}, uw[4] = {uv.x, uv.y, uv.z, uv.w};
    uint32_t o0[4], o1[4], oa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t r0 = 0, r1 = 0, ra = 0;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const float dav = bf16_to_f32((dw[i] >> (16 * hh)) & 0xFFFFu);
        const float g = bf16_to_f32((gw[i] >> (16 * hh)) & 0xFFFFu);
        const float u = bf16_to_f32((uw[i] >> (16 * hh)) & 0xFFFFu);
        float d0, d1, dp, av;
        act_grad_out_rt(act, g, u, dav, p, d0, d1, dp, av);
        psum += dp;
        r0 |= f32_to_bf16_bits(d0) << (16 * hh);
        r1 |= f32_to_bf16_bits(d1) << (16 * hh);
        ra |= (__float_as_uint(av) >> 16) << (16 * hh);
      }
      o0[i] = r0;
      o1[i] = r1;
      oa[i] = ra;
    }
    *reinterpret_cast<uint4*>(dh + row * F1 + f) = make_uint4(o0[0], o0[1], o0[2], o0[3]);
    if (glu) *reinterpret_cast<uint4*>(dh + row * F1 + ffn + f) = make_uint4(o1[0], o1[1], o1[2], o1[3]);
    if (a2) *reinterpret_cast<uint4*>(a2 + row * ffn + f) = make_uint4(oa[0], oa[1], oa[2], oa[3]);
  }
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) psum += __shfl_xor(psum, o, 64);
  if ((tid & 31) == 0) dprob_part[(int64_t)blockIdx.x * M + row] = psum;
}

hipError_t launch_dact_bf16(const uint16_t* da, const uint16_t* h, const float* probs, Act act, int64_t ffn, int64_t M,
                            uint16_t* dh, uint16_t* a2, float* dprob_part, hipStream_t s) {
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL(dact_bf16_kernel, dim3((unsigned)((ffn + 255) / 256), (unsigned)((M + 7) / 8)), dim3(256), 0, s,
                     da, h, probs, act, ffn, M, dh, a2, dprob_part);
  return hipGetLastError();
}

}  // namespace gmlp
