// Grouped GEMMs of the MoE MLP on CDNA4 matrix cores.  Every GEMM stores its result as it is:
// bf16 or fp32, or (weight gradients) added in fp32 to what the output holds.  The activation,
// its gradient and dprob run as memory-bound passes of their own over the stored h and da
// (quant.hip), unlike the pages' kernels, which fuse them into the fc1 and fc2-dgrad GEMMs.
//
// Sources: "GEMM + Swiglu fused Grouped MLP for MXFP8" (sequence diagram: the fc1 GEMM
// with the bf16 pre-activation, the fc2 GEMM, the fc2 dgrad, the fc1 dgrad and the wgrad
// grouped GEMMs) and "Reduce NVFP4 quantization work ..." (Description and commits: the
// accumulator is rounded through the bf16 C dtype before the activation).
//
// Every GEMM here is C = A . B^T with both operands K-contiguous:
//   FPROP  A = row-wise [rows of group g, K], B = expert g's [N, K]      (fc1, fc2, both dgrads)
//   WGRAD  A = column-wise [N_a, P_g], B = column-wise [N_b, P_g]        (both wgrads, K = tokens)
//
// One persistent kernel: workgroup tile 256 x 256, 4 waves of 128 x 128 (4 x 4 tiles of
// 32 x 32), K staged through a 4-slot LDS ring of 64-byte rows (64 fp8, or 32 bf16 for
// NVFP4) filled by buffer-to-LDS DMA, 16-byte chunks XOR-swizzled by row so that the MFMA
// fragment reads are bank-conflict-free.  bf16 outputs take the transposed product and a
// bf16-staged epilogue (mx_epilogue_tr); fp32 outputs and the fused amax stage fp32
// (mx_epilogue).
//
// MXFP8: V_MFMA_SCALE_F32_32X32X64_F8F6F4 with E8M0 block scales.  Lane (m + 32j)
// holds row m, K bytes [16j, 16j+16) and [32+16j, 48+16j) of the 64-K step, and
// supplies the scale of row m's 32-block j; the MFMA-ready scale word of a row
// holds the 4 blocks of a 128-K stage, so lane group j shifts it by 8j bytes and
// selects byte 2s for K-step s.
// NVFP4: E2M1 x E4M3 products have at most 6 significant bits and exponents in
// [2^-10, 2688], so a pass before the GEMM expands both operands exactly to bf16 in the
// same 64-byte panels and the GEMM runs on V_MFMA_F32_32X32X16_BF16; the per-group global
// scales multiply the fp32 result.  (The block-scaled MFMA takes E8M0 scales per 32
// elements; NVFP4's E4M3 scales per 16 cannot be folded into it exactly.)
#include "activation.h"
#include "device_common.h"
#include "kernels.h"

#include <algorithm>

namespace gmlp {

constexpr int BM = 256, BN = 256;
constexpr int NTHREADS = 256;
// A ring of 4 stages of 64 K (one MFMA K-step), 3 in flight while one is computed.
constexpr int MX_BK = 64;
constexpr int MX_OPB = BM * MX_BK;               // 16 KB per operand
constexpr int MX_SC_OFF = 2 * MX_OPB;            // scale words: A [256] then B [256] (u32)
constexpr int MX_STAGE = 2 * MX_OPB + 2048;      // 34 KB
constexpr int MX_NSTAGE = 4;
constexpr int MX_DMA_PER_STAGE = 9;              // per wave: 4 A + 4 B data DMAs + 1 scale-word DMA

// Wave-uniform copies (the values are uniform by construction; this tells the compiler so
// that descriptors and bases live in SGPRs).
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uni(int64_t v) {
  const uint64_t u = (uint64_t)v;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
// A copy of a uniform value that the compiler cannot see through: derived addresses are then
// computed where they are used instead of being hoisted out of the tile loop (where they
// would stay live, and spill, across the whole main loop).
__device__ __forceinline__ int64_t opaque(int64_t v) {
  asm volatile("" : "+s"(v));
  return v;
}
template <class T>
__device__ __forceinline__ T* uni_ptr(T* p) { return reinterpret_cast<T*>(uni((int64_t)reinterpret_cast<uintptr_t>(p))); }
// 64-byte rows (MXFP8 stages): four rows share a 256-byte bank line, so the chunk is XORed
// with (row >> 2) & 3; 16 consecutive rows then cover all 16 bank groups.
__device__ __forceinline__ int swz64(int row, int chunk) { return row * MX_BK + ((chunk ^ ((row >> 2) & 3)) << 4); }

// ----------------------------------------------------------------------------- tile context
struct Ctx {
  int g;             // group / expert
  int64_t arow0;     // FPROP: first global row of the tile; WGRAD: first A feature row
  int arows;         // valid A rows in the tile
  int64_t nrow0;     // first output column (FPROP) / B feature row (WGRAD)
  int nt;            // n-tile index
  int64_t kvalid;    // contraction length (K, or the group's tokens)
  int nk;            // stages
  // operand bases (element offsets of row 0 of the operand matrix for this group)
  int64_t a_base, b_base, a_ld, b_ld;
  int64_t a_rtot, b_rtot;                           // MXFP8: rows per 64-byte K panel of A and B
  int64_t a_sw_base, b_sw_base, a_sw_ld, b_sw_ld;   // MXFP8 scale words: base + kt * ld + row
  float alpha;
};

// ----------------------------------------------------------------------------- stage loads
// MXFP8: direct buffer -> LDS DMA (buffer_load_dwordx4 ... lds).  One instruction moves a
// wave's 64 x 16 bytes into 1 KB of LDS (lane l lands at +16 l), i.e. 16 rows of a 64-K
// stage; each lane fetches the logical chunk that the swizzle places at its slot.
// Wave w loads A rows and B rows [64 w, 64 w + 64) of the tile through one buffer resource
// each, whose size ends at the last valid row: rows past it read as zero (hardware range
// check), so partial tiles need no clamping and every lane keeps one 32-bit offset.
constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw buffer, 32-bit data format (gfx9 family)

// Buffer descriptor {base, stride 0, num_records, format}: loads at offsets >= num_records
// return zero (hardware range check).
struct Rsrc {
  v4i w;
};
__device__ __forceinline__ Rsrc make_rsrc(const void* base, int64_t bytes) {
  const uint64_t a = (uint64_t)uni((int64_t)reinterpret_cast<uintptr_t>(base));
  const int32_t n = (int32_t)(bytes < 0 ? 0 : (bytes > 0x7FFFFFFF ? 0x7FFFFFFF : bytes));
  Rsrc r;
  r.w = v4i{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xFFFFu), uni(n), (int)kRsrcWord3};
  return r;
}

// One buffer -> LDS DMA of 16 bytes per active lane: lane l's bytes land at lds + 16 l.  Issued
// through inline asm so that the compiler's wait-count pass does not treat it as a pending
// LDS write (it would otherwise wait for every outstanding DMA before any LDS read); the
// kernel accounts for these loads itself with explicit vmcnt waits.
__device__ __forceinline__ void dma16(const Rsrc& r, uint32_t voff, const uint8_t* lds) {
  const uint32_t m0 = (uint32_t)(uintptr_t)lds;          // low 32 bits of a shared address = LDS offset
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :: "v"(voff), "s"(r.w), "s"(__builtin_amdgcn_readfirstlane(m0)) : "memory");
}

// The same with an instruction offset, which moves the global and the LDS address alike: the
// four 1 KB instructions of one 64-row band share one M0 and one lane offset.
template <int OFF>
__device__ __forceinline__ void dma16_at(const Rsrc& r, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen offset:%3 lds"
               :: "v"(voff), "s"(r.w), "s"(m0), "i"(OFF) : "memory");
}

// Persistent kernel DMAs: the per-stage offset can go in SOFFSET, and M0 is written once per band:
// the A band's four instructions run back to back on one M0, then the B band's, then the scale
// words' (nothing else in the kernel uses M0).
template <int OFF>
__device__ __forceinline__ void dma_set_m0(const Rsrc& r, uint32_t voff, uint32_t soff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen offset:%4 lds"
               :: "v"(voff), "s"(r.w), "s"(soff), "s"(m0), "i"(OFF) : "memory");
}
template <int OFF>
__device__ __forceinline__ void dma_same_m0(const Rsrc& r, uint32_t voff, uint32_t soff) {
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen offset:%3 lds" :: "v"(voff), "s"(r.w), "s"(soff), "i"(OFF)
               : "memory");
}

// s_waitcnt with only the vector-memory counter: vmcnt <= n (expcnt, lgkmcnt untouched).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// MXFP8 operands are stored in 64-byte K panels: byte (r, k) of an R-row operand sits at
// ((k / 64) R + r) 64 + k % 64, so one stage of a 64-row band is 4 KB of contiguous memory
// and every DMA instruction reads 16 whole rows (1 KB, 8 full cache lines).
struct DmaPlan {
  const uint8_t* a0;               // this wave's A band, panel 0
  const uint8_t* b0;               // this wave's B band, panel 0
  int64_t a_pstride, b_pstride;    // bytes per panel (R x 64)
  int32_t a_bytes, b_bytes;        // valid rows of the band x 64: the resource range
  uint32_t lane_off;               // (lane / 4) 64 + 16 x logical chunk
};

// Stage kt (64 K): wave w fetches A and B rows [64 w, 64 w + 64) (4 + 4 DMAs) and one 1 KB DMA
// of MFMA scale words for the stage's 128-K word: waves 0 and 2 the 256 A rows' words, waves 1
// and 3 the 256 B rows' words (waves 2 and 3 repeat the same bytes).  Every wave issues the
// same 9 DMAs per stage, so one vmcnt bound serves all waves; a stage past the end (live ==
// false) is issued with empty resources so that the count stays the same without a branch.
struct StageDma {
  Rsrc ra, rb, rs;       // the stage's A band, B band and scale words
  uint32_t s_voff;
  uint8_t* lds;          // the stage's slot
  uint32_t s_lds;        // scale-word destination offset in the slot
  uint32_t m0a, m0b, m0s;  // LDS destinations (M0) of this wave's A band, B band and scale words
  uint32_t soa, sob, sos;  // SOFFSET of the three resources (0 unless the resource is a tile's)
};
__device__ __forceinline__ void stage_m0(StageDma& s, int wave) {
  const uint32_t base = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)s.lds);
  s.m0a = base + 4096u * (uint32_t)wave;
  s.m0b = base + MX_OPB + 4096u * (uint32_t)wave;
  s.m0s = base + s.s_lds;
}

// A tile of the persistent kernel, reduced to what fixes its DMA sources and its epilogue.
struct TileRef {
  int32_t nk;                // 64-K stages; 0: no tile
  int32_t arows;             // valid A rows in the tile
  int64_t arow0;             // FPROP: first global row; WGRAD: first A feature row
  int32_t g, nt;             // expert / group, n-tile
  int32_t off, woff;         // WGRAD: the group's padded token offset and 128-token word offset
};

// Field-wise uniform select (keeps both operands in scalar registers).
__device__ __forceinline__ TileRef sel_ref(bool c, const TileRef& a, const TileRef& b) {
  TileRef r;
  r.nk = c ? a.nk : b.nk;
  r.arows = c ? a.arows : b.arows;
  r.arow0 = c ? a.arow0 : b.arow0;
  r.g = c ? a.g : b.g;
  r.nt = c ? a.nt : b.nt;
  r.off = c ? a.off : b.off;
  r.woff = c ? a.woff : b.woff;
  return r;
}

// The per-wave DMA sources of a tile, as 32-bit offsets from the operands' bases (the launch
// keeps every operand below 4 GB): six scalars, so that three of them fit the scalar registers.
struct DmaTile {
  uint32_t a_off, b_off;     // bytes: this wave's A / B band in panel 0
  uint32_t s_off;            // words: this wave's scale words (A or B rows) of the first 128-K word
  uint32_t ab_bytes;         // resource ranges of the A and B bands (low / high 16 bits)
  uint32_t s_bytes;          // resource range of the scale words
  int32_t nk;                // 64-K stages; 0: no tile
};
// Per-launch constants of the DMA sources.
struct DmaConst {
  const uint8_t* a;          // operand bases
  const uint8_t* b;
  const uint32_t* s;         // this wave's scale-word base (A or B)
  uint32_t a_ps, b_ps;       // bytes per 64-K panel
  uint32_t s_ld;             // words per 128-K word
  uint32_t a_total, b_total, s_total;   // bytes of the operands and of this wave's scale words
};

// Field-wise uniform select (scalar selects, no branch).
__device__ __forceinline__ DmaTile sel_tile(bool c, const DmaTile& a, const DmaTile& b) {
  DmaTile r;
  r.a_off = c ? a.a_off : b.a_off;
  r.b_off = c ? a.b_off : b.b_off;
  r.s_off = c ? a.s_off : b.s_off;
  r.ab_bytes = c ? a.ab_bytes : b.ab_bytes;
  r.s_bytes = c ? a.s_bytes : b.s_bytes;
  r.nk = c ? a.nk : b.nk;
  return r;
}

// BF: bf16 operands (2 bytes per element in the same 64-byte panels, no scale words: their
// DMA keeps its slot with an empty resource, which reads nothing and lands zeros).
template <int MODE, int EPI, int BF = 0>
__device__ __forceinline__ DmaConst dma_const(const GemmArgs& A, int wave) {
  constexpr int64_t EB = BF ? 2 : 1;
  DmaConst k;
  k.a = A.a.data;
  k.b = A.b.data;
  k.s = (wave & 1) ? A.b.scale_mfma : A.a.scale_mfma;
  if (MODE == MODE_FPROP) {
    const int64_t brows = A.N;
    const int64_t kw = (A.K + 127) / 128;
    k.a_ps = (uint32_t)(A.M * 64);
    k.b_ps = (uint32_t)(brows * 64);
    k.s_ld = (uint32_t)((wave & 1) ? brows : A.M);
    k.a_total = (uint32_t)(EB * A.M * A.K);
    k.b_total = (uint32_t)(EB * A.G * brows * A.K);
    k.s_total = BF ? 0u : (uint32_t)(4 * kw * ((wave & 1) ? A.G * brows : A.M));
  } else {
    const int64_t P = A.T.col_off[A.G], W = A.T.colw_off[A.G];
    k.a_ps = (uint32_t)(A.N * 64);
    k.b_ps = (uint32_t)(A.K * 64);
    k.s_ld = (uint32_t)((wave & 1) ? A.K : A.N);
    k.a_total = (uint32_t)(EB * A.N * P);
    k.b_total = (uint32_t)(EB * A.K * P);
    k.s_total = BF ? 0u : (uint32_t)(4 * W * ((wave & 1) ? A.K : A.N));
  }
  return k;
}

template <int MODE, int EPI, int BF = 0>
__device__ __forceinline__ DmaTile dma_tile(const GemmArgs& A, const TileRef& r, int wave) {
  constexpr int64_t EB = BF ? 2 : 1;
  DmaTile t;
  const int64_t nb = (MODE == MODE_FPROP) ? A.N : A.K;
  const int64_t b_first = (int64_t)r.nt * BN + 64 * wave;
  const int64_t b_rows = min((int64_t)64, max((int64_t)0, nb - b_first));
  const int64_t a_rows = min(64, max(0, r.arows - 64 * wave));
  int64_t a_base, b_base, a_sw, b_sw;
  if (MODE == MODE_FPROP) {
    const int64_t brows = A.N;
    a_base = 0;
    a_sw = 0;
    b_base = EB * (int64_t)r.g * brows * A.K;
    b_sw = (int64_t)r.g * ((A.K + 127) / 128) * brows;
  } else {
    a_base = A.N * (int64_t)r.off;
    a_sw = A.N * (int64_t)r.woff;
    b_base = A.K * (int64_t)r.off;
    b_sw = A.K * (int64_t)r.woff;
  }
  t.a_off = (uint32_t)(a_base + (r.arow0 + 64 * wave) * 64);
  t.b_off = (uint32_t)(b_base + b_first * 64);
  t.ab_bytes = (uint32_t)(a_rows * 64) | ((uint32_t)(b_rows * 64) << 16);
  if ((wave & 1) == 0) {
    t.s_off = (uint32_t)(a_sw + r.arow0);
    t.s_bytes = (uint32_t)(4 * r.arows);
  } else {
    const int64_t n0 = (int64_t)r.nt * BN;
    t.s_off = (uint32_t)(b_sw + n0);
    t.s_bytes = (uint32_t)(4 * max((int64_t)0, nb - n0));
  }
  if (BF) t.s_bytes = 0;
  t.nk = r.nk;
  return t;
}

// Stage k of tile t into slot `stage` (empty resources when k is past the tile's stages).
__device__ __forceinline__ StageDma dma_tile_stage(const DmaConst& K, const DmaTile& t, int k, uint8_t* stage,
                                                   uint32_t s_voff, int wave) {
  StageDma s;
  const bool live = k < t.nk;
  s.lds = stage;
  s.ra = make_rsrc(K.a + t.a_off + (uint64_t)k * K.a_ps, live ? (t.ab_bytes & 0xFFFFu) : 0);
  s.rb = make_rsrc(K.b + t.b_off + (uint64_t)k * K.b_ps, live ? (t.ab_bytes >> 16) : 0);
  s.rs = make_rsrc(K.s + t.s_off + (uint64_t)(k >> 1) * K.s_ld, live ? t.s_bytes : 0);
  s.s_voff = s_voff;
  s.s_lds = MX_SC_OFF + ((wave & 1) ? 1024 : 0);
  s.soa = s.sob = s.sos = 0;
  stage_m0(s, wave);
  return s;
}

// A stage of the current tile from running source addresses (the common case: no selection).
// Interior stages of a tile: three resources fixed for the tile (its bands in panel 0) and the
// stage offset in SOFFSET.  SOFFSET counts in the range check, so these resources reach to the
// end of the operand: rows past a partial band's valid ones are then read from the neighbouring
// rows instead of as zeros.  They only feed output rows and columns past the tile's valid
// range, which are never stored (the MFMA rows and columns are independent); the buffer end
// still bounds every access.
struct RunDma {
  Rsrc ra, rb, rs;
};
__device__ __forceinline__ uint32_t rest(uint32_t total, uint32_t off) { return total > off ? total - off : 0u; }
__device__ __forceinline__ RunDma run_rsrc(const DmaConst& K, const DmaTile& t) {
  RunDma r;
  const uint64_t pa = (uint64_t)(uintptr_t)K.a + t.a_off;
  const uint64_t pb = (uint64_t)(uintptr_t)K.b + t.b_off;
  const uint64_t ps = (uint64_t)(uintptr_t)(K.s + t.s_off);
  auto word = [](uint32_t v) { return __builtin_amdgcn_readfirstlane((int)v); };   // uniform: scalar registers
  // a band with no valid row (past a partial tile's rows or columns) reads nothing
  const uint32_t na = (t.ab_bytes & 0xFFFFu) ? rest(K.a_total, t.a_off) : 0u;
  const uint32_t nbb = (t.ab_bytes >> 16) ? rest(K.b_total, t.b_off) : 0u;
  r.ra.w = v4i{word((uint32_t)pa), word((uint32_t)(pa >> 32) & 0xFFFFu), word(na), (int)kRsrcWord3};
  r.rb.w = v4i{word((uint32_t)pb), word((uint32_t)(pb >> 32) & 0xFFFFu), word(nbb), (int)kRsrcWord3};
  r.rs.w = v4i{word((uint32_t)ps), word((uint32_t)(ps >> 32) & 0xFFFFu), word(rest(K.s_total, 4 * t.s_off)),
               (int)kRsrcWord3};
  return r;
}
__device__ __forceinline__ StageDma run_stage(const RunDma& r, uint32_t soa, uint32_t sob, uint32_t sos, uint8_t* stage,
                                              uint32_t s_voff, int wave) {
  StageDma s;
  s.lds = stage;
  s.ra = r.ra;
  s.rb = r.rb;
  s.rs = r.rs;
  s.soa = (uint32_t)__builtin_amdgcn_readfirstlane((int)soa);
  s.sob = (uint32_t)__builtin_amdgcn_readfirstlane((int)sob);
  s.sos = (uint32_t)__builtin_amdgcn_readfirstlane((int)sos);
  s.s_voff = s_voff;
  s.s_lds = MX_SC_OFF + ((wave & 1) ? 1024 : 0);
  stage_m0(s, wave);
  return s;
}

// DMA number I (0..8) of a stage: I < 4 an A instruction, 4 <= I < 8 a B instruction, 8 the
// scale words.
template <int I>
__device__ __forceinline__ void mx_dma_one(const StageDma& s, const DmaPlan& d, int wave) {
  if constexpr (I == 0) dma_set_m0<0>(s.ra, d.lane_off, s.soa, s.m0a);
  else if constexpr (I < 4) dma_same_m0<1024 * I>(s.ra, d.lane_off, s.soa);
  else if constexpr (I == 4) dma_set_m0<0>(s.rb, d.lane_off, s.sob, s.m0b);
  else if constexpr (I < 8) dma_same_m0<1024 * (I - 4)>(s.rb, d.lane_off, s.sob);
  else dma_set_m0<0>(s.rs, s.s_voff, s.sos, s.m0s);
}

// ----------------------------------------------------------------------------- MFMA stage
// Fragments of one stage for one wave, read from LDS into registers before the next stage's DMA
// is issued (the compiler cannot prove that the DMA target and the buffer being read differ,
// so any LDS read after a DMA would wait for the DMA to land).
struct MxFrags {
  v8i a[4], b[4];              // one 64-K step
  uint32_t sa[4], sb[4];       // E8M0 scale of this lane's 32-block in byte 0
};

// Per-lane byte offsets of the fragment reads within a stage slot.  Tile t of a fragment adds
// the constant 2048 t (32 rows of 64 bytes: the swizzle term (row / 4) % 4 is the same), so
// each read is one of six per-step bases plus an immediate offset.
struct ReadPlan {
  uint32_t a0, a1, b0, b1;   // K bytes [16 j, 16 j + 16) and [32 + 16 j, ...) of A / B row (128 wm|wn + m)
  uint32_t sa, sb;           // scale bytes j of the row words (the step parity adds 2)
};
__device__ __forceinline__ ReadPlan make_read_plan(int wm, int wn, int lane) {
  const int m = lane & 31, j = lane >> 5;
  ReadPlan r;
  r.a0 = (uint32_t)swz64(wm * 128 + m, j);
  r.a1 = (uint32_t)swz64(wm * 128 + m, 2 + j);
  r.b0 = (uint32_t)(MX_OPB + swz64(wn * 128 + m, j));
  r.b1 = (uint32_t)(MX_OPB + swz64(wn * 128 + m, 2 + j));
  r.sa = (uint32_t)(MX_SC_OFF + j + 4 * (wm * 128 + m));
  r.sb = (uint32_t)(MX_SC_OFF + 1024 + j + 4 * (wn * 128 + m));
  return r;
}
template <int T, int PAR, int BF = 0>
__device__ __forceinline__ void mx_read_tp(const uint8_t* stage, const ReadPlan& r, MxFrags& f) {
  const uint4 x0 = *reinterpret_cast<const uint4*>(stage + r.a0 + 2048 * T);
  const uint4 x1 = *reinterpret_cast<const uint4*>(stage + r.a1 + 2048 * T);
  const uint4 y0 = *reinterpret_cast<const uint4*>(stage + r.b0 + 2048 * T);
  const uint4 y1 = *reinterpret_cast<const uint4*>(stage + r.b1 + 2048 * T);
  f.a[T] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
  f.b[T] = v8i{(int)y0.x, (int)y0.y, (int)y0.z, (int)y0.w, (int)y1.x, (int)y1.y, (int)y1.z, (int)y1.w};
  if constexpr (!BF) {
    f.sa[T] = stage[r.sa + 2 * PAR + 128 * T];
    f.sb[T] = stage[r.sb + 2 * PAR + 128 * T];
  }
}
template <int PAR, int BF = 0>
__device__ __forceinline__ void mx_read_p(const uint8_t* stage, const ReadPlan& r, MxFrags& f) {
  mx_read_tp<0, PAR, BF>(stage, r, f);
  mx_read_tp<1, PAR, BF>(stage, r, f);
  mx_read_tp<2, PAR, BF>(stage, r, f);
  mx_read_tp<3, PAR, BF>(stage, r, f);
}

// bf16 operands (NVFP4 expanded exactly) travel in the same 64-byte stage rows: a lane's 32
// fragment bytes are K elements [8 j, 8 j + 8) and [16 + 8 j, 24 + 8 j) of the stage's 32, which
// are exactly its operands of two 32x32x16 bf16 MFMAs (elements 0..15, then 16..31).
__device__ __forceinline__ v8bf frag_lo(const v8i& v) { return __builtin_bit_cast(v8bf, v4i{v[0], v[1], v[2], v[3]}); }
__device__ __forceinline__ v8bf frag_hi(const v8i& v) { return __builtin_bit_cast(v8bf, v4i{v[4], v[5], v[6], v[7]}); }

// Z: the tile's first step, which starts the accumulators from zero (the MFMA's C operand is the
// constant 0, so no register has to be cleared between tiles).
// TR: the transposed product (B fragments as the MFMA's first operand, with their scales), so that
// a lane's accumulators hold consecutive output columns of one row (see mx_epilogue_tr).
template <int TM, int TN, int BF = 0, bool Z = false, int TR = 0>
__device__ __forceinline__ void mx_mma_one(const MxFrags& f, v16f (&acc)[4][4]) {
  const v16f c = Z ? v16f{} : acc[TM][TN];
  if constexpr (BF) {
    if constexpr (TR) {
      acc[TM][TN] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_lo(f.b[TN]), frag_lo(f.a[TM]), c, 0, 0, 0);
      acc[TM][TN] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_hi(f.b[TN]), frag_hi(f.a[TM]), acc[TM][TN], 0, 0, 0);
    } else {
      acc[TM][TN] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_lo(f.a[TM]), frag_lo(f.b[TN]), c, 0, 0, 0);
      acc[TM][TN] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_hi(f.a[TM]), frag_hi(f.b[TN]), acc[TM][TN], 0, 0, 0);
    }
  } else if constexpr (TR) {
    acc[TM][TN] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.b[TN], f.a[TM], c, 0, 0, 0,
                                                                   (int)f.sb[TN], 0, (int)f.sa[TM]);
  } else {
    acc[TM][TN] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[TM], f.b[TN], c, 0, 0, 0,
                                                                   (int)f.sa[TM], 0, (int)f.sb[TN]);
  }
}

#define GMLP_SB() __builtin_amdgcn_sched_barrier(0)

// One step's instruction order.  The 9 DMAs of the stage three ahead are spread over the 16
// MFMAs (one per 64-cycle MFMA pair at most), so that the address unit's queue, shared by the
// four waves, is fed at the rate it drains: a wave whose DMA waits for room stalls under a
// running MFMA instead of holding back a block of them.  The reads of the next stage are
// spread over the second half.
//   before the barrier: D0 M00 M01 D1 M02 M03 D2 M10 M11 D3 M12 M13 D4
//   after the barrier:  R0 M20 D5 R1 M21 M22 D6 R2 M23 M30 D7 R3 M31 M32 D8 M33
constexpr int MX_DMA_BEFORE_BARRIER = 5;

template <int BF = 0, bool Z = false, int TR = 0>
__device__ __forceinline__ void mx_phase1(const MxFrags& f, v16f (&acc)[4][4], const StageDma& s, const DmaPlan& d,
                                          int wave) {
  mx_dma_one<0>(s, d, wave); GMLP_SB();
  mx_mma_one<0, 0, BF, Z, TR>(f, acc); GMLP_SB(); mx_mma_one<0, 1, BF, Z, TR>(f, acc); GMLP_SB();
  mx_dma_one<1>(s, d, wave); GMLP_SB();
  mx_mma_one<0, 2, BF, Z, TR>(f, acc); GMLP_SB(); mx_mma_one<0, 3, BF, Z, TR>(f, acc); GMLP_SB();
  mx_dma_one<2>(s, d, wave); GMLP_SB();
  mx_mma_one<1, 0, BF, Z, TR>(f, acc); GMLP_SB(); mx_mma_one<1, 1, BF, Z, TR>(f, acc); GMLP_SB();
  mx_dma_one<3>(s, d, wave); GMLP_SB();
  mx_mma_one<1, 2, BF, Z, TR>(f, acc); GMLP_SB(); mx_mma_one<1, 3, BF, Z, TR>(f, acc); GMLP_SB();
  mx_dma_one<4>(s, d, wave); GMLP_SB();
}

template <int PAR, int BF = 0, bool Z = false, int TR = 0>
__device__ __forceinline__ void mx_phase2p(const MxFrags& f, v16f (&acc)[4][4], const StageDma& s, const DmaPlan& d,
                                           int wave, const uint8_t* nstage, const ReadPlan& rp, MxFrags& nf) {
  mx_read_tp<0, PAR, BF>(nstage, rp, nf); GMLP_SB();
  mx_mma_one<2, 0, BF, Z, TR>(f, acc); GMLP_SB();
  mx_dma_one<5>(s, d, wave); GMLP_SB();
  mx_read_tp<1, PAR, BF>(nstage, rp, nf); GMLP_SB();
  mx_mma_one<2, 1, BF, Z, TR>(f, acc); GMLP_SB(); mx_mma_one<2, 2, BF, Z, TR>(f, acc); GMLP_SB();
  mx_dma_one<6>(s, d, wave); GMLP_SB();
  mx_read_tp<2, PAR, BF>(nstage, rp, nf); GMLP_SB();
  mx_mma_one<2, 3, BF, Z, TR>(f, acc); GMLP_SB(); mx_mma_one<3, 0, BF, Z, TR>(f, acc); GMLP_SB();
  mx_dma_one<7>(s, d, wave); GMLP_SB();
  mx_read_tp<3, PAR, BF>(nstage, rp, nf); GMLP_SB();
  mx_mma_one<3, 1, BF, Z, TR>(f, acc); GMLP_SB(); mx_mma_one<3, 2, BF, Z, TR>(f, acc); GMLP_SB();
  mx_dma_one<8>(s, d, wave); GMLP_SB();
  mx_mma_one<3, 3, BF, Z, TR>(f, acc); GMLP_SB();
}

// ----------------------------------------------------------------------------- tile mapping
template <int MODE, int EPI>
__device__ __forceinline__ int tiles_n(const GemmArgs& A) {
  if (MODE == MODE_FPROP)
    return (int)((A.N + BN - 1) / BN);
  return (int)((A.K + BN - 1) / BN);
}

// Stages of a weight-gradient tile over `tokens` tokens at `eb` bytes per token (64-byte stage
// rows): the stages that hold a token, at least 2 for a non-empty group (the persistent kernel's
// DMA window of three tiles needs every tile to span two stages), 0 for an empty one.
__device__ __forceinline__ int wgrad_stages(int64_t tokens, int eb) {
  return tokens > 0 ? (int)max((int64_t)2, (eb * tokens + 63) / 64) : 0;
}

// Context of tile bid of an ntm x ntn tile grid.
template <int MODE, int EPI>
__device__ __forceinline__ bool tile_ctx(const GemmArgs& A, int bid, int ntm, int ntn, int& mt, Ctx& c) {
  // Order: groups of group_rows tile rows, column-major inside a group, so that the
  // workgroups resident together on one XCD share few A row blocks and B blocks.  WGRAD tiles,
  // and FPROP tiles when expert_groups is set, are ordered expert by expert (the row groups stay
  // inside one expert), so that an expert's tiles are one contiguous range of the sequence and
  // a group's column tiles share one weight panel.
  const int gr = A.group_rows;
  const int gsz = gr * ntn;
  int tile_m;
  if (MODE == MODE_WGRAD) {
    const int per_g = (int)((A.N + BM - 1) / BM);
    const int tpg = per_g * ntn;
    const int e = bid / tpg, loc = bid - e * tpg;
    const int grp = loc / gsz, rem = loc - grp * gsz;
    const int rows_here = min(gr, per_g - grp * gr);
    tile_m = e * per_g + grp * gr + rem % rows_here;
    c.nt = rem / rows_here;
  } else if (A.expert_groups) {
    // expert e's tiles: [t256_off[e] ntn, t256_off[e + 1] ntn) of the sequence
    if (A.G <= 0 || bid >= ntm * ntn) return false;
    const int e = find_group(A.T.t256_off, A.G, bid / ntn);
    const int r0 = A.T.t256_off[e], r = A.T.t256_off[e + 1] - r0;
    const int loc = bid - r0 * ntn;
    const int grp = loc / gsz, rem = loc - grp * gsz;
    const int rows_here = min(gr, r - grp * gr);
    tile_m = r0 + grp * gr + rem % rows_here;
    c.nt = rem / rows_here;
  } else {
    const int grp = bid / gsz, rem = bid - grp * gsz;
    const int rows_here = min(gr, ntm - grp * gr);
    tile_m = grp * gr + rem % rows_here;
    c.nt = rem / rows_here;
  }
  c.alpha = 1.0f;
  if (MODE == MODE_FPROP) {
    if (A.G <= 0 || tile_m >= A.T.t256_off[A.G]) return false;
    c.g = find_group(A.T.t256_off, A.G, tile_m);
    const int64_t gstart = A.T.row_off[c.g];
    const int m = A.T.row_off[c.g + 1] - (int)gstart;
    mt = tile_m - A.T.t256_off[c.g];
    c.arow0 = gstart + (int64_t)mt * BM;
    c.arows = min(BM, m - mt * BM);
    c.nrow0 = (int64_t)c.nt * BN;
    c.kvalid = A.K;
    c.a_base = 0;
    c.a_ld = A.K;
    // B rows per expert; weight scale words are per expert: [E][ceil(K/128)][brows]
    const int64_t brows = A.N;
    c.b_base = (int64_t)c.g * brows * A.K;
    c.b_ld = A.K;
    c.a_rtot = A.M;
    c.b_rtot = brows;
    c.a_sw_base = 0;
    c.a_sw_ld = A.M;
    c.b_sw_base = (int64_t)c.g * ((A.K + 127) / 128) * brows;
    c.b_sw_ld = brows;
    c.nk = (int)((A.K + 63) / 64);              // 64-K stages (both formats)
  } else {
    const int ntm = (int)((A.N + BM - 1) / BM);
    const int per_g = ntm;
    c.g = tile_m / per_g;
    if (c.g >= A.G) return false;
    mt = tile_m % per_g;
    // the column-wise operands hold P tokens per group (the group's tokens padded with zeros to
    // a multiple of 128); the stages stop at the last 64 (32 for bf16) that hold a token, but a
    // tile keeps at least 2 (wgrad_stages)
    const int64_t P = A.T.col_off[c.g + 1] - A.T.col_off[c.g];
    const int64_t tokens = min((int64_t)(A.T.row_off[c.g + 1] - A.T.row_off[c.g]), P);
    c.arow0 = (int64_t)mt * BM;
    c.arows = (int)min((int64_t)BM, A.N - c.arow0);
    c.nrow0 = (int64_t)c.nt * BN;
    c.kvalid = tokens;
    c.a_base = A.N * (int64_t)A.T.col_off[c.g];
    c.a_ld = P;
    c.b_base = A.K * (int64_t)A.T.col_off[c.g];
    c.b_ld = P;
    c.a_rtot = A.N;
    c.b_rtot = A.K;
    c.a_sw_base = A.N * (int64_t)A.T.colw_off[c.g];
    c.a_sw_ld = A.N;
    c.b_sw_base = A.K * (int64_t)A.T.colw_off[c.g];
    c.b_sw_ld = A.K;
    c.nk = wgrad_stages(tokens, 1);
  }
  return true;
}

// ----------------------------------------------------------------------------- dprob reduce
// ----------------------------------------------------------------------------- persistent MXFP8 kernel
// One workgroup per CU walks a list of tiles.  The 64-K stages of its non-empty tiles form one
// sequence that flows through the 4-slot ring without a break: while a tile's last steps run,
// the DMAs already fetch the first stages of the next tiles, so neither the pipeline fill nor
// the epilogue's stores stall the matrix cores between tiles.  The epilogue stages its output
// through the one ring slot that holds no pending stage (that of the last stage consumed), in
// row chunks of at most 32 KB.
//
// Tile list: XCD x = blockIdx % 8 owns the contiguous tile range [x T / 8, (x + 1) T / 8) of
// the T valid tiles and its workgroups take them in lockstep (tile lo + l, lo + l + n, ...),
// so the tiles resident together on an XCD are neighbours in the group order of tile_ctx.

// fp32-staged epilogue (fp32 outputs, the fused amax): the 256 x 256 fp32 tile leaves the
// accumulators in 8 chunks of 64 rows x 128 columns (32 KB, one ring slot).  Chunk ch holds
// MFMA tile row tm = ch / 2 of both wave halves (staged row sr -> tile row chunk_row(tm, sr))
// and two of each wave's four MFMA column tiles: tn = 2 q, 2 q + 1 (q = ch % 2), so that every
// output row segment a chunk stores is a whole 128-byte line (half-line streaming stores cost
// about twice as much).  The accumulators are written to LDS straight from the accumulator
// registers (inline ds_write_b32 with an AGPR operand), so they are never copied to vector
// registers.
__device__ __forceinline__ int chunk_row(int tm, int sr) { return ((sr >> 5) << 7) + 32 * tm + (sr & 31); }
constexpr int EPC_LD = 136;        // floats per staged row: rows 4 apart are 32 banks apart

template <int OFF>
__device__ __forceinline__ void lds_write_acc(uint32_t addr, float v) {
  asm volatile("ds_write_b32 %0, %1 offset:%2" :: "v"(addr), "a"(v), "i"(OFF) : "memory");
}
__device__ __forceinline__ void lds_writes_done() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Stage chunk ch: wave (wm, wn) writes acc[tm][tn0 + d tn1] (d = 0, 1) at staged rows
// 32 wm + (r / 4) 8 + 4 j + r % 4, staged columns 64 wn + 32 d + m.
#define GMLP_W(D, TN, R) lds_write_acc<((8 * ((R) >> 2) + ((R) & 3)) * EPC_LD + 32 * (D)) * 4>(base, acc[TM][TN][R]);
#define GMLP_W16(D, TN) GMLP_W(D, TN, 0) GMLP_W(D, TN, 1) GMLP_W(D, TN, 2) GMLP_W(D, TN, 3) GMLP_W(D, TN, 4) \
  GMLP_W(D, TN, 5) GMLP_W(D, TN, 6) GMLP_W(D, TN, 7) GMLP_W(D, TN, 8) GMLP_W(D, TN, 9) GMLP_W(D, TN, 10)          \
  GMLP_W(D, TN, 11) GMLP_W(D, TN, 12) GMLP_W(D, TN, 13) GMLP_W(D, TN, 14) GMLP_W(D, TN, 15)
template <int TM, int TN0, int TN1>
__device__ __forceinline__ void stage_chunk(const v16f (&acc)[4][4], uint32_t base) {
  // base = LDS byte address of staged (32 wm + 4 j, 64 wn + m)
  GMLP_W16(0, TN0)
  GMLP_W16(1, TN1)
  lds_writes_done();
}
#undef GMLP_W16
#undef GMLP_W

// Output stores of the persistent kernel: one buffer resource per output matrix and tile, based
// at the tile's first row and column and sized to its valid rows, so that the rows past the
// last token fall outside the range and are dropped by the hardware check; a lane whose columns
// lie past the matrix gets an offset beyond the range.  The row of each store goes in SOFFSET.
// Stores stream past the L2 (nontemporal): the output is not read again by this kernel, and
// keeping it out of the cache leaves the L2 to the operand panels.
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kStoreNT = 2;                       // aux bits of a nontemporal buffer store

__device__ __forceinline__ __amdgpu_buffer_rsrc_t out_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)(uint32_t)bytes, (int)kRsrcWord3);
}
__device__ __forceinline__ uint4 out_load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  typedef uint32_t v4u __attribute__((ext_vector_type(4)));
  const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void out_store(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint32_t x,
                                          uint32_t y, uint32_t z, uint32_t w) {
  typedef uint32_t v4u __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128((v4u){x, y, z, w}, r, voff, soff, kStoreNT);
}

// A staged fp32 quad, times the group's scale for NVFP4 (bf16-expanded) operands.
template <int BF>
__device__ __forceinline__ float4 ld_st4(const float* p, float alpha) {
  float4 v = *reinterpret_cast<const float4*>(p);
  if constexpr (BF != 0) {
    v.x = __fmul_rn(v.x, alpha);
    v.y = __fmul_rn(v.y, alpha);
    v.z = __fmul_rn(v.z, alpha);
    v.w = __fmul_rn(v.w, alpha);
  }
  return v;
}

// A kernel argument read where it is used (a volatile load of the argument), so that the compiler
// does not keep it in a register across the main loop: the epilogue-only arguments would otherwise
// add to the main loop's scalar-register pressure.
template <class T>
__device__ __forceinline__ T* late_ptr(T* const& arg) {
  return *reinterpret_cast<T* const volatile*>(&arg);
}

// EPI_STORE_AMAX: the fc2-input amax of a staged chunk, read after the store loop (which only
// reads the staged values too, so no barrier is needed in between).  The chunk holds tile rows
// 32 TM + [0, 32) and 128 + 32 TM + [0, 32) (staged rows [0, 32) and [32, 64)): four whole
// 16-token blocks of the group, since tiles start at multiples of 256 rows from the group's first
// row; and 128 columns.  Thread tid takes the (block, column) pairs tid and tid + 256 (a wave's 64
// pairs share the block, so the token probabilities it reads from LDS are one address per wave):
// the column's 16 values as the stored bf16 h (the same fp32 product and rounding as the store),
// a = bf16(relu(h)^2 p) of each token with the function the standalone amax pass and the casts
// use, zeros for the rows past the group's end and the columns past N (the zero padding of the
// column-wise cast), then the signed Hadamard of the block.  pre / post: running maxima of |a|
// and of the unscaled |H16 (s * a)|.
template <int TM, int Q>
__device__ __forceinline__ void epi_chunk_amax(const GemmArgs& A, const Ctx& c, const float* st, const float* probs,
                                               int tid, uint32_t mask, float& pre, float& post) {
#pragma unroll 1
  for (int k = 0; k < 2; ++k) {
    const int p = tid + 256 * k;
    const int blk = p >> 7, sc = p & 127;
    const int col = 128 * (sc >> 6) + 64 * Q + (sc & 63);
    const bool col_ok = c.nrow0 + col < A.N;
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int sr = 16 * blk + i;
      const int tr = chunk_row(TM, sr);
      const bool ok = col_ok && tr < c.arows;
      const float h = round_bf16(__fmul_rn(st[sr * EPC_LD + sc], c.alpha));
      const float a = !ok ? 0.0f
                          : A.act.kind == ACT_TANH_SRELU ? act_out<ACT_TANH_SRELU>(h, 0.0f, probs[tr], A.act.c)
                                                         : act_out<ACT_SRELU>(h, 0.0f, probs[tr], A.act.c);
      pre = fmaxf(pre, fabsf(a));
      v[i] = a;
    }
    signed_fwht16(v, mask);
#pragma unroll
    for (int i = 0; i < 16; ++i) post = fmaxf(post, fabsf(v[i]));
  }
}

template <int MODE, int EPI, int CH, int BF = 0>
__device__ __forceinline__ void epi_chunk(const GemmArgs& A, const Ctx& c, const v16f (&acc)[4][4], uint8_t* buf,
                                          int tid, int wm, int wn, int lane, const float* probs, uint32_t mask,
                                          float& pre, float& post) {
  constexpr int TM = CH >> 1, Q = CH & 1;
  const float* st = reinterpret_cast<const float*>(buf);
  {
    const int m = lane & 31, j = lane >> 5;
    const uint32_t base = (uint32_t)(uintptr_t)buf + (uint32_t)(((32 * wm + 4 * j) * EPC_LD + m) * 4);
    stage_chunk<TM, 2 * Q, 2 * Q + 1>(acc, base + 256u * (uint32_t)wn);
  }
  __syncthreads();
  {
    // lanes [LPR r, LPR r + LPR) store staged row r of each group of RPI rows
    constexpr int ESZ = (EPI == EPI_STORE32 || EPI == EPI_ACC32) ? 4 : 2;
    constexpr int PER = 16 / ESZ;                 // output elements per 16-byte store
    constexpr int LPR = 128 / PER;
    constexpr int RPI = NTHREADS / LPR;
    constexpr int NIT = 64 / RPI;
    const int64_t ncols = (MODE == MODE_FPROP) ? A.N : A.K;
    const int64_t orow0 = (MODE == MODE_FPROP) ? c.arow0 : (int64_t)c.g * A.N + c.arow0;
    const uint32_t rowb = (uint32_t)(ncols * ESZ);
    const __amdgpu_buffer_rsrc_t r =
        out_rsrc(static_cast<uint8_t*>(A.c) + (orow0 * ncols + c.nrow0) * ESZ, (int64_t)c.arows * rowb);
    const int lrow = tid / LPR, sc = (tid % LPR) * PER;
    const int col = 128 * (sc >> 6) + 64 * Q + (sc & 63);
    const uint32_t voff = (c.nrow0 + col < ncols) ? (uint32_t)lrow * rowb + (uint32_t)(col * ESZ) : kOutOfRange;
    const float* src = st + lrow * EPC_LD + sc;
    // The staged values are all read before the first store: a buffer store may alias LDS as far
    // as the compiler knows, so a read placed after a store would wait for it and for its own
    // LDS latency, once per store.
    // EPI_ACC32 (C += tile): the chunk's old fp32 values are fetched first (one 16-byte load per
    // store, same offsets, so the range check drops the same lanes), then added in fp32.
    uint4 old[NIT];
    if constexpr (EPI == EPI_ACC32) {
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const uint32_t ur = (uint32_t)(128 * ((RPI * it) >> 5) + 32 * TM + ((RPI * it) & 31));
        old[it] = out_load(r, voff, ur * rowb);
      }
    }
    float4 v0[NIT], v1[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      v0[it] = ld_st4<BF>(src + RPI * it * EPC_LD, c.alpha);
      if constexpr (ESZ == 2) v1[it] = ld_st4<BF>(src + RPI * it * EPC_LD + 4, c.alpha);
    }
    if constexpr (EPI == EPI_ACC32) {
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const uint32_t ur = (uint32_t)(128 * ((RPI * it) >> 5) + 32 * TM + ((RPI * it) & 31));
        const float4 v = v0[it];
        out_store(r, voff, ur * rowb, __float_as_uint(__fadd_rn(__uint_as_float(old[it].x), v.x)),
                  __float_as_uint(__fadd_rn(__uint_as_float(old[it].y), v.y)),
                  __float_as_uint(__fadd_rn(__uint_as_float(old[it].z), v.z)),
                  __float_as_uint(__fadd_rn(__uint_as_float(old[it].w), v.w)));
      }
    } else {
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const uint32_t ur = (uint32_t)(128 * ((RPI * it) >> 5) + 32 * TM + ((RPI * it) & 31));   // tile row - lrow
        const float4 a = v0[it];
        if (EPI == EPI_STORE32) {
          out_store(r, voff, ur * rowb, __float_as_uint(a.x), __float_as_uint(a.y), __float_as_uint(a.z),
                    __float_as_uint(a.w));
        } else {
          const float4 b = v1[it];
          out_store(r, voff, ur * rowb, pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y),
                    pack_bf16x2(b.z, b.w));
        }
      }
    }
  }
  if constexpr (EPI == EPI_STORE_AMAX) epi_chunk_amax<TM, Q>(A, c, st, probs, tid, mask, pre, post);
  __syncthreads();
}

// Output tile of a group with no tokens (weight gradients only): zeros, stored directly (an
// accumulated gradient is left as it is).
template <int MODE, int EPI>
__device__ __forceinline__ void epi_zero(const GemmArgs& A, const Ctx& c, int tid) {
  if constexpr (EPI == EPI_ACC32) return;
  const int64_t ncols = (MODE == MODE_FPROP) ? A.N : A.K;
  const int esz = (EPI == EPI_STORE32) ? 4 : 2;
  for (int it = 0; it < 32 * esz / 2; ++it) {
    const int per_row = 256 * esz / 16;             // 16-byte pieces per tile row
    const int idx = it * NTHREADS + tid;
    const int row = idx / per_row;
    const int col = (idx % per_row) * (16 / esz);
    const int64_t gcol = c.nrow0 + col;
    if (row >= c.arows || gcol >= ncols) continue;
    const int64_t orow = (MODE == MODE_FPROP) ? c.arow0 + row : (int64_t)c.g * A.N + c.arow0 + row;
    uint8_t* dst = static_cast<uint8_t*>(A.c) + (orow * ncols + gcol) * esz;
    if (gcol + 16 / esz <= ncols) {
      *reinterpret_cast<uint4*>(dst) = make_uint4(0, 0, 0, 0);
    } else {
      for (int q = 0; q < (int)(ncols - gcol) * esz; ++q) dst[q] = 0;
    }
  }
}

// red: 8 floats of LDS for the workgroup's amax reduction (EPI_STORE_AMAX); tile: the tile's index
// in the launch's sequence (its amax slot).
// probs: 256 floats of LDS for the tile's token probabilities (EPI_STORE_AMAX).  They are loaded
// once, before the first chunk's stores: a vector load waits for every memory operation issued
// before it (the wait counter retires in order), so a load after the stores would wait for them.
template <int MODE, int EPI, int BF = 0>
__device__ __forceinline__ void mx_epilogue(const GemmArgs& A, const Ctx& c, const v16f (&acc)[4][4], uint8_t* buf,
                                            int tid, int wm, int wn, int lane, int tile, float* red, float* probs) {
  float pre = 0.0f, post = 0.0f;
  uint32_t mask = 0;
  if constexpr (EPI == EPI_STORE_AMAX) {
    probs[tid] = tid < c.arows ? late_ptr(A.probs)[c.arow0 + tid] : 0.0f;   // visible after chunk 0's barrier
    mask = *reinterpret_cast<const volatile uint32_t*>(&A.rht_mask);
  }
  epi_chunk<MODE, EPI, 0, BF>(A, c, acc, buf, tid, wm, wn, lane, probs, mask, pre, post);
  epi_chunk<MODE, EPI, 1, BF>(A, c, acc, buf, tid, wm, wn, lane, probs, mask, pre, post);
  epi_chunk<MODE, EPI, 2, BF>(A, c, acc, buf, tid, wm, wn, lane, probs, mask, pre, post);
  epi_chunk<MODE, EPI, 3, BF>(A, c, acc, buf, tid, wm, wn, lane, probs, mask, pre, post);
  epi_chunk<MODE, EPI, 4, BF>(A, c, acc, buf, tid, wm, wn, lane, probs, mask, pre, post);
  epi_chunk<MODE, EPI, 5, BF>(A, c, acc, buf, tid, wm, wn, lane, probs, mask, pre, post);
  epi_chunk<MODE, EPI, 6, BF>(A, c, acc, buf, tid, wm, wn, lane, probs, mask, pre, post);
  epi_chunk<MODE, EPI, 7, BF>(A, c, acc, buf, tid, wm, wn, lane, probs, mask, pre, post);
  if constexpr (EPI == EPI_STORE_AMAX) {
    // the tile's maxima into one of its group's slots, as the standalone pass does: the
    // post-transform amax is bf16(max |y| / 4) (the factor is exact and rounding is monotone)
    post = wave_max(round_bf16(post * 0.25f));
    pre = wave_max(pre);
    const int wave = tid >> 6;
    if (lane == 0) {
      red[wave] = pre;
      red[4 + wave] = post;
    }
    __syncthreads();
    if (tid == 0) {
      const float a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
      const float b = fmaxf(fmaxf(red[4], red[5]), fmaxf(red[6], red[7]));
      const int slot = tile % kAmaxSlots;
      uint32_t* slots = late_ptr(A.T.amax_slots);
      atomicMax(slots + ((int64_t)c.g * kAmaxSlots + slot), __float_as_uint(a));
      atomicMax(slots + ((int64_t)(A.G + c.g) * kAmaxSlots + slot), __float_as_uint(b));
    }
  }
}

// bf16 epilogue of the transposed accumulators (EPI_STORE): lane (m + 32 j) of wave (wm, wn)
// holds in acc[tm][tn][4 q + t] the output at tile row 128 wm + 32 tm + m and tile column
// 128 wn + 32 tn + 8 q + 4 j + t, so four consecutive columns of one row are rounded to bf16 in
// registers (the same product by the group scale and the same rounding as the fp32-staged
// epilogue) and staged with one 8-byte LDS write.  Chunk tm (4 per tile) stages tile rows
// 32 tm + [0, 32) and 128 + 32 tm + [0, 32) (staged row sr: tile row chunk_row(tm, sr)) across
// all 256 columns: 64 rows of 512 bytes, one 32 KB ring slot.  The 16-byte column chunk c of
// staged row sr sits at chunk c ^ (sr & 31), so that the 32 rows one write instruction covers
// spread over the banks; each read instruction takes two whole rows.
__device__ __forceinline__ uint32_t trs_off(int sr, int c) { return (uint32_t)(sr * 512 + ((c ^ (sr & 31)) << 4)); }

// One accumulator register read where it is used (element access to the accumulator vectors
// would have the compiler copy all of them to vector registers at once).  The epilogue reads the
// MFMA tile rows in the order the last step computed them (tm = 0 first, whose MFMAs issue
// first), so every read comes at least eight MFMAs (about 500 cycles) after the MFMA that wrote
// its register, far past the MFMA-to-read wait the hardware requires.
__device__ __forceinline__ float acc_read(float a) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
}

template <int MODE, int TM, int BF>
__device__ __forceinline__ void epi_chunk_tr(const GemmArgs& A, const Ctx& c, const v16f (&acc)[4][4], uint8_t* buf,
                                             int tid, int wm, int wn, int lane) {
  {
    const int m = lane & 31, j = lane >> 5;
    const int sr = 32 * wm + m;
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float v0 = acc_read(acc[TM][tn][4 * q]), v1 = acc_read(acc[TM][tn][4 * q + 1]);
        float v2 = acc_read(acc[TM][tn][4 * q + 2]), v3 = acc_read(acc[TM][tn][4 * q + 3]);
        if constexpr (BF != 0) {
          v0 = __fmul_rn(v0, c.alpha);
          v1 = __fmul_rn(v1, c.alpha);
          v2 = __fmul_rn(v2, c.alpha);
          v3 = __fmul_rn(v3, c.alpha);
        }
        *reinterpret_cast<uint2*>(buf + trs_off(sr, 16 * wn + 4 * tn + q) + 8 * j) =
            make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
      }
      GMLP_SB();   // a column tile at a time: few accumulators in vector registers at once
    }
  }
  __syncthreads();
  {
    // thread tid stores 16-byte column chunk cc of staged rows 8 it + r0 (it = 0..7): one wave
    // instruction covers two whole 512-byte rows
    const int64_t ncols = (MODE == MODE_FPROP) ? A.N : A.K;
    const int64_t orow0 = (MODE == MODE_FPROP) ? c.arow0 : (int64_t)c.g * A.N + c.arow0;
    const uint32_t rowb = (uint32_t)(ncols * 2);
    const __amdgpu_buffer_rsrc_t r =
        out_rsrc(static_cast<uint8_t*>(A.c) + (orow0 * ncols + c.nrow0) * 2, (int64_t)c.arows * rowb);
    const int cc = tid & 31, r0 = tid >> 5;
    const uint32_t voff = (c.nrow0 + 8 * cc < ncols) ? (uint32_t)r0 * rowb + (uint32_t)(16 * cc) : kOutOfRange;
    uint4 v[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) v[it] = *reinterpret_cast<const uint4*>(buf + trs_off(8 * it + r0, cc));
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      // tile row of staged row 8 it + r0 = 128 (it / 4) + 32 TM + 8 (it % 4) + r0; r0 goes in voff
      const uint32_t ur = (uint32_t)(128 * (it >> 2) + 32 * TM + 8 * (it & 3));
      out_store(r, voff, ur * rowb, v[it].x, v[it].y, v[it].z, v[it].w);
    }
  }
  __syncthreads();
}

template <int MODE, int BF>
__device__ __forceinline__ void mx_epilogue_tr(const GemmArgs& A, const Ctx& c, const v16f (&acc)[4][4], uint8_t* buf,
                                               int tid, int wm, int wn, int lane) {
  epi_chunk_tr<MODE, 0, BF>(A, c, acc, buf, tid, wm, wn, lane);
  epi_chunk_tr<MODE, 1, BF>(A, c, acc, buf, tid, wm, wn, lane);
  epi_chunk_tr<MODE, 2, BF>(A, c, acc, buf, tid, wm, wn, lane);
  epi_chunk_tr<MODE, 3, BF>(A, c, acc, buf, tid, wm, wn, lane);
}

template <int MODE, int EPI, int BF = 0>
__device__ __forceinline__ TileRef tile_ref(const GemmArgs& A, int t, int ntm, int ntn) {
  int mt;
  Ctx c;
  tile_ctx<MODE, EPI>(A, t, ntm, ntn, mt, c);
  TileRef r;
  // bf16: 32 contraction elements per 64-byte stage; token offsets of the column-wise
  // operands count 2 bytes per token
  r.nk = uni((MODE == MODE_WGRAD && BF) ? wgrad_stages(c.kvalid, 2) : BF ? (int)((2 * c.kvalid + 63) / 64) : c.nk);
  r.arows = uni(c.arows);
  r.arow0 = uni(c.arow0);
  r.g = uni(c.g);
  r.nt = uni(c.nt);
  r.off = (MODE == MODE_WGRAD) ? uni((BF ? 2 : 1) * A.T.col_off[c.g]) : 0;
  r.woff = (MODE == MODE_WGRAD) ? uni(A.T.colw_off[c.g]) : 0;
  return r;
}

// WGRAD: the XCD ranges [lo, hi) of the tile sequence hold equal shares of the work rather than
// equal numbers of tiles, because experts' token counts (each tile's contraction length) can
// differ by orders of magnitude.  A tile of expert g costs its stages plus an epilogue's worth
// (kEpiStages); expert g's tiles are the contiguous range [g tpg, (g + 1) tpg).  The boundary
// for cost c is the first tile whose preceding tiles cost at least c, so the ranges of the 8
// XCDs tile the sequence exactly.
constexpr int64_t kEpiStages = 8;
template <int BF>
__device__ __forceinline__ int64_t wgrad_tile_cost(const GemmArgs& A, int g) {
  const int64_t P = A.T.col_off[g + 1] - A.T.col_off[g];
  const int64_t tokens = min((int64_t)(A.T.row_off[g + 1] - A.T.row_off[g]), P);
  return wgrad_stages(tokens, BF ? 2 : 1) + kEpiStages;
}
// Only when the costs are skewed (the dearest tile above twice the mean): with near-equal costs
// the equal-count ranges are whole rounds of the XCD's workgroups, which cost-cut ranges break.
template <int BF>
__device__ __forceinline__ void wgrad_xcd_range(const GemmArgs& A, int tpg, int x, int& lo, int& hi) {
  int64_t W = 0, wmax = 0;
  for (int g = 0; g < A.G; ++g) {
    const int64_t w = wgrad_tile_cost<BF>(A, g);
    W += tpg * w;
    wmax = w > wmax ? w : wmax;
  }
  if (wmax * A.G * tpg <= 2 * W) return;
  const int64_t c0 = W * x / 8, c1 = W * (x + 1) / 8;
  lo = hi = A.G * tpg;
  bool have_lo = false;
  int64_t pre = 0;
  for (int g = 0; g < A.G; ++g) {
    const int64_t w = wgrad_tile_cost<BF>(A, g);
    const int64_t end = pre + tpg * w;
    if (!have_lo && end > c0) {
      lo = g * tpg + (int)((c0 - pre + w - 1) / w);
      have_lo = true;
    }
    if (end > c1) {
      hi = g * tpg + (int)((c1 - pre + w - 1) / w);
      break;
    }
    pre = end;
  }
}

template <int MODE, int EPI, int BF>
__global__ __launch_bounds__(NTHREADS) void gemm_mx_kernel(GemmArgs A) {
  __shared__ __align__(16) uint8_t smem[MX_NSTAGE * MX_STAGE];
  __shared__ float red[8];
  __shared__ float tile_probs[(EPI == EPI_STORE_AMAX) ? 256 : 1];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = uni(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  // the bf16-store epilogue takes the transposed accumulators
  constexpr int TR = (EPI == EPI_STORE) ? 1 : 0;
  // valid tiles and this workgroup's share
  const int ntn = tiles_n<MODE, EPI>(A);
  const int ntm = (MODE == MODE_FPROP) ? (A.G > 0 ? uni(A.T.t256_off[A.G]) : 0) : A.G * (int)((A.N + BM - 1) / BM);
  const int64_t nt = (int64_t)ntm * ntn;
  const int nwx = gridDim.x / 8, x = blockIdx.x % 8, lw = blockIdx.x / 8;
  int lo = (int)(nt * x / 8), hi = (int)(nt * (x + 1) / 8);
  if (MODE == MODE_WGRAD) wgrad_xcd_range<BF>(A, ntm / A.G * ntn, x, lo, hi);
  lo = uni(lo);
  hi = uni(hi);
  int t = lo + lw;
  if (t >= hi) return;

  const uint32_t lane_off = (uint32_t)(lane >> 2) * 64u + 16u * (uint32_t)((lane & 3) ^ ((lane >> 4) & 3));
  const DmaPlan dpl{nullptr, nullptr, 0, 0, 0, 0, lane_off};
  const uint32_t s_voff = 16u * lane;
  auto slot = [&](uint32_t st) { return smem + (st & (MX_NSTAGE - 1)) * MX_STAGE; };

  // DMA window: the current non-empty tile (R0, and its full sources D0) and the next two
  int dnext = t;
  auto next_ref = [&]() -> TileRef {
    while (dnext < hi) {
      const TileRef r = tile_ref<MODE, EPI, BF>(A, dnext, ntm, ntn);
      dnext += nwx;
      if (r.nk > 0) return r;
    }
    TileRef r{};
    return r;                          // nk = 0: no tile (its stages are issued empty)
  };
  const DmaConst KC = dma_const<MODE, EPI, BF>(A, wave);
  const ReadPlan rp = make_read_plan(wm, wn, lane);
  DmaTile D0 = dma_tile<MODE, EPI, BF>(A, next_ref(), wave);
  DmaTile D1 = dma_tile<MODE, EPI, BF>(A, next_ref(), wave);
  DmaTile D2 = dma_tile<MODE, EPI, BF>(A, next_ref(), wave);
  // stage `off` positions past the first stage of D0 (selects only: the step has no branch)
  auto window_stage = [&](int off, uint8_t* dst) -> StageDma {
    const bool u1 = off >= D0.nk;
    const int o1 = off - D0.nk;
    const bool u2 = u1 && o1 >= D1.nk;
    const int o2 = o1 - D1.nk;
    return dma_tile_stage(KC, sel_tile(u2, D2, sel_tile(u1, D1, D0)), u2 ? o2 : (u1 ? o1 : off), dst, s_voff, wave);
  };

  uint32_t gs = 0;                     // sequence number of the next stage to compute
  for (int o = 0; o < 3; ++o) {
    const StageDma sd = window_stage(o, slot(o));
    mx_dma_one<0>(sd, dpl, wave); mx_dma_one<1>(sd, dpl, wave); mx_dma_one<2>(sd, dpl, wave);
    mx_dma_one<3>(sd, dpl, wave); mx_dma_one<4>(sd, dpl, wave); mx_dma_one<5>(sd, dpl, wave);
    mx_dma_one<6>(sd, dpl, wave); mx_dma_one<7>(sd, dpl, wave); mx_dma_one<8>(sd, dpl, wave);
  }

  for (; t < hi; t += nwx) {
    // every non-empty tile is R0 of the DMA window when the compute reaches it
    const TileRef cr = tile_ref<MODE, EPI, BF>(A, t, ntm, ntn);
    Ctx c;
    c.arows = cr.arows;
    c.arow0 = cr.arow0;
    c.g = cr.g;
    c.nt = cr.nt;
    c.nrow0 = (int64_t)cr.nt * BN;
    c.alpha = 1.0f;
    if (BF) {
      // NVFP4 operands carry dec(E2M1) dec(E4M3); the group's global scales divide the product
      const float sa = nvfp4_global_scale(A.a.amax[cr.g]);
      const float sb = nvfp4_global_scale(A.b.amax[cr.g]);
      c.alpha = __fmul_rn(__fdiv_rn(1.0f, sa), __fdiv_rn(1.0f, sb));
    }
    const int nk = cr.nk;
    if (nk == 0) {                     // an empty group's weight gradient: zeros
      int tid_t = tid;
      asm volatile("" : "+v"(tid_t));
      epi_zero<MODE, EPI>(A, c, tid_t);
      continue;
    }
    v16f acc[4][4];                    // set by the first step (MFMAs onto zero)
    MxFrags f0, f1;
    {
      // stage gs (this tile's first) has landed once at most the two stages after it are pending
      wait_vmcnt<2 * MX_DMA_PER_STAGE>();
      __syncthreads();
      mx_read_p<0, BF>(slot(gs), rp, f0);
      // One step: the DMAs of sequence stage gs + 3 (whose slot held stage gs - 1, read by every
      // wave before the previous step's barrier), then the MFMAs of stage gs with the reads of
      // stage gs + 1 in between.  Stage gs + 1 may be the next tile's first (read again after
      // the epilogue) or no stage at all; such reads go unused.  Two steps per trip keep the two
      // fragment sets in fixed registers
      // (stage kt + 1 of an even kt has parity 1, of an odd kt parity 0).  A weight gradient's
      // nk may be odd: its last trip runs the first step only.  Every tile has at least 2
      // stages, so the stage three ahead always lies in the window's three tiles.
      // The first pair: its first step starts the accumulators (DMA targets 3 and 4 may be past
      // the tile).
      {
        const StageDma sd = window_stage(3, slot(gs + 3));
        GMLP_SB();
        mx_phase1<BF, true, TR>(f0, acc, sd, dpl, wave);
        wait_vmcnt<MX_DMA_PER_STAGE + MX_DMA_BEFORE_BARRIER>();
        __syncthreads();
        mx_phase2p<1, BF, true, TR>(f0, acc, sd, dpl, wave, slot(gs + 1), rp, f1);
        ++gs;
      }
      {
        const StageDma sd = window_stage(4, slot(gs + 3));
        GMLP_SB();
        mx_phase1<BF, false, TR>(f1, acc, sd, dpl, wave);
        wait_vmcnt<MX_DMA_PER_STAGE + MX_DMA_BEFORE_BARRIER>();
        __syncthreads();
        mx_phase2p<0, BF, false, TR>(f1, acc, sd, dpl, wave, slot(gs + 1), rp, f0);
        ++gs;
      }
      int kt = 2;
      if (nk > 6) {
        // steps whose DMA target (kt + 3, kt + 4) is still in this tile: fixed resources, the
        // stage in SOFFSET (32-bit: every operand is below 4 GB)
        const RunDma rr = run_rsrc(KC, D0);
        uint32_t soa = 5u * KC.a_ps, sob = 5u * KC.b_ps;
        const uint32_t s_step = 4u * KC.s_ld;
        uint32_t sos = 2u * s_step;                  // 128-K word (kt + 3) / 2 = 2
        do {
          {
            const StageDma sd = run_stage(rr, soa, sob, sos, slot(gs + 3), s_voff, wave);
            GMLP_SB();
            mx_phase1<BF, false, TR>(f0, acc, sd, dpl, wave);
            wait_vmcnt<MX_DMA_PER_STAGE + MX_DMA_BEFORE_BARRIER>();
            __syncthreads();
            mx_phase2p<1, BF, false, TR>(f0, acc, sd, dpl, wave, slot(gs + 1), rp, f1);
            ++gs;
          }
          soa += KC.a_ps;
          sob += KC.b_ps;
          {
            const StageDma sd = run_stage(rr, soa, sob, sos + s_step, slot(gs + 3), s_voff, wave);
            GMLP_SB();
            mx_phase1<BF, false, TR>(f1, acc, sd, dpl, wave);
            wait_vmcnt<MX_DMA_PER_STAGE + MX_DMA_BEFORE_BARRIER>();
            __syncthreads();
            mx_phase2p<0, BF, false, TR>(f1, acc, sd, dpl, wave, slot(gs + 1), rp, f0);
            ++gs;
          }
          soa += KC.a_ps;
          sob += KC.b_ps;
          sos += s_step;
          kt += 2;
        } while (kt < nk - 4);
      }
      while (kt < nk) {                  // the last two pairs (or one): DMA targets may be past the tile
        {
          const StageDma sd = window_stage(kt + 3, slot(gs + 3));
          GMLP_SB();
          mx_phase1<BF, false, TR>(f0, acc, sd, dpl, wave);
          wait_vmcnt<MX_DMA_PER_STAGE + MX_DMA_BEFORE_BARRIER>();
          __syncthreads();
          mx_phase2p<1, BF, false, TR>(f0, acc, sd, dpl, wave, slot(gs + 1), rp, f1);
          ++gs;
        }
        if (kt + 1 < nk) {
          const StageDma sd = window_stage(kt + 4, slot(gs + 3));
          GMLP_SB();
          mx_phase1<BF, false, TR>(f1, acc, sd, dpl, wave);
          wait_vmcnt<MX_DMA_PER_STAGE + MX_DMA_BEFORE_BARRIER>();
          __syncthreads();
          mx_phase2p<0, BF, false, TR>(f1, acc, sd, dpl, wave, slot(gs + 1), rp, f0);
          ++gs;
        }
        kt += 2;
      }
      D0 = D1;
      D1 = D2;
      D2 = dma_tile<MODE, EPI, BF>(A, next_ref(), wave);
    }
    // the slot of the last consumed stage holds nothing pending (the ones after it do).  The
    // thread index is laundered per tile so that the epilogue's per-thread addresses are
    // formed here rather than hoisted out of the tile loop (they would stay live, and spill,
    // across every main loop).
    int tid_t = tid;
    asm volatile("" : "+v"(tid_t));
    if constexpr (TR) {
      mx_epilogue_tr<MODE, BF>(A, c, acc, slot(gs + 3), tid_t, wm, wn, tid_t & 63);
    } else {
      mx_epilogue<MODE, EPI, BF>(A, c, acc, slot(gs + 3), tid_t, wm, wn, tid_t & 63, t, red, tile_probs);
    }
  }
  wait_vmcnt<0>();                     // the DMAs past the last tile (empty) before the LDS is released
}

// One thread per row sums the partials in tile order; the loads of 8 partials are issued
// together (small blocks: enough of them to spread over every CU).
__global__ __launch_bounds__(64) void dprob_reduce_kernel(const float* __restrict__ part, int nparts, int64_t M,
                                                          float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= M) return;
  float s = 0.0f;
  int p = 0;
  for (; p + 8 <= nparts; p += 8) {
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = part[(int64_t)(p + k) * M + i];
#pragma unroll
    for (int k = 0; k < 8; ++k) s += v[k];
  }
  for (; p < nparts; ++p) s += part[(int64_t)p * M + i];
  out[i] = s;
}

// ----------------------------------------------------------------------------- launchers
int gemm_fprop_ntiles_n(const GemmArgs& g) {
  return (int)((g.N + BN - 1) / BN);
}

static int cu_count() {
  static int n[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (n[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    n[dev] = v;
  }
  return n[dev];
}

template <int MODE, int EPI, int BF>
static hipError_t launch_mx(const GemmArgs& g, hipStream_t s) {
  int64_t tiles;
  if (MODE == MODE_FPROP) {
    tiles = ((g.M + BM - 1) / BM + g.G) * (int64_t)gemm_fprop_ntiles_n(g);
  } else {
    tiles = (int64_t)g.G * ((g.N + BM - 1) / BM) * ((g.K + BN - 1) / BN);
  }
  if (tiles <= 0) return hipSuccess;
  // the DMA sources are 32-bit offsets: every operand (data and scale words) below 4 GB
  {
    const int64_t brows = g.N;
    const int64_t rows_bound = g.M + 127LL * g.G;                    // padded tokens of all groups
    const int64_t eb = BF ? 2 : 1;
    const int64_t big = eb * ((MODE == MODE_FPROP) ? std::max(g.M * g.K, (int64_t)g.G * brows * g.K)
                                                   : std::max(g.N, g.K) * rows_bound);
    if (big >= (1LL << 32)) return hipErrorInvalidValue;
    // epilogue stores address one tile (256 rows) of an output through one buffer resource,
    // with kOutOfRange marking a lane's columns as outside it
    const int64_t orow_bytes = (MODE == MODE_FPROP ? g.N : g.K) * 4;
    if (256 * orow_bytes >= (int64_t)kOutOfRange) return hipErrorInvalidValue;
  }
  GemmArgs a = g;
  // Row tiles per launch-order group.  FPROP: 4, so that 4 x 8 tiles are one XCD's round of 32
  // workgroups (2, 8 and 16 measured 0.5-2% slower on the 8- and 128-expert workloads).  When
  // the groups average at most two 256-row tiles, most 4-row groups would straddle experts and
  // fetch several weight panels per column tile: then groups of 8 rows inside one expert
  // (the 128-expert workload: 19-26% fewer bytes fetched by its forward-shaped GEMMs, 1% off
  // the step; with 8 experts of 3-4K rows the same order was 1-2% slower, with the 64 Zipf-sized
  // experts of 768 rows on average 2-4%).  WGRAD: 2 (3% faster
  // than 4 on the 128-expert workload's fc1 weight gradient, 8 is 6% slower, 1 is 1% slower).
  a.expert_groups = (MODE == MODE_FPROP && g.G > 0 && g.M <= 512LL * g.G) ? 1 : 0;
  a.group_rows = MODE == MODE_WGRAD ? 2 : (a.expert_groups ? 8 : 4);
  // one workgroup per CU (the LDS ring allows no more), a multiple of 8 for the XCD split
  int64_t wgs = std::min<int64_t>(cu_count(), tiles);
  wgs = (wgs + 7) / 8 * 8;
  hipLaunchKernelGGL((gemm_mx_kernel<MODE, EPI, BF>), dim3((unsigned)wgs), dim3(NTHREADS), 0, s, a);
  return hipGetLastError();
}

// NVFP4: both operands expanded exactly to bf16 panels in the caller's scratch, then the
// persistent kernel on the bf16 MFMA with the groups' global scales in the epilogue.  The
// fc2-dgrad form (EPI_DACT) stores da and runs the activation gradient as its own pass.
static hipError_t launch_nvfp4(const GemmArgs& g, int epi, hipStream_t s) {
  if ((!g.a.bf16 && !g.xa) || (!g.b.bf16 && !g.xb) || (epi == EPI_DACT && !g.da_tmp)) return hipErrorInvalidValue;
  hipError_t e;
  const int64_t bound = g.M + 127LL * g.G;                 // padded tokens of all groups
  if (!g.a.bf16) {
    e = g.mode == MODE_FPROP ? launch_nv_expand(g.a.data, g.a.scale, g.xa, g.M, g.K, 1, s)
                             : launch_nv_expand_groups(g.a.data, g.a.scale, g.xa, g.N, bound, g.T.col_off, g.G, s);
    if (e != hipSuccess) return e;
  }
  if (!g.b.bf16) {
    e = g.mode == MODE_FPROP ? launch_nv_expand(g.b.data, g.b.scale, g.xb, g.N, g.K, g.G, s)
                             : launch_nv_expand_groups(g.b.data, g.b.scale, g.xb, g.K, bound, g.T.col_off, g.G, s);
    if (e != hipSuccess) return e;
  }
  GemmArgs a = g;
  a.fmt = FMT_NVFP4_BF16;
  a.a.data = g.a.bf16 ? g.a.bf16 : g.xa;
  a.b.data = g.b.bf16 ? g.b.bf16 : g.xb;
  // no scale words: their DMA slot runs with empty resources; give them a real base anyway
  a.a.scale_mfma = reinterpret_cast<const uint32_t*>(a.a.data);
  a.b.scale_mfma = reinterpret_cast<const uint32_t*>(a.b.data);
  if (g.mode == MODE_WGRAD) {
    if (epi == EPI_ACC32) return launch_mx<MODE_WGRAD, EPI_ACC32, 1>(a, s);
    return epi == EPI_STORE32 ? launch_mx<MODE_WGRAD, EPI_STORE32, 1>(a, s) : launch_mx<MODE_WGRAD, EPI_STORE, 1>(a, s);
  }
  if (epi == EPI_STORE32) return launch_mx<MODE_FPROP, EPI_STORE32, 1>(a, s);
  if (epi == EPI_STORE) return launch_mx<MODE_FPROP, EPI_STORE, 1>(a, s);
  if (epi == EPI_STORE_AMAX) {
    if ((e = launch_mx<MODE_FPROP, EPI_STORE_AMAX, 1>(a, s)) != hipSuccess) return e;
    return launch_amax_finalize(g.T, g.G, g.amax_pre_out, g.amax_post_out, s);
  }
  if (epi != EPI_DACT) return hipErrorInvalidValue;
  a.epi = EPI_STORE;
  a.c = g.da_tmp;
  a.out_fp32 = 0;
  if ((e = launch_mx<MODE_FPROP, EPI_STORE, 1>(a, s)) != hipSuccess) return e;
  return launch_dact_bf16(g.da_tmp, g.h, g.probs, g.act, g.ffn, g.M, g.dh, g.a_out, g.dprob_part, s);
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t s) {
  if (g.epi == EPI_STORE_AMAX &&
      (g.mode != MODE_FPROP || g.fmt != FMT_NVFP4 || !g.probs || !g.amax_pre_out || !g.amax_post_out))
    return hipErrorInvalidValue;
  if (g.mode == MODE_FPROP && g.M == 0) {
    // no rows: every group's fc2-input amax is zero
    return g.epi == EPI_STORE_AMAX ? launch_amax_finalize(g.T, g.G, g.amax_pre_out, g.amax_post_out, s) : hipSuccess;
  }
  const int epi = (g.epi != EPI_STORE || !g.out_fp32) ? g.epi : (g.out_fp32 == 2 ? (int)EPI_ACC32 : (int)EPI_STORE32);
  if (epi == EPI_ACC32 && g.mode != MODE_WGRAD) return hipErrorInvalidValue;
  if (g.fmt == FMT_NVFP4) return launch_nvfp4(g, epi, s);
#define GMLP_DISPATCH_MX(MO, E) \
  if (g.fmt == FMT_MXFP8 && g.mode == MO && epi == E) return launch_mx<MO, E, 0>(g, s);
  GMLP_DISPATCH_MX(MODE_FPROP, EPI_STORE)
  GMLP_DISPATCH_MX(MODE_FPROP, EPI_STORE32)
  GMLP_DISPATCH_MX(MODE_WGRAD, EPI_STORE32)
  GMLP_DISPATCH_MX(MODE_WGRAD, EPI_STORE)
  GMLP_DISPATCH_MX(MODE_WGRAD, EPI_ACC32)
#undef GMLP_DISPATCH_MX
  return hipErrorInvalidValue;
}

hipError_t launch_dprob_reduce(const float* part, int nparts, int64_t M, float* out, hipStream_t s) {
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL(dprob_reduce_kernel, dim3((unsigned)((M + 63) / 64)), dim3(64), 0, s, part, nparts, M, out);
  return hipGetLastError();
}

}  // namespace gmlp
