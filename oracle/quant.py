"""MXFP8 and NVFP4 group quantization and their layouts.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
* "GEMM + Swiglu fused Grouped MLP for MXFP8" -- Greptile summary and sequence
  diagram: MXFP8 operands with row-wise data + ``sfd_row`` and column-wise data
  + ``sfd_col``; grouped tensors keep every data and scale field as one flat
  1-D buffer with per-group offsets.
* "Reduce NVFP4 quantization work for the fused GroupedMLP fc2 input with
  activation recompute" -- Description and Changes: row-wise NVFP4 data for
  the fc2 GEMM, column-wise data (with the RHT) for wgrad, a per-group
  (pre-RHT, post-RHT) amax and ``nvfp4_group_quantize_with_amax``.
* OCP Microscaling Formats (MX) v1.0 for the MXFP8 shared-exponent rule.

MXFP8 block of 32 values v (readings S1-S4):
  A = max|v_i|.  A == 0 -> scale code 127 (2^0) and every element encodes v_i.
  Otherwise X = clamp(floor(log2 A) - 8, -127, 127)  (8 = emax of E4M3),
  scale code = X + 127 and q_i = E4M3(v_i * 2^-X); the multiply is exact.

NVFP4 block of 16 values v with group amax A (pre-RHT amax for row-wise casts,
post-RHT amax for column-wise casts), every step in fp32 (readings S5, S6):
  S = 2688 / A (A > 0; clipped to FLT_MAX), S = 1 when A == 0; 2688 = 6 * 448
  b = max|v_i|;  s = (b / 6) * S;  q = E4M3(s) (saturating)
  r = S / dec(q), clipped to FLT_MAX like S  (r = 0 when q == 0);  c_i = E2M1(v_i * r)
  dequantized value: dec(c_i) * dec(q) / S.

Layouts (ours; the pages fix none):
* row-wise: [R, K] with blocks along K.  MXFP8 data u8 [R, K], scales u8
  [R, K/32].  NVFP4 data u8 [R, K/2] (element 2i in the low nibble), E4M3
  scales [R, K/16].
* column-wise, per group g with m_g rows: the group's [m_g, K] slab transposed
  to [K, P_g] with P_g = m_g rounded up to 128 (zero padded; a multiple of both
  block sizes and of the 128-token contraction stage of the wgrad GEMM, so one
  padded offset table serves both recipes), blocks along tokens.
  Group g's data starts at K * sum_{h<g} P_h elements (bytes for MXFP8, nibbles
  for NVFP4) and its scales at K * sum_{h<g} P_h / B (B = 32 or 16).
* MFMA-ready MXFP8 scales: a scale matrix [R, nkb] becomes u32 [ceil(nkb/4), R]
  where word (t, r) holds the codes of blocks 4t..4t+3 of row r in bytes 0..3
  (missing blocks = 127).  For column-wise scales each group's [K, P_g/32]
  matrix is converted on its own and placed at word offset K * sum_{h<g} P_h / 128.
"""
import numpy as np

from .formats import (FLT_MAX, bf16_bits_to_f64, e2m1_decode, e2m1_encode, e4m3_decode,
                      e4m3_encode, e8m0_decode, f32, pack_fp4, unpack_fp4)
from .rht import RHT_BLOCK, rht16

MX_BLOCK = 32
NV_BLOCK = 16
COL_PAD = 128


def padded(m, to=COL_PAD):
    return -(-int(m) // to) * to


def col_offsets(m_splits, to=COL_PAD):
    """Exclusive prefix sum of the padded group sizes P_g."""
    p = [padded(m, to) for m in m_splits]
    return np.concatenate([[0], np.cumsum(p)]).astype(np.int64)


# ----------------------------------------------------------------------------- MXFP8
def mxfp8_quantize_rows(v):
    """Quantize [R, K] fp64 values in blocks of 32 along K -> (E4M3 codes [R, K], E8M0 codes [R, K/32])."""
    r, k = v.shape
    assert k % MX_BLOCK == 0
    b = v.reshape(r, k // MX_BLOCK, MX_BLOCK)
    amax = np.max(np.abs(b), axis=-1)
    _, e = np.frexp(amax)                          # amax = m * 2^e, m in [0.5, 1) -> floor(log2) = e - 1
    x = np.clip(e - 1 - 8, -127, 127)
    x = np.where(amax == 0, 0, x).astype(np.int64)
    q = e4m3_encode(b * np.ldexp(1.0, -x)[..., None])
    return q.reshape(r, k), (x + 127).astype(np.uint8)


def mxfp8_dequant_rows(q, s):
    r, k = q.shape
    d = e4m3_decode(q).reshape(r, k // MX_BLOCK, MX_BLOCK) * e8m0_decode(s)[..., None]
    return d.reshape(r, k)


def mfma_scale_layout(s):
    """[R, nkb] E8M0 codes -> u32 [ceil(nkb/4), R] (4 consecutive blocks of a row per word)."""
    r, nkb = s.shape
    nkt = -(-nkb // 4)
    full = np.full((r, nkt * 4), 127, dtype=np.uint32)
    full[:, :nkb] = s
    full = full.reshape(r, nkt, 4)
    words = full[..., 0] | (full[..., 1] << 8) | (full[..., 2] << 16) | (full[..., 3] << 24)
    return np.ascontiguousarray(words.T).astype(np.uint32)


def _group_col_slab(x, off, m, k):
    p = padded(m)
    t = np.zeros((k, p), dtype=np.float64)
    t[:, :m] = x[off:off + m].T
    return t


def mxfp8_group_quantize(x_bits, m_splits, row=True, col=True):
    """Group-quantize a bf16 [M, K] tensor whose rows are split into groups by ``m_splits``.

    Returns a dict: ``row_data`` [M, K], ``row_scale`` [M, K/32], ``row_scale_mfma``;
    ``col_data`` and ``col_scale`` flat in the column-wise layout, ``col_scale_mfma`` flat
    u32, plus the per-group column slabs ``col_groups`` = [(data [K, P_g], scale [K, P_g/32])].
    """
    x = bf16_bits_to_f64(x_bits)
    m_total, k = x.shape
    assert sum(m_splits) == m_total
    out = {}
    if row:
        q, s = mxfp8_quantize_rows(x)
        out["row_data"], out["row_scale"] = q, s
        out["row_scale_mfma"] = mfma_scale_layout(s)
    if col:
        groups, data, scales, words = [], [], [], []
        off = 0
        for m in m_splits:
            q, s = mxfp8_quantize_rows(_group_col_slab(x, off, m, k))
            off += m
            groups.append((q, s))
            data.append(q.reshape(-1))
            scales.append(s.reshape(-1))
            words.append(mfma_scale_layout(s).reshape(-1) if s.size else np.zeros(0, np.uint32))
        out["col_groups"] = groups
        out["col_data"] = np.concatenate(data) if data else np.zeros(0, np.uint8)
        out["col_scale"] = np.concatenate(scales) if scales else np.zeros(0, np.uint8)
        out["col_scale_mfma"] = np.concatenate(words) if words else np.zeros(0, np.uint32)
    return out


# ----------------------------------------------------------------------------- NVFP4
def nvfp4_global_scale(amax):
    """S = fp32(2688 / amax), clipped to FLT_MAX; 1 when amax == 0."""
    a = np.float64(np.float32(amax))
    if a == 0:
        return 1.0
    with np.errstate(over="ignore"):
        s = f32(2688.0 / a)
    return float(min(s, FLT_MAX))


def nvfp4_quantize_rows(v, amax):
    """Quantize [R, K] fp64 values in blocks of 16 along K with one global amax.

    Returns (E2M1 nibbles [R, K] unpacked, E4M3 block-scale codes [R, K/16]).
    """
    r, k = v.shape
    assert k % NV_BLOCK == 0
    S = nvfp4_global_scale(amax)
    blk = v.reshape(r, k // NV_BLOCK, NV_BLOCK)
    b = np.max(np.abs(blk), axis=-1)
    s = f32(f32(b / 6.0) * S)
    q = e4m3_encode(s)
    dq = e4m3_decode(q)
    with np.errstate(divide="ignore"):
        with np.errstate(over="ignore"):
            rr = np.where(q == 0, 0.0, np.minimum(f32(S / np.where(q == 0, 1.0, dq)), FLT_MAX))
    c = e2m1_encode(f32(blk * rr[..., None]))
    return c.reshape(r, k), q


def nvfp4_dequant_rows(nibbles, q, amax):
    r, k = nibbles.shape
    S = nvfp4_global_scale(amax)
    d = e2m1_decode(nibbles).reshape(r, k // NV_BLOCK, NV_BLOCK) * e4m3_decode(q)[..., None] / S
    return d.reshape(r, k)


def nvfp4_col_values(x_group, padded_rows, rht, mask):
    """Group rows [m_g, K] -> column-wise values [K, P_g] (RHT along tokens when ``rht``)."""
    m, k = x_group.shape
    t = np.zeros((k, padded_rows), dtype=np.float64)
    t[:, :m] = x_group.T
    if rht:
        t = rht16(t.reshape(k, padded_rows // RHT_BLOCK, RHT_BLOCK), mask).reshape(k, padded_rows)
    return t


def nvfp4_group_quantize_with_amax(x_bits, m_splits, amax_pre, amax_post, mask,
                                   row=True, col=True, rht=True):
    """NVFP4 group quantize with given per-group amax.

    Row-wise casts use the group's pre-RHT amax and no transform; column-wise casts
    transform each 16-token block (when ``rht``) and use the group's post-RHT amax.
    Returns a dict like ``mxfp8_group_quantize`` with packed data.
    """
    x = bf16_bits_to_f64(x_bits)
    m_total, k = x.shape
    assert sum(m_splits) == m_total
    out = {}
    off = 0
    row_c = np.zeros((m_total, k), dtype=np.uint8)
    row_s = np.zeros((m_total, k // NV_BLOCK), dtype=np.uint8)
    groups, data, scales = [], [], []
    for g, m in enumerate(m_splits):
        xg = x[off:off + m]
        if row and m:
            c, q = nvfp4_quantize_rows(xg, amax_pre[g])
            row_c[off:off + m] = c
            row_s[off:off + m] = q
        if col:
            p = padded(m)
            vals = nvfp4_col_values(xg, p, rht, mask)
            c, q = nvfp4_quantize_rows(vals, amax_post[g])
            groups.append((pack_fp4(c), q))
            data.append(pack_fp4(c).reshape(-1))
            scales.append(q.reshape(-1))
        off += m
    if row:
        out["row_nibbles"] = row_c
        out["row_data"] = pack_fp4(row_c)
        out["row_scale"] = row_s
    if col:
        out["col_groups"] = groups
        out["col_data"] = np.concatenate(data) if data else np.zeros(0, np.uint8)
        out["col_scale"] = np.concatenate(scales) if scales else np.zeros(0, np.uint8)
    return out


def nvfp4_dequant_packed(packed, q, amax):
    return nvfp4_dequant_rows(unpack_fp4(packed), q, amax)
