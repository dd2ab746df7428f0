"""Pins for the oracle's MXFP8 / NVFP4 block quantization and layouts (CPU only)."""
import numpy as np
import pytest

from conftest import read_golden
from oracle import formats as F
from oracle import quant as Q
from workloads import random_bf16, to_bf16_bits


def _blocks(name, header_fields):
    blocks, cur = [], None
    for line in read_golden(name):
        parts = line.split()
        if parts[0] == "block":
            cur = {"hdr": parts[1:1 + header_fields], "vals": [], "codes": []}
            blocks.append(cur)
        else:
            cur["vals"].append(float(parts[0]))
            cur["codes"].append(int(parts[1], 16))
    return blocks


def _bf16(vals):
    return to_bf16_bits(np.array(vals, dtype=np.float32))


# ----------------------------------------------------------------------------- MXFP8
def test_mxfp8_hand_worked_blocks():
    for blk in _blocks("mxfp8_blocks.txt", 1):
        assert len(blk["vals"]) == 32
        v = F.bf16_bits_to_f64(_bf16(blk["vals"]))[None, :]
        q, s = Q.mxfp8_quantize_rows(v)
        assert int(s[0, 0]) == int(blk["hdr"][0])
        assert q[0].tolist() == blk["codes"], (q[0].tolist(), blk["codes"])


@pytest.mark.parametrize("k", [-20, -1, 0, 3, 40])
def test_mxfp8_closed_forms(k):
    rng = np.random.default_rng(k + 100)
    # amax = 448 * 2^k -> X = k; the amax element encodes exactly as the max code
    v = rng.uniform(-1, 1, size=32) * 448 * 2.0 ** k
    v[7] = -448 * 2.0 ** k
    v = F.round_bf16(v)
    q, s = Q.mxfp8_quantize_rows(v[None])
    assert int(s[0, 0]) == k + 127
    assert int(q[0, 7]) == 0xFE
    # amax = 2^k -> X = k - 8 and the amax element becomes exactly 256 (code 0x78)
    v = F.round_bf16(rng.uniform(-1, 1, size=32) * 2.0 ** k)
    v[3] = 2.0 ** k
    q, s = Q.mxfp8_quantize_rows(v[None])
    assert int(s[0, 0]) == k - 8 + 127
    assert int(q[0, 3]) == 0x78
    assert F.e4m3_decode(q[0, 3]) * 2.0 ** (k - 8) == 2.0 ** k


def test_mxfp8_constant_and_zero_blocks():
    v = np.full((1, 64), 3.0)
    v[0, 32:] = 0.0
    v[0, 40] = -0.0
    q, s = Q.mxfp8_quantize_rows(v)
    assert s.tolist() == [[1 + 127 - 8, 127]]          # floor(log2 3) = 1 -> X = -7
    assert set(q[0, :32].tolist()) == {int(F.e4m3_encode(3.0 * 2 ** 7))}
    assert q[0, 32:].tolist() == [0x80 if i == 8 else 0 for i in range(32)]


def test_mxfp8_nearest_and_error_bound():
    """Every element is the nearest E4M3 value to v * 2^-X (brute force) and no block overflows."""
    x = random_bf16((64, 128), seed=3, dist="wide")
    v = F.bf16_bits_to_f64(x)
    q, s = Q.mxfp8_quantize_rows(v)
    X = s.astype(np.int64) - 127
    scaled = v.reshape(64, 4, 32) * np.ldexp(1.0, -X)[..., None]
    # the scaled block max lies in [256, 512) unless the exponent was clamped
    amax = np.max(np.abs(scaled), axis=-1)
    unclamped = (X > -127) & (X < 127)
    assert np.all((amax[unclamped] >= 256) & (amax[unclamped] < 512))
    dec = F.e4m3_decode(q).reshape(64, 4, 32)
    mags = F.E4M3_VALUES[:127]
    best = np.min(np.abs(np.abs(scaled)[..., None] - mags), axis=-1)
    assert np.all(np.abs(np.abs(dec) - np.minimum(np.abs(scaled), 448)) <= best + 0.0)
    # relative error of normal-range elements is at most 2^-4
    deq = Q.mxfp8_dequant_rows(q, s).reshape(64, 4, 32)
    big = np.abs(scaled) >= 2.0 ** -6
    err = np.abs(deq - v.reshape(64, 4, 32))[big & (np.abs(scaled) <= 448)]
    assert np.all(err <= np.abs(v.reshape(64, 4, 32))[big & (np.abs(scaled) <= 448)] * 2.0 ** -4)


def test_mxfp8_group_col_layout():
    """Column-wise data = per-group transpose, zero padded to 128, quantized along tokens."""
    splits = [0, 1, 31, 33, 0, 64]
    k = 64
    x = random_bf16((sum(splits), k), seed=4)
    out = Q.mxfp8_group_quantize(x, splits)
    offs = Q.col_offsets(splits)
    assert offs.tolist() == [0, 0, 128, 256, 384, 384, 512]
    v = F.bf16_bits_to_f64(x)
    row_off = np.concatenate([[0], np.cumsum(splits)])
    for g, m in enumerate(splits):
        p = Q.padded(m)
        data = out["col_data"][k * offs[g]:k * offs[g + 1]].reshape(k, p)
        scale = out["col_scale"][k * offs[g] // 32:k * offs[g + 1] // 32].reshape(k, p // 32)
        if p == 0:
            continue
        t = np.zeros((k, p))
        t[:, :m] = v[row_off[g]:row_off[g] + m].T
        q2, s2 = Q.mxfp8_quantize_rows(t)
        assert np.array_equal(data, q2) and np.array_equal(scale, s2)
        # the padding tokens encode as +0
        assert np.all(data[:, m:] == 0)
    assert out["col_data"].size == k * offs[-1]


def test_mfma_scale_layout_is_a_permutation():
    s = np.arange(3 * 6, dtype=np.uint8).reshape(3, 6) + 1
    w = Q.mfma_scale_layout(s)
    assert w.shape == (2, 3)
    # word (t, r) = blocks 4t..4t+3 of row r, missing blocks = 127
    assert w[0, 1] == (7 | 8 << 8 | 9 << 16 | 10 << 24)
    assert w[1, 2] == (17 | 18 << 8 | 127 << 16 | 127 << 24)
    back = np.stack([(w >> (8 * i)) & 0xFF for i in range(4)], axis=-1)    # [2, 3, 4]
    back = back.transpose(1, 0, 2).reshape(3, 8)[:, :6]
    assert np.array_equal(back, s)


# ----------------------------------------------------------------------------- NVFP4
def test_nvfp4_hand_worked_blocks():
    blocks = _blocks("nvfp4_blocks.txt", 2)
    for blk in blocks:
        amax = float(blk["hdr"][0])
        assert Q.nvfp4_global_scale(amax) == 448.0
        v = F.bf16_bits_to_f64(_bf16(blk["vals"]))[None, :]
        c, q = Q.nvfp4_quantize_rows(v, amax)
        assert int(q[0, 0]) == int(blk["hdr"][1], 16), (hex(int(q[0, 0])), blk["hdr"])
        assert c[0].tolist() == blk["codes"], (c[0].tolist(), blk["codes"])


def _nvfp4_block_alt(v, amax, s_order="ours", r_order="ours"):
    """The NVFP4 block cast of one row with one step done in another order (planted mistakes for
    the fixture test below; "ours" everywhere is the oracle's reading)."""
    S = Q.nvfp4_global_scale(amax)
    b = float(np.max(np.abs(v)))
    s = {"ours": F.f32(F.f32(b / 6) * S), "exact": F.f32(b * S / 6), "bS/6": F.f32(F.f32(b * S) / 6),
         "S/6": F.f32(b * F.f32(S / 6))}[s_order]
    q = int(F.e4m3_encode(s))
    d = float(F.e4m3_decode(q))
    if q == 0:
        return q, [int(c) for c in F.e2m1_encode(v * 0.0)]
    x = {"ours": F.f32(v * F.f32(S / d)), "exact": v * S / d, "dec/S": F.f32(v / F.f32(d / S)),
         "1/dec": F.f32(v * F.f32(S * F.f32(1 / d)))}[r_order]
    return q, [int(c) for c in F.e2m1_encode(x)]


def test_nvfp4_hand_worked_blocks_inexact_global_scale():
    """Blocks at group amaxes 5, 7.25 and 13 (global scales 537.59998, 370.75861, 206.76923) worked
    by hand with exact arithmetic: scale codes and nibbles, and S itself."""
    blocks = _blocks("nvfp4_blocks_inexact.txt", 3)
    assert len(blocks) == 8
    for blk in blocks:
        amax, S = float(blk["hdr"][0]), float(blk["hdr"][1])
        assert Q.nvfp4_global_scale(amax) == S
        v = F.bf16_bits_to_f64(_bf16(blk["vals"]))[None, :]
        assert np.array_equal(v[0], np.array(blk["vals"])), "fixture values must be bf16"
        c, q = Q.nvfp4_quantize_rows(v, amax)
        assert int(q[0, 0]) == int(blk["hdr"][2], 16), (hex(int(q[0, 0])), blk["hdr"])
        assert c[0].tolist() == blk["codes"], (c[0].tolist(), blk["codes"])
        assert _nvfp4_block_alt(v[0], amax) == (int(q[0, 0]), c[0].tolist())


@pytest.mark.parametrize("s_order,r_order", [("exact", "ours"), ("bS/6", "ours"), ("S/6", "ours"),
                                             ("ours", "exact"), ("ours", "dec/S"), ("ours", "1/dec")])
def test_nvfp4_inexact_blocks_catch_other_step_orders(s_order, r_order):
    """Planted mistake: one fp32 step of the block cast in another order.  At least one hand-worked
    block must then disagree with the fixture."""
    diffs = 0
    for blk in _blocks("nvfp4_blocks_inexact.txt", 3):
        v = F.bf16_bits_to_f64(_bf16(blk["vals"]))
        q, c = _nvfp4_block_alt(v, float(blk["hdr"][0]), s_order, r_order)
        diffs += (q != int(blk["hdr"][2], 16)) or (c != blk["codes"])
    assert diffs > 0


def test_nvfp4_global_scale_edges():
    assert Q.nvfp4_global_scale(0.0) == 1.0
    assert Q.nvfp4_global_scale(6.0) == 448.0
    assert Q.nvfp4_global_scale(1e-45) == F.FLT_MAX          # overflow clips to FLT_MAX
    assert Q.nvfp4_global_scale(3.0) == 896.0


def test_nvfp4_amax_block_closed_form():
    """A block holding the group amax gets scale code 0x7E and its max element becomes +-6."""
    rng = np.random.default_rng(5)
    for _ in range(200):
        amax = float(F.round_bf16(np.exp(rng.uniform(-30, 30))))
        v = F.round_bf16(rng.uniform(-1, 1, 16) * amax)
        i = rng.integers(16)
        v[i] = amax * (1 if rng.random() < 0.5 else -1)
        c, q = Q.nvfp4_quantize_rows(v[None], amax)
        assert int(q[0, 0]) == 0x7E
        assert F.e2m1_decode(c[0, i]) == np.sign(v[i]) * 6.0


def test_nvfp4_nearest_element():
    """Each element is the nearest E2M1 value to fp32(v * r) (brute force, ties even)."""
    x = random_bf16((8, 64), seed=6)
    v = F.bf16_bits_to_f64(x)
    amax = float(np.max(np.abs(v)))
    c, q = Q.nvfp4_quantize_rows(v, amax)
    S = Q.nvfp4_global_scale(amax)
    for r in range(8):
        for b in range(4):
            blk = v[r, b * 16:(b + 1) * 16]
            s = F.f32(F.f32(np.max(np.abs(blk)) / 6) * S)
            assert int(q[r, b]) == int(F.e4m3_encode(s))
            rr = F.f32(S / F.e4m3_decode(q[r, b]))
            for j in range(16):
                t = min(abs(F.f32(blk[j] * rr)), 6.0)
                d = np.abs(F.E2M1_MAGS - t)
                best = np.flatnonzero(d == d.min())
                want = best[0] if len(best) == 1 else [k for k in best if k % 2 == 0][0]
                assert int(c[r, b * 16 + j]) & 7 == want


def test_nvfp4_zero_elements_cast_to_signed_zero():
    """A zero element encodes as +0 (nibble 0x0) and -0 as 0x8 at any global scale, including one
    clipped to FLT_MAX (amax 1e-36), where S / dec(q) overflows for blocks below 6 / FLT_MAX and the
    reading clips it the same way; every other element encodes a finite E2M1 value."""
    rng = np.random.default_rng(9)
    tiny = [2.0 ** -127, 2.0 ** -130, 2.0 ** -133, 1e-38, 3e-39]
    for amax in (1e-36, 1e-30, 5.0, 1e30, 3e38):
        v = np.zeros((64, 16))
        v[:, 0] = rng.choice(tiny + [1e-3, 1.0, 100.0], size=64) * rng.choice([-1, 1], size=64)
        v[:, 1] = rng.choice(tiny, size=64)
        v[::2, 2:8] = -0.0
        v = F.round_bf16(v)
        c, q = Q.nvfp4_quantize_rows(v, amax)
        zero = v == 0
        assert np.all(c[zero & ~np.signbit(v)] == 0x0), amax
        assert np.all(c[zero & np.signbit(v)] == 0x8), amax
        assert np.all(np.isfinite(F.e2m1_decode(c))), amax


def test_nvfp4_zero_group_and_dequant_error():
    v = np.zeros((2, 32))
    c, q = Q.nvfp4_quantize_rows(v, 0.0)
    assert np.all(c == 0) and np.all(q == 0)
    x = random_bf16((16, 256), seed=7)
    v = F.bf16_bits_to_f64(x)
    amax = float(np.max(np.abs(v)))
    c, q = Q.nvfp4_quantize_rows(v, amax)
    d = Q.nvfp4_dequant_rows(c, q, amax)
    # NVFP4 relative Frobenius error on Gaussian data is around 10%
    err = np.linalg.norm(d - v) / np.linalg.norm(v)
    assert 0.03 < err < 0.2


def test_nvfp4_group_quantize_layout_and_rht_choice():
    splits = [5, 0, 40]
    k = 32
    x = random_bf16((45, k), seed=8)
    pre = np.array([1.0, 0.0, 2.0], np.float32)
    post = np.array([3.0, 0.0, 4.0], np.float32)
    out = Q.nvfp4_group_quantize_with_amax(x, splits, pre, post, 0x1234)
    v = F.bf16_bits_to_f64(x)
    # row-wise: group 2's rows with pre amax, no transform
    c, qq = Q.nvfp4_quantize_rows(v[5:45], 2.0)
    assert np.array_equal(out["row_nibbles"][5:45], c) and np.array_equal(out["row_scale"][5:45], qq)
    # column-wise: group 0 padded to 128 tokens, transformed, post amax
    t = np.zeros((k, 128))
    t[:, :5] = v[:5].T
    from oracle.rht import rht16
    y = rht16(t.reshape(k, 8, 16), 0x1234).reshape(k, 128)
    c0, q0 = Q.nvfp4_quantize_rows(y, 3.0)
    assert np.array_equal(out["col_groups"][0][0], F.pack_fp4(c0))
    assert np.array_equal(out["col_groups"][0][1], q0)
    assert out["col_data"].size == k * (128 + 0 + 128) // 2
    assert out["col_scale"].size == k * (128 + 0 + 128) // 16
