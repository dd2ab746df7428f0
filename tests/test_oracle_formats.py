"""Pins for the oracle's number formats (CPU only).

Each check ties ``oracle.formats`` to something other than itself: the OCP spec
landmarks in tests/golden, hand-derived rounding cases, brute-force nearest
searches over every code, and torch's own fp32 -> bf16 cast.
"""
import numpy as np
import pytest
import torch

from conftest import read_golden
from oracle import formats as F
from workloads import all_bf16_finite


def _parse_pairs(name, key_hex):
    rows = []
    for line in read_golden(name):
        a, b = line.split()
        if key_hex:
            rows.append((int(a, 16), float(b)))
        else:
            rows.append((float(a), int(b, 16)))
    return rows


def test_e4m3_spec_landmarks():
    for code, val in _parse_pairs("e4m3_spec.txt", True):
        got = F.e4m3_decode(code)
        if np.isnan(val):
            assert np.isnan(got), hex(code)
        else:
            assert got == val and np.signbit(got) == np.signbit(val), hex(code)


def test_e4m3_decode_structure():
    # 126 positive finite non-zero values, strictly increasing with the code
    pos = F.E4M3_VALUES[1:127]
    assert np.all(np.diff(pos) > 0)
    # negative half mirrors the positive half
    assert np.array_equal(F.E4M3_VALUES[128:255], -F.E4M3_VALUES[0:127])
    # each binade above the subnormals holds 8 values spaced 2^(e-10)
    for e in range(1, 16):
        vals = F.E4M3_VALUES[e * 8:e * 8 + 8]
        vals = vals[~np.isnan(vals)]
        assert np.allclose(np.diff(vals), 2.0 ** (e - 10))


def test_e4m3_encode_decode_identity():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(F.e4m3_encode(F.e4m3_decode(codes)), codes)


def test_e4m3_rounding_cases():
    for val, code in _parse_pairs("e4m3_rounding.txt", False):
        assert int(F.e4m3_encode(val)) == code, (val, hex(code), hex(int(F.e4m3_encode(val))))


def test_e4m3_encode_brute_force():
    """Against an exhaustive nearest search (ties -> even code) on random and tie values."""
    rng = np.random.default_rng(1)
    mags = F.E4M3_VALUES[:127]
    mids = (mags[1:] + mags[:-1]) / 2
    xs = np.concatenate([rng.standard_normal(3000) * 50, rng.standard_normal(2000) * 0.01,
                         mids, -mids, [0.0, -0.0, 447.9, 455.9, 456.0, 456.1, 1e9]])
    got = F.e4m3_encode(xs)
    for x, c in zip(xs, got):
        a = min(abs(x), 448.0)
        d = np.abs(mags - a)
        best = np.flatnonzero(d == d.min())
        want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        want |= 0x80 if np.signbit(x) else 0
        assert int(c) == want, (x, hex(int(c)), hex(want))


def test_e2m1_spec_and_rounding():
    for code, val in _parse_pairs("e2m1_spec.txt", True):
        got = F.e2m1_decode(code)
        assert got == val and np.signbit(got) == np.signbit(val)
    for val, code in _parse_pairs("e2m1_rounding.txt", False):
        assert int(F.e2m1_encode(val)) == code, (val, code)
    codes = np.arange(16, dtype=np.uint8)
    assert np.array_equal(F.e2m1_encode(F.e2m1_decode(codes)), codes)


def test_fp4_pack_order():
    nib = np.array([[1, 2, 3, 4, 0xF, 0]], dtype=np.uint8)
    packed = F.pack_fp4(nib)
    assert packed.tolist() == [[0x21, 0x43, 0x0F]]
    assert np.array_equal(F.unpack_fp4(packed), nib)


def test_e8m0_spec():
    for code, val in _parse_pairs("e8m0_spec.txt", True):
        got = F.e8m0_decode(code)
        assert (np.isnan(got) and np.isnan(val)) or got == val


def test_bf16_round_trip_all_patterns():
    bits = all_bf16_finite()
    assert np.array_equal(F.f64_to_bf16_bits(F.bf16_bits_to_f64(bits)), bits)


def test_bf16_rounding_matches_torch_on_fp32_values():
    """For inputs that are fp32 values the direct fp64->bf16 rounding equals torch's fp32->bf16 cast."""
    rng = np.random.default_rng(2)
    u = rng.integers(0, 1 << 32, size=200000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = F.f64_to_bf16_bits(f.astype(np.float64))
    assert np.array_equal(got, want)


def test_bf16_ties_and_fp32_emulation():
    # 1 + 2^-8 is the midpoint between 1 and 1 + 2^-7 -> even (1.0)
    assert F.round_bf16(1 + 2 ** -8) == 1.0
    assert F.round_bf16(1 + 3 * 2 ** -8) == 1 + 2 ** -6
    # a value just above the midpoint that fp32 would first round onto the midpoint
    v = 1 + 2 ** -8 + 2 ** -40
    assert F.round_bf16(v) == 1 + 2 ** -7
    assert F.f32(1 + 2 ** -30) == 1.0
    assert F.f32(1 / 3) == float(np.float32(1 / 3))
