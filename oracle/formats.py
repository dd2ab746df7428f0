"""Number formats, written out from their public definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* E4M3 ("E4M3FN"): OCP 8-bit Floating Point Specification v1.0 -- sign bit,
  4 exponent bits with bias 7, 3 mantissa bits, no infinities, S.1111.111 is
  NaN, largest finite magnitude 448, subnormals m * 2^-9.
* E8M0: OCP Microscaling Formats (MX) v1.0 -- an unsigned power of two
  2^(code - 127); code 0xFF is NaN.
* E2M1 (FP4): OCP MX v1.0 -- magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}.

The pages (the MXFP8 page: "32-element blocks, E4M3 data, E8M0 scales"; the
NVFP4 page: 16-element blocks with E4M3 block scales) name these formats but do
not define their bits, so the definitions above are the specs'.

Readings taken where the pages are silent:
* every encode rounds to nearest, ties to the even code (IEEE RNE);
* every encode saturates at the largest finite magnitude (448 for E4M3, 6 for
  E2M1) instead of producing NaN (OCP "satfinite");
* the sign of zero is kept: a negative input that rounds to zero encodes as
  0x80 (E4M3) or nibble 0x8 (E2M1).
"""
import numpy as np

FLT_MAX = float(np.finfo(np.float32).max)
BF16_MAX = float(np.float32(np.frombuffer(np.uint32(0x7F7F0000).tobytes(), np.float32)[0]))


def f32(x):
    """Round fp64 value(s) to the nearest fp32 (ties to even), returned as fp64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------- bf16
def bf16_bits_to_f64(bits):
    """bf16 bit patterns (uint16) -> exact fp64 values (a bf16 is the top half of an fp32)."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x):
    """Round fp64 value(s) directly to bf16 (8 significant bits, ties to even).

    Direct rounding from fp64 (no detour through fp32, which could round twice).
    Overflow past the largest bf16 goes to +-inf, as IEEE RNE does.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros(x.shape, dtype=np.float64)
    nz = (x != 0) & np.isfinite(x)
    _, e = np.frexp(x[nz])                      # |x| = m * 2^e, m in [0.5, 1)
    q_exp = np.maximum(e - 8, -133)             # exponent of one ulp (subnormal ulp 2^-133)
    q = np.rint(np.ldexp(x[nz], -q_exp))        # np.rint rounds half to even
    out[nz] = np.ldexp(q, q_exp)
    out[~nz] = x[~nz]
    big = np.abs(out) > BF16_MAX
    out[big] = np.copysign(np.inf, out[big])
    bits = (out.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return bits


def round_bf16(x):
    """fp64 -> nearest bf16 value, returned as fp64."""
    return bf16_bits_to_f64(f64_to_bf16_bits(x))


# ----------------------------------------------------------------------------- E4M3
def _e4m3_value(code):
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return np.nan
    if e == 0:
        return s * m * 2.0 ** -9               # subnormal: m/8 * 2^(1-7)
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_VALUES = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)
E4M3_MAX = 448.0


def e4m3_decode(codes):
    return E4M3_VALUES[np.asarray(codes).astype(np.int64)]


def _encode_nearest(a, mags):
    """Index of the nearest entry of the increasing table ``mags`` to a >= 0; ties -> even index."""
    idx = np.searchsorted(mags, a, side="left")
    hi = np.clip(idx, 0, len(mags) - 1)
    lo = np.clip(idx - 1, 0, len(mags) - 1)
    dlo = a - mags[lo]
    dhi = mags[hi] - a
    pick = np.where(dhi < dlo, hi, lo)
    tie = dhi == dlo
    even = np.where(lo % 2 == 0, lo, hi)
    return np.where(tie, even, pick)


def e4m3_encode(x):
    """fp64 -> E4M3 code: round to nearest even, saturate to +-448, keep the sign of zero."""
    x = np.asarray(x, dtype=np.float64)
    mags = E4M3_VALUES[:127]                    # codes 0x00..0x7E, increasing
    a = np.minimum(np.abs(x), E4M3_MAX)
    code = _encode_nearest(a, mags).astype(np.uint8)
    return code | (np.signbit(x).astype(np.uint8) << np.uint8(7))


# ----------------------------------------------------------------------------- E2M1
E2M1_MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E2M1_VALUES = np.concatenate([E2M1_MAGS, -E2M1_MAGS])
E2M1_MAX = 6.0


def e2m1_decode(nibbles):
    return E2M1_VALUES[np.asarray(nibbles).astype(np.int64) & 0xF]


def e2m1_encode(x):
    """fp64 -> E2M1 nibble: round to nearest even, saturate to +-6, keep the sign of zero."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E2M1_MAX)
    code = _encode_nearest(a, E2M1_MAGS).astype(np.uint8)
    return code | (np.signbit(x).astype(np.uint8) << np.uint8(3))


def pack_fp4(nibbles):
    """Pack E2M1 nibbles along the last axis: element 2i -> low nibble of byte i."""
    n = np.asarray(nibbles, dtype=np.uint8)
    return (n[..., 0::2] & 0xF) | ((n[..., 1::2] & 0xF) << 4)


def unpack_fp4(packed):
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


# ----------------------------------------------------------------------------- E8M0
def e8m0_decode(codes):
    c = np.asarray(codes).astype(np.int64)
    v = np.ldexp(1.0, c - 127)
    return np.where(c == 255, np.nan, v)
