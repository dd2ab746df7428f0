"""16x16 randomized Hadamard transform (RHT) with a sign mask, and the group amax.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "Reduce NVFP4 quantization work for the fused GroupedMLP fc2 input with
activation recompute" -- Changes (the quantizer's ``rht_sign_mask``; a post-RHT
amax computed for the plain transform leaves the global scale off by the sign
pattern) and the commit on passing the RHT sign mask to the Hadamard-fused GEMM
kernel (the fused kernel's amax values are rounded the same way the quantizer
rounds its data, so they agree with the standalone pass bit for bit;
``nvfp4_group_hadamard_amax`` returns the pre- and post-RHT amax of each group).

The pages fix neither the matrix nor where the signs go.  Readings:
* The transform acts on 16 consecutive tokens of one feature column of one
  group (the column-wise cast runs along tokens), the group's last block padded
  with zeros.
* Signs multiply the input BEFORE the Hadamard: u_j = s_j * x_j with s_j = -1
  when bit j of the 16-bit mask is set.  A sign applied after the Hadamard
  leaves every |y| and so the amax unchanged, which contradicts the pages'
  statement that ignoring the mask changes the global scale.
* y = 0.25 * H16 u with H16 the Sylvester Hadamard matrix
  H[i][j] = (-1)^popcount(i & j) (so 0.25 * H16 is orthogonal), evaluated as
  the fp32 butterfly over strides 1, 2, 4, 8, each stage replacing
  (v[i], v[i+h]) by (v[i] + v[i+h], v[i] - v[i+h]) for i with (i & h) == 0,
  then the exact multiply by 0.25.
* The result is rounded to bf16 (round to nearest even) -- the reading of the
  amax being rounded the way the quantizer rounds: the quantizer sees bf16 data.
"""
import numpy as np

from .formats import f32, round_bf16, bf16_bits_to_f64

RHT_BLOCK = 16


def hadamard16():
    """Sylvester Hadamard matrix of order 16, entries (-1)^popcount(i & j)."""
    i = np.arange(16)
    pc = np.array([[bin(a & b).count("1") for b in i] for a in i])
    return np.where(pc % 2 == 0, 1.0, -1.0)


def sign_vector(mask):
    """s_j = -1 where bit j of the 16-bit mask is set, else +1."""
    return np.array([-1.0 if (int(mask) >> j) & 1 else 1.0 for j in range(16)])


def rht16(blocks, mask):
    """Apply the signed 16-point transform to the last axis (length 16) of ``blocks``.

    ``blocks`` holds bf16 values as fp64.  Returns the bf16-rounded outputs as fp64.
    """
    v = np.array(blocks, dtype=np.float64) * sign_vector(mask)     # exact
    for h in (1, 2, 4, 8):
        for i in range(16):
            if i & h:
                continue
            a = v[..., i].copy()
            b = v[..., i + h].copy()
            v[..., i] = f32(a + b)
            v[..., i + h] = f32(a - b)
    y = f32(v * 0.25)
    return round_bf16(y)


def col_blocks(x_group, padded_rows):
    """Group rows [m_g, K] (fp64) -> [K, padded_rows/16, 16]: column k's tokens in 16-blocks, zero padded."""
    m, k = x_group.shape
    t = np.zeros((k, padded_rows), dtype=np.float64)
    t[:, :m] = x_group.T
    return t.reshape(k, padded_rows // RHT_BLOCK, RHT_BLOCK)


def group_hadamard_amax(x_bits, m_splits, mask, pad_to=128):
    """Per-group (pre-RHT amax, post-RHT amax), as fp32 values.

    pre_g  = max |x| over the rows of group g;
    post_g = max |RHT(block)| over every 16-token block of every column of group g
             (blocks taken over the group's rows zero-padded to a multiple of ``pad_to``;
             the all-zero padding blocks contribute 0).
    An empty group gives (0, 0).
    """
    x = bf16_bits_to_f64(x_bits)
    pre, post = [], []
    off = 0
    for m in m_splits:
        xg = x[off:off + m]
        off += m
        if m == 0:
            pre.append(0.0)
            post.append(0.0)
            continue
        pre.append(float(np.max(np.abs(xg))))
        p = -(-m // pad_to) * pad_to
        y = rht16(col_blocks(xg, p), mask)
        post.append(float(np.max(np.abs(y))))
    return np.array(pre, dtype=np.float32), np.array(post, dtype=np.float32)
