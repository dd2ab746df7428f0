"""Pins for the oracle's signed 16-point Hadamard transform and group amax (CPU only)."""
import numpy as np

from conftest import read_golden
from oracle import formats as F
from oracle import rht as R
from workloads import random_bf16, to_bf16_bits


def _cases():
    out, cur = [], None
    for line in read_golden("rht_blocks.txt"):
        if line.startswith("case"):
            cur = {"mask": int(line.split()[1], 16)}
            out.append(cur)
        elif line.startswith("x:"):
            cur["x"] = np.array([float(t) for t in line[2:].split()])
        elif line.startswith("y:"):
            cur["y"] = np.array([float(t) for t in line[2:].split()])
    return out


def test_hand_worked_blocks():
    for c in _cases():
        assert np.array_equal(R.rht16(c["x"][None], c["mask"])[0], c["y"]), c


def test_hadamard_orthogonal():
    h = R.hadamard16()
    assert np.array_equal(h @ h.T, 16 * np.eye(16))
    assert np.array_equal(h, h.T)
    # Sylvester recursion H_2n = [[H, H], [H, -H]]
    h8 = h[:8, :8]
    assert np.array_equal(h, np.block([[h8, h8], [h8, -h8]]))


def test_butterfly_equals_matrix_on_exact_inputs():
    """Small-integer inputs keep every butterfly sum exact, so the fp32 butterfly must equal the matrix."""
    rng = np.random.default_rng(9)
    h = R.hadamard16()
    for _ in range(50):
        mask = int(rng.integers(0, 1 << 16))
        x = rng.integers(-64, 65, size=(4, 16)).astype(np.float64)
        want = 0.25 * (x * R.sign_vector(mask)) @ h.T
        got = R.rht16(x, mask)
        assert np.array_equal(got, F.round_bf16(want))


def test_sign_vector_bits():
    s = R.sign_vector(0b1000000000000101)
    assert s.tolist() == [-1, 1, -1] + [1] * 12 + [-1]


def test_zero_mask_is_the_plain_transform_and_constant_block():
    x = F.round_bf16(np.random.default_rng(10).standard_normal((8, 16)))
    h = R.hadamard16()
    plain = F.round_bf16(0.25 * x @ h.T)
    got = R.rht16(x, 0)
    # the fp32 butterfly may differ from the fp64 product by a rounding; allow 1 bf16 ulp
    ulp = np.ldexp(1.0, np.frexp(np.abs(plain) + 1e-300)[1] - 8)
    assert np.all(np.abs(got - plain) <= ulp)
    c = R.rht16(np.full((1, 16), 3.0), 0)[0]
    assert c[0] == 12.0 and np.all(c[1:] == 0)


def test_orthogonality_cancels_in_wgrad():
    """(T A)^T (T B) = A^T B for the exact transform T = blockdiag(0.25 H16 S)."""
    rng = np.random.default_rng(11)
    a = rng.standard_normal((64, 5))
    b = rng.standard_normal((64, 7))
    t16 = 0.25 * R.hadamard16() * R.sign_vector(0xBEEF)[None, :]
    t = np.kron(np.eye(4), t16)
    assert np.allclose((t @ a).T @ (t @ b), a.T @ b, atol=1e-12)


def test_group_amax_bounds_and_nonnegative_closed_form():
    splits = [0, 7, 32, 50]
    x = random_bf16((89, 48), seed=12, dist="srelu")
    v = F.bf16_bits_to_f64(x)
    pre, post = R.group_hadamard_amax(x, splits, 0)
    pre_m, post_m = R.group_hadamard_amax(x, splits, 0x5A5A)
    assert pre[0] == 0 and post[0] == 0 and post_m[0] == 0
    off = 0
    for g, m in enumerate(splits):
        if m:
            xg = v[off:off + m]
            assert pre[g] == np.max(np.abs(xg))
            # x >= 0: every |y_i| <= y_0 = sum/4, so the unsigned post amax is the largest block sum / 4
            p = -(-m // 128) * 128
            blocks = R.col_blocks(xg, p)
            sums = F.round_bf16(F.f32(np.max(np.sum(blocks, axis=-1)) / 4))
            assert abs(post[g] - sums) <= sums * 2 ** -7
            # a sign mask can only lower it for non-negative data
            assert post_m[g] <= post[g]
            # |y| <= 4 max|x| and max|y| >= max|x| / 4 (orthogonal rows of norm 1, 16 entries)
            assert pre[g] / 4 * (1 - 2 ** -7) <= post_m[g] <= 4 * pre[g] * (1 + 2 ** -7)
        off += m


def test_sign_mask_changes_post_amax_on_srelu_data():
    """Ignoring the mask overstates the post-RHT amax of SReLU-shaped activations.

    The pages report the resulting global scale up to ~17% too large; with
    channel-correlated non-negative activations the plain/signed ratio must be > 1,
    and a sign applied after the transform (which would not change |y|) is excluded.
    """
    rng = np.random.default_rng(13)
    m, k = 256, 256
    common = rng.standard_normal((m, 1))
    h = 0.5 * common + np.sqrt(0.75) * rng.standard_normal((m, k))
    a = np.maximum(h, 0) ** 2
    x = to_bf16_bits(a.astype(np.float32))
    ratios = []
    for mask in rng.integers(1, 1 << 16, size=8):
        _, plain = R.group_hadamard_amax(x, [m], 0)
        _, signed = R.group_hadamard_amax(x, [m], int(mask))
        ratios.append(plain[0] / signed[0])
    ratios = np.array(ratios)
    assert np.all(ratios >= 1.0)
    assert np.median(ratios) > 1.02
    assert np.max(ratios) < 3.0
