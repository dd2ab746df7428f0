"""GPU parity of the group-quantize kernels with the CPU oracle: bit-exact on identical bf16 inputs."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_mxfp8_amd as g
from gpu_util import (assert_bytes_equal, bits16, col_total, dev_bf16, dev_f32, dev_splits, f32bits, u32, u8,
                      unpanel, unpanel_groups)
from oracle import formats as F
from oracle import quant as Q
from oracle import rht as R
from workloads import all_bf16_finite, random_bf16

pytestmark = pytest.mark.gpu

CASES = [
    ([64, 128], 128, "normal"),
    ([0, 1, 31, 33, 0, 300], 256, "normal"),
    ([517], 96, "wide"),
    ([200, 0, 57], 160, "srelu"),
    ([129, 255, 3], 384, "wide"),
]


def _check_mx(q, ref, splits, M, K, row=True, col=True):
    if row:
        assert_bytes_equal(unpanel(u8(q.bufs["row_data"])[:M * K], M, K), ref["row_data"], "row data")
        assert_bytes_equal(u8(q.bufs["row_scale"])[:M * K // 32], ref["row_scale"], "row scales")
        assert_bytes_equal(u32(q.bufs["row_scale_mfma"])[:((K + 127) // 128) * M], ref["row_scale_mfma"], "row mfma scales")
    if col:
        P = col_total(splits)
        assert_bytes_equal(unpanel_groups(u8(q.bufs["col_data"])[:K * P], K, splits), ref["col_data"], "col data")
        assert_bytes_equal(u8(q.bufs["col_scale"])[:K * P // 32], ref["col_scale"], "col scales")
        assert_bytes_equal(u32(q.bufs["col_scale_mfma"])[:K * P // 128], ref["col_scale_mfma"], "col mfma scales")


@pytest.mark.parametrize("splits,K,dist", CASES)
def test_mxfp8_group_quantize(splits, K, dist):
    M = sum(splits)
    print(f"mxfp8 group_quantize splits={splits} K={K} dist={dist}", flush=True)
    x = random_bf16((M, K), seed=M + K, dist=dist)
    q = g.group_quantize(dev_bf16(x), dev_splits(splits), g.recipe("mxfp8"), True, True)
    torch.cuda.synchronize()
    _check_mx(q, Q.mxfp8_group_quantize(x, splits), splits, M, K)


@pytest.mark.parametrize("order", ["sorted", "shuffled"])
def test_mxfp8_every_bf16_pattern(order):
    """All 65280 finite bf16 patterns, in blocks of similar magnitude (many scales) and shuffled."""
    v = all_bf16_finite()
    if order == "sorted":
        mag = v & 0x7FFF
        v = v[np.argsort(mag, kind="stable")]
    else:
        v = np.random.default_rng(0).permutation(v)
    K = 256
    M = -(-v.size // K)
    x = np.zeros(M * K, np.uint16)
    x[:v.size] = v
    x = x.reshape(M, K)
    splits = [100, M - 100]
    print(f"mxfp8 exhaustive sweep order={order} M={M}", flush=True)
    q = g.group_quantize(dev_bf16(x), dev_splits(splits), g.recipe("mxfp8"), True, True)
    torch.cuda.synchronize()
    _check_mx(q, Q.mxfp8_group_quantize(x, splits), splits, M, K)


def test_mxfp8_row_only_and_col_only():
    splits, K = [70, 0, 190], 256
    M = sum(splits)
    x = random_bf16((M, K), seed=11)
    ref = Q.mxfp8_group_quantize(x, splits)
    q = g.group_quantize(dev_bf16(x), dev_splits(splits), g.recipe("mxfp8"), True, False)
    torch.cuda.synchronize()
    _check_mx(q, ref, splits, M, K, row=True, col=False)
    q = g.group_quantize(dev_bf16(x), dev_splits(splits), g.recipe("mxfp8"), False, True)
    torch.cuda.synchronize()
    _check_mx(q, ref, splits, M, K, row=False, col=True)


def test_empty_input_and_clamped_splits():
    """M = 0 launches nothing harmful; splits that overrun M are clamped on the device and flagged."""
    q = g.group_quantize(dev_bf16(np.zeros((0, 128), np.uint16)), dev_splits([0, 0]), g.recipe("mxfp8"))
    torch.cuda.synchronize()
    splits_dev = dev_splits([100, 100])            # claims 200 rows, x has 150
    x = random_bf16((150, 128), seed=12)
    ws = g.quant_workspace(2, "cuda")
    q = g.group_quantize(dev_bf16(x), splits_dev, g.recipe("mxfp8"), True, True, ws=ws)
    torch.cuda.synchronize()
    assert g.read_device_flags(ws) & 2
    ref = Q.mxfp8_group_quantize(x, [100, 50])
    _check_mx(q, ref, [100, 50], 150, 128)


@pytest.mark.parametrize("splits,K,dist", CASES)
def test_nvfp4_hadamard_amax(splits, K, dist):
    M = sum(splits)
    mask = 0xB5E3
    print(f"nvfp4 hadamard amax splits={splits} K={K}", flush=True)
    x = random_bf16((M, K), seed=M * 3 + K, dist=dist)
    pre, post = g.group_hadamard_amax(dev_bf16(x), dev_splits(splits), mask)
    torch.cuda.synchronize()
    rpre, rpost = R.group_hadamard_amax(x, splits, mask)
    assert_bytes_equal(f32bits(pre), rpre.view(np.uint32), "pre-RHT amax")
    assert_bytes_equal(f32bits(post), rpost.view(np.uint32), "post-RHT amax")


def test_nvfp4_hadamard_amax_many_groups():
    """300 groups (many empty or tiny): the per-group slots span several finalize blocks, and two
    passes in a row start from cleared slots."""
    rng = np.random.default_rng(5)
    splits = [int(v) for v in rng.choice([0, 0, 1, 3, 17, 40, 130], size=300)]
    M, K, mask = sum(splits), 128, 0x5A5A
    print(f"nvfp4 amax, {len(splits)} groups, M={M}", flush=True)
    x = random_bf16((M, K), seed=77, dist="normal")
    rpre, rpost = R.group_hadamard_amax(x, splits, mask)
    dx, ds = dev_bf16(x), dev_splits(splits)
    ws = g.quant_workspace(len(splits), "cuda")
    for _ in range(2):
        pre, post = g.group_hadamard_amax(dx, ds, mask, ws=ws)
        torch.cuda.synchronize()
        assert_bytes_equal(f32bits(pre), rpre.view(np.uint32), "pre-RHT amax")
        assert_bytes_equal(f32bits(post), rpost.view(np.uint32), "post-RHT amax")


@pytest.mark.parametrize("splits,K,dist", CASES)
def test_nvfp4_group_quantize(splits, K, dist):
    """Amax pass + cast (row-wise with the pre-RHT amax, column-wise RHT with the post-RHT amax)."""
    M = sum(splits)
    mask = 0x6A0F
    print(f"nvfp4 group_quantize splits={splits} K={K}", flush=True)
    x = random_bf16((M, K), seed=M * 5 + K, dist=dist)
    rec = g.recipe("nvfp4", mask)
    q = g.group_quantize(dev_bf16(x), dev_splits(splits), rec, True, True)
    torch.cuda.synchronize()
    pre, post = R.group_hadamard_amax(x, splits, mask)
    ref = Q.nvfp4_group_quantize_with_amax(x, splits, pre, post, mask)
    assert_bytes_equal(f32bits(q.bufs["amax_pre"]), pre.view(np.uint32), "pre amax")
    assert_bytes_equal(f32bits(q.bufs["amax_post"]), post.view(np.uint32), "post amax")
    assert_bytes_equal(u8(q.bufs["row_data"])[:M * K // 2], ref["row_data"], "row data")
    assert_bytes_equal(u8(q.bufs["row_scale"])[:M * K // 16], ref["row_scale"], "row scales")
    P = col_total(splits)
    assert_bytes_equal(u8(q.bufs["col_data"])[:K * P // 2], ref["col_data"], "col data")
    assert_bytes_equal(u8(q.bufs["col_scale"])[:K * P // 16], ref["col_scale"], "col scales")


def test_nvfp4_quantize_with_given_amax():
    """The cast reads the amax it is given (the recompute path re-uses the forward's)."""
    splits, K, mask = [33, 0, 160], 128, 0x0F0F
    M = sum(splits)
    x = random_bf16((M, K), seed=21, dist="srelu")
    pre = np.array([3.0, 0.0, 1.5], np.float32)        # deliberately not the data's amax
    post = np.array([2.5, 0.0, 7.0], np.float32)
    q = g.group_quantize_with_amax(dev_bf16(x), dev_splits(splits), g.recipe("nvfp4", mask), dev_f32(pre),
                                   dev_f32(post), True, True)
    torch.cuda.synchronize()
    ref = Q.nvfp4_group_quantize_with_amax(x, splits, pre, post, mask)
    assert_bytes_equal(u8(q.bufs["row_data"])[:M * K // 2], ref["row_data"], "row data")
    assert_bytes_equal(u8(q.bufs["row_scale"])[:M * K // 16], ref["row_scale"], "row scales")
    P = col_total(splits)
    assert_bytes_equal(u8(q.bufs["col_data"])[:K * P // 2], ref["col_data"], "col data")
    assert_bytes_equal(u8(q.bufs["col_scale"])[:K * P // 16], ref["col_scale"], "col scales")


def _nv_values_bf16(packed, scales):
    """bf16 bits of dec(E2M1) * dec(E4M3) for the oracle's packed codes [R, C/2] and scales [R, C/16]."""
    nib = F.unpack_fp4(packed)
    vals = F.e2m1_decode(nib) * np.repeat(F.e4m3_decode(scales), 16, axis=-1)
    return F.f64_to_bf16_bits(vals)


def _unpanel16(buf, R, C):
    """bf16 operand panels (2-byte elements, 32 per 64-byte row) -> [R, C] uint16."""
    return np.ascontiguousarray(unpanel(np.asarray(buf).reshape(-1)[:2 * R * C], R, 2 * C)).view(np.uint16)


def test_nvfp4_bf16_panels():
    """The cast's bf16 GEMM panels hold exactly dec(E2M1) dec(E4M3) of the oracle's codes, row-wise and
    per group column-wise (RHT), next to the packed form."""
    splits, K, mask = [33, 0, 160, 200], 256, 0x2D4B
    M, G = sum(splits), len(splits)
    print(f"nvfp4 bf16 panels splits={splits} K={K}", flush=True)
    x = random_bf16((M, K), seed=41, dist="wide")
    rec = g.recipe("nvfp4", mask)
    q = g.alloc_grouped_q(rec, M, K, G, True, True)
    PR = g.col_rows_bound(M, G)
    q.bufs["row_bf16"] = torch.empty(2 * M * K, dtype=torch.uint8, device="cuda")
    q.bufs["col_bf16"] = torch.empty(2 * K * PR, dtype=torch.uint8, device="cuda")
    g.group_quantize(dev_bf16(x), dev_splits(splits), rec, True, True, out=q)
    torch.cuda.synchronize()
    pre, post = R.group_hadamard_amax(x, splits, mask)
    ref = Q.nvfp4_group_quantize_with_amax(x, splits, pre, post, mask)
    assert_bytes_equal(u8(q.bufs["row_data"])[:M * K // 2], ref["row_data"], "row data")
    assert_bytes_equal(_unpanel16(u8(q.bufs["row_bf16"]), M, K), _nv_values_bf16(ref["row_data"].reshape(M, K // 2),
                                                                               ref["row_scale"]), "row bf16 panels")
    col = u8(q.bufs["col_bf16"])
    off = 0
    for gi, (packed, sc) in enumerate(ref["col_groups"]):
        P = -(-splits[gi] // 128) * 128
        if P:
            assert_bytes_equal(_unpanel16(col[2 * off:2 * (off + K * P)], K, P), _nv_values_bf16(packed, sc),
                               f"col bf16 panels of group {gi}")
        off += K * P


@pytest.mark.parametrize("kind", ["mxfp8", "nvfp4"])
def test_weight_quantize(kind):
    """fprop operand (blocks along K) and dgrad operand (W_e^T, blocks along N), stacked and discrete."""
    from oracle.mlp import Recipe, quantize_weight
    E, N, K = 3, 256, 384
    w = random_bf16((E, N, K), seed=31, std=0.05)
    rec = g.recipe(kind)
    ref, _ = quantize_weight(w, Recipe(kind))
    wd = dev_bf16(w.reshape(E * N, K)).view(E, N, K)
    for q in (g.weight_quantize(wd, rec), g.weight_quantize([wd[e] for e in range(E)], rec)):
        torch.cuda.synchronize()
        if kind == "mxfp8":
            rows = u8(q.bufs["row_data"]).reshape(E, N * K)
            got = np.stack([unpanel(rows[e], N, K) for e in range(E)])
            assert_bytes_equal(got, np.stack([r[0] for r in ref["row"]]), "w row data")
            want = np.concatenate([Q.mfma_scale_layout(r[1]).reshape(-1) for r in ref["row"]])
            assert_bytes_equal(u32(q.bufs["row_scale_mfma"]), want, "w row mfma scales")
            cols = u8(q.bufs["col_data"]).reshape(E, N * K)
            got = np.stack([unpanel(cols[e], K, N) for e in range(E)])
            assert_bytes_equal(got, np.stack([r[0] for r in ref["colT"]]), "w col data")
            want = np.concatenate([Q.mfma_scale_layout(r[1]).reshape(-1) for r in ref["colT"]])
            assert_bytes_equal(u32(q.bufs["col_scale_mfma"]), want, "w col mfma scales")
        else:
            assert_bytes_equal(f32bits(q.bufs["amax_pre"]), ref["amax"].view(np.uint32), "w amax")
            assert_bytes_equal(u8(q.bufs["row_data"]), np.stack([r[0] for r in ref["row"]]), "w row data")
            assert_bytes_equal(u8(q.bufs["row_scale"]), np.stack([r[1] for r in ref["row"]]), "w row scales")
            assert_bytes_equal(u8(q.bufs["col_data"]), np.stack([r[0] for r in ref["colT"]]), "w col data")
            assert_bytes_equal(u8(q.bufs["col_scale"]), np.stack([r[1] for r in ref["colT"]]), "w col scales")
            rb, cb = u8(q.bufs["row_bf16"]), u8(q.bufs["col_bf16"])
            for e in range(E):
                n2 = 2 * N * K
                assert_bytes_equal(_unpanel16(rb[e * n2:(e + 1) * n2], N, K), _nv_values_bf16(*ref["row"][e]),
                                   f"w row bf16 panels, expert {e}")
                assert_bytes_equal(_unpanel16(cb[e * n2:(e + 1) * n2], K, N), _nv_values_bf16(*ref["colT"][e]),
                                   f"w col bf16 panels, expert {e}")
