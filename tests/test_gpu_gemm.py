"""GPU parity of the grouped GEMMs on identical quantized operands: relative Frobenius error
<= 1e-3 against the oracle's fp64 product rounded to the output dtype, and bitwise equality
where the inputs make every product and sum exact."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_mxfp8_amd as g
from gpu_util import bits16, dev_bf16, dev_splits
from oracle import formats as F
from oracle import mlp as O
from workloads import random_bf16

pytestmark = pytest.mark.gpu

FPROP_CASES = [([0, 37, 300, 129], 256, 384), ([512], 128, 256), ([1, 0, 700], 384, 128), ([257, 3], 640, 512)]
WGRAD_CASES = [([0, 37, 300, 129], 256, 384), ([5, 0, 600], 128, 256), ([128, 256], 384, 128),
               # skewed experts: the XCD tile ranges are cut by work (one big expert, empty and
               # one-row experts; with 14 tiles some XCDs get none)
               ([3000, 1, 0, 40], 256, 128), ([2500, 3, 0, 7, 90, 0, 1], 384, 256)]


def _fprop_ref(x, w, splits, kind, mask):
    rec = O.Recipe(kind, mask)
    _, xd = O.quantize_activation(x, splits, rec, row=True, col=False)
    _, wd = O.quantize_weight(w, rec)
    out, off = [], 0
    for e, m in enumerate(splits):
        out.append(xd["row"][off:off + m] @ wd["row"][e].T)
        off += m
    return np.concatenate(out)


@pytest.mark.parametrize("kind", ["mxfp8", "nvfp4"])
@pytest.mark.parametrize("splits,N,K", FPROP_CASES)
def test_gemm_fprop(kind, splits, N, K):
    M, E, mask = sum(splits), len(splits), 0x3C5A
    print(f"gemm fprop {kind} splits={splits} N={N} K={K}", flush=True)
    x = random_bf16((M, K), seed=M + N)
    w = random_bf16((E, N, K), seed=K + N, std=1 / np.sqrt(K))
    rec = g.recipe(kind, mask)
    sd = dev_splits(splits)
    aq = g.group_quantize(dev_bf16(x), sd, rec, True, False)
    wq = g.weight_quantize(dev_bf16(w.reshape(E * N, K)).view(E, N, K), rec)
    c = g.grouped_gemm(g.GEMM_FPROP, rec, aq, wq, sd, M, N, K)
    c32 = g.grouped_gemm(g.GEMM_FPROP, rec, aq, wq, sd, M, N, K, out_dtype=g.OUT_FP32)
    torch.cuda.synchronize()
    ref = _fprop_ref(x, w, splits, kind, mask)
    got = F.bf16_bits_to_f64(bits16(c)).reshape(M, N)
    assert O.rel_fro(got, F.round_bf16(ref)) <= 1e-3
    # the fp32 result of the block-scaled MFMA is within ~2e-5 of the exact product
    assert O.rel_fro(c32.cpu().double().numpy(), ref) <= 5e-5


def _wgrad_ref(a, b, splits, kind, mask):
    rec = O.Recipe(kind, mask)
    _, ad = O.quantize_activation(a, splits, rec, row=False, col=True)
    _, bd = O.quantize_activation(b, splits, rec, row=False, col=True)
    return np.stack([ad["col"][e] @ bd["col"][e].T for e in range(len(splits))])


@pytest.mark.parametrize("kind", ["mxfp8", "nvfp4"])
@pytest.mark.parametrize("splits,Na,Nb", WGRAD_CASES)
def test_gemm_wgrad(kind, splits, Na, Nb):
    M, E, mask = sum(splits), len(splits), 0x91E7
    print(f"gemm wgrad {kind} splits={splits} Na={Na} Nb={Nb}", flush=True)
    a = random_bf16((M, Na), seed=M + Na)
    b = random_bf16((M, Nb), seed=M + Nb + 1, dist="srelu")
    rec = g.recipe(kind, mask)
    sd = dev_splits(splits)
    aq = g.group_quantize(dev_bf16(a), sd, rec, False, True)
    bq = g.group_quantize(dev_bf16(b), sd, rec, False, True)
    c = g.grouped_gemm(g.GEMM_WGRAD, rec, aq, bq, sd, M, Na, Nb)
    torch.cuda.synchronize()
    ref = _wgrad_ref(a, b, splits, kind, mask)
    got = F.bf16_bits_to_f64(bits16(c)).reshape(E, Na, Nb)
    assert O.rel_fro(got, F.round_bf16(ref)) <= 1e-3
    for e, m in enumerate(splits):
        if m == 0:
            assert np.all(got[e] == 0), "an empty expert must get a zero weight gradient"


def _tiny_expert_splits():
    """512 experts, most with one token, every 37th with 65, 129, 130 or 200 (odd stage counts),
    a few empty: 2 tiles per expert at Na = 256, Nb = 512, so each workgroup runs 4 tiles in a row,
    most of them of the shortest kind."""
    splits = [1] * 512
    for i, e in enumerate(range(5, 512, 37)):
        splits[e] = (65, 129, 130, 200)[i % 4]
    for e in (3, 200, 201, 450):
        splits[e] = 0
    return splits


@pytest.mark.parametrize("kind", ["mxfp8", "nvfp4"])
def test_gemm_wgrad_runs_of_tiny_experts(kind):
    """Weight gradients stop at the last 64-token stage (32 for bf16) that holds a token, so a
    tile may span an odd number of stages, but never fewer than two: the persistent kernel
    prefetches three stages ahead through a window of three tiles.  Sampled experts (a run of
    one-token experts, every larger one, an empty one) against the oracle."""
    splits, Na, Nb = _tiny_expert_splits(), 256, 512
    M, E, mask = sum(splits), len(splits), 0x2D4B
    print(f"gemm wgrad {kind} {E} tiny experts, M={M} Na={Na} Nb={Nb}", flush=True)
    a = random_bf16((M, Na), seed=41)
    b = random_bf16((M, Nb), seed=42, dist="srelu")
    rec = g.recipe(kind, mask)
    sd = dev_splits(splits)
    aq = g.group_quantize(dev_bf16(a), sd, rec, False, True)
    bq = g.group_quantize(dev_bf16(b), sd, rec, False, True)
    c = g.grouped_gemm(g.GEMM_WGRAD, rec, aq, bq, sd, M, Na, Nb)
    torch.cuda.synchronize()
    got = F.bf16_bits_to_f64(bits16(c)).reshape(E, Na, Nb)
    orec = O.Recipe(kind, mask)
    _, ad = O.quantize_activation(a, splits, orec, row=False, col=True)
    _, bd = O.quantize_activation(b, splits, orec, row=False, col=True)
    sample = sorted(set(range(100, 140)) | {e for e in range(E) if splits[e] > 1} | {200})
    ref = np.stack([ad["col"][e] @ bd["col"][e].T for e in sample])
    assert O.rel_fro(got[sample], F.round_bf16(ref)) <= 1e-3
    assert np.all(got[200] == 0), "an empty expert must get a zero weight gradient"


@pytest.mark.parametrize("kind", ["mxfp8", "nvfp4"])
def test_gemm_fprop_more_tiles_than_workgroups(kind):
    """287 tiles of 256 x 256 for one workgroup per CU: every workgroup takes a second tile and
    the last round is short (ragged and empty experts).  Within the GEMM tolerance of the oracle
    (bf16 and fp32 outputs), bitwise repeatable, and the bf16 output is the fp32 one rounded."""
    splits, N, K = [5000, 0, 3000, 2240], 1792, 2048
    M, E, mask = sum(splits), len(splits), 0x5A3C
    print(f"gemm fprop {kind} splits={splits} N={N} K={K}", flush=True)
    x = random_bf16((M, K), seed=31)
    w = random_bf16((E, N, K), seed=32, std=1 / np.sqrt(K))
    rec = g.recipe(kind, mask)
    sd = dev_splits(splits)
    aq = g.group_quantize(dev_bf16(x), sd, rec, True, False)
    wq = g.weight_quantize(dev_bf16(w.reshape(E * N, K)).view(E, N, K), rec)
    c = g.grouped_gemm(g.GEMM_FPROP, rec, aq, wq, sd, M, N, K)
    c2 = g.grouped_gemm(g.GEMM_FPROP, rec, aq, wq, sd, M, N, K)
    c32 = g.grouped_gemm(g.GEMM_FPROP, rec, aq, wq, sd, M, N, K, out_dtype=g.OUT_FP32)
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.int16), c2.view(torch.int16)), "not repeatable"
    ref = _fprop_ref(x, w, splits, kind, mask)
    got = F.bf16_bits_to_f64(bits16(c)).reshape(M, N)
    assert O.rel_fro(got, F.round_bf16(ref)) <= 1e-3
    assert O.rel_fro(c32.cpu().double().numpy(), ref) <= 5e-5
    # bf16 output = the fp32 output rounded (the same sum, converted once)
    assert torch.equal(c32.to(torch.bfloat16).view(torch.int16), c.view(torch.int16))


def _many_small_expert_splits():
    """64 experts of 0..500 rows (seeded), with the row counts at the 64-, 128- and 256-row
    boundaries spelled out: full and partial 256-row tiles (down to one valid row, and 64-row
    bands with none), in the expert-by-expert launch order (at most 512 rows per expert on
    average)."""
    rng = np.random.default_rng(77)
    s = list(rng.integers(0, 501, size=52))
    return s + [0, 1, 64, 65, 127, 128, 129, 255, 256, 257, 383, 384]


@pytest.mark.parametrize("kind", ["mxfp8", "nvfp4"])
def test_gemm_fprop_many_small_experts(kind):
    """More tiles than workgroups (540 tiles, three rounds) over 64 small experts, ordered
    expert by expert.  Within the GEMM tolerance of the oracle, every expert on its own too,
    bitwise repeatable, and the bf16 output is the fp32 one rounded."""
    splits, N, K = _many_small_expert_splits(), 1536, 256
    M, E, mask = sum(splits), len(splits), 0x1D2B
    print(f"gemm fprop many small experts {kind} M={M} E={E} N={N} K={K}", flush=True)
    x = random_bf16((M, K), seed=41)
    w = random_bf16((E, N, K), seed=42, std=1 / np.sqrt(K))
    rec = g.recipe(kind, mask)
    sd = dev_splits(splits)
    aq = g.group_quantize(dev_bf16(x), sd, rec, True, False)
    wq = g.weight_quantize(dev_bf16(w.reshape(E * N, K)).view(E, N, K), rec)
    c = g.grouped_gemm(g.GEMM_FPROP, rec, aq, wq, sd, M, N, K)
    c2 = g.grouped_gemm(g.GEMM_FPROP, rec, aq, wq, sd, M, N, K)
    c32 = g.grouped_gemm(g.GEMM_FPROP, rec, aq, wq, sd, M, N, K, out_dtype=g.OUT_FP32)
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.int16), c2.view(torch.int16)), "not repeatable"
    ref = _fprop_ref(x, w, splits, kind, mask)
    got = F.bf16_bits_to_f64(bits16(c)).reshape(M, N)
    assert O.rel_fro(got, F.round_bf16(ref)) <= 1e-3
    # every expert on its own (a wrong row mapping of one small tile would hide in the total)
    off = 0
    for e, m in enumerate(splits):
        if m:
            assert O.rel_fro(got[off:off + m], F.round_bf16(ref[off:off + m])) <= 2e-3, (e, m)
        off += m
    assert O.rel_fro(c32.cpu().double().numpy(), ref) <= 5e-5
    assert torch.equal(c32.to(torch.bfloat16).view(torch.int16), c.view(torch.int16))


@pytest.mark.parametrize("kind", ["mxfp8", "nvfp4"])
def test_gemm_wgrad_accumulates_into_fp32(kind):
    """WGRAD with OUT_FP32_ACCUMULATE adds the product to the fp32 tensor given, twice in a row:
    each result is bit for bit the fp32 sum of the previous contents and the plain fp32 output
    (an empty expert's slice stays as it was), and within the GEMM tolerance of the oracle's
    fp32(main_grad + dW)."""
    splits, Na, Nb = [300, 0, 37, 129], 256, 384
    M, E, mask = sum(splits), len(splits), 0x91E7
    print(f"gemm wgrad accumulate {kind} splits={splits} Na={Na} Nb={Nb}", flush=True)
    a = random_bf16((M, Na), seed=11)
    b = random_bf16((M, Nb), seed=12, dist="srelu")
    rec = g.recipe(kind, mask)
    sd = dev_splits(splits)
    aq = g.group_quantize(dev_bf16(a), sd, rec, False, True)
    bq = g.group_quantize(dev_bf16(b), sd, rec, False, True)
    c32 = g.grouped_gemm(g.GEMM_WGRAD, rec, aq, bq, sd, M, Na, Nb, out_dtype=g.OUT_FP32)
    torch.cuda.synchronize()
    c = c32.cpu().numpy()
    main0 = (np.random.default_rng(13).standard_normal((E, Na, Nb)) * c.std()).astype(np.float32)
    main = torch.from_numpy(main0).to("cuda")
    want = main0
    for _ in range(2):
        out = g.grouped_gemm(g.GEMM_WGRAD, rec, aq, bq, sd, M, Na, Nb, out_dtype=g.OUT_FP32_ACCUMULATE, out=main)
        assert out is main
        torch.cuda.synchronize()
        want = want + c
        assert np.array_equal(main.cpu().numpy().view(np.uint32), want.view(np.uint32))
    got = main.cpu().numpy()
    assert np.array_equal(got[1].view(np.uint32), main0[1].view(np.uint32)), "empty expert changed"
    ref = _wgrad_ref(a, b, splits, kind, mask)
    assert O.rel_fro(got.astype(np.float64), O.accumulate_main_grad(O.accumulate_main_grad(main0, ref), ref)) <= 5e-5


def test_gemm_exact_inputs_bitwise():
    """Small-integer data quantizes exactly to MXFP8 and every fp32 partial sum is exact, so the
    MFMA result equals the fp64 product and the bf16 outputs must match bit for bit."""
    rng = np.random.default_rng(5)
    splits, N, K = [96, 0, 300], 256, 512
    M, E = sum(splits), len(splits)
    from workloads import to_bf16_bits
    x = to_bf16_bits(rng.integers(-4, 5, size=(M, K)).astype(np.float32))
    w = to_bf16_bits(rng.integers(-4, 5, size=(E, N, K)).astype(np.float32))
    rec = g.recipe("mxfp8")
    sd = dev_splits(splits)
    aq = g.group_quantize(dev_bf16(x), sd, rec, True, True)
    wq = g.weight_quantize(dev_bf16(w.reshape(E * N, K)).view(E, N, K), rec)
    c = g.grouped_gemm(g.GEMM_FPROP, rec, aq, wq, sd, M, N, K)
    torch.cuda.synchronize()
    ref = _fprop_ref(x, w, splits, "mxfp8", 0)
    assert np.array_equal(bits16(c).reshape(M, N), F.f64_to_bf16_bits(ref))
    # wgrad on the same data: exact too
    c = g.grouped_gemm(g.GEMM_WGRAD, rec, aq, aq, sd, M, K, K)
    torch.cuda.synchronize()
    ref = _wgrad_ref(x, x, splits, "mxfp8", 0)
    assert np.array_equal(bits16(c).reshape(E, K, K), F.f64_to_bf16_bits(ref))
