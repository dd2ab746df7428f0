"""GPU checks against values fixed by hand or by exhaustive enumeration rather than by samples:

* the one-token grouped-MLP cases worked by hand (tests/golden/mlp_single_token.txt) through the
  fused forward + backward: every output exact (they pin the bf16 rounding of h, a, da and dh,
  the prob placement and the SwiGLU operand order on the kernels themselves);
* the NVFP4 blocks worked by hand at non-power-of-two global scales
  (tests/golden/nvfp4_blocks_inexact.txt) through the NVFP4 cast: scale codes and nibbles exact;
* every finite bf16 pattern through the NVFP4 cast at several global scales, row-wise and
  column-wise, with the Hadamard transform (activation casts) and without it (weight casts),
  bit for bit against the oracle;
* NVFP4 grouped GEMMs on operands whose products and sums are exact in fp32 and whose global
  scales are powers of two: bit for bit;
* the grouped GEMM in the dgrad orientation (the weight's column-wise operand as B) within the
  GEMM tolerance.
"""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_mxfp8_amd as g
from conftest import read_golden
from gpu_util import assert_bytes_equal, bits16, col_total, dev_bf16, dev_f32, dev_splits, f32bits, u8, unpanel
from oracle import formats as F
from oracle import mlp as O
from oracle import quant as Q
from oracle import rht as R
from workloads import all_bf16_finite, random_bf16, to_bf16_bits

pytestmark = pytest.mark.gpu


# ----------------------------------------------------------------------------- one-token cases
def _cases():
    cases, cur = [], None
    for line in read_golden("mlp_single_token.txt"):
        p = line.split()
        if p[0] == "case":
            kv = dict(zip(p[3::2], p[4::2]))
            cur = {"name": p[1], "act": p[2], "ffn": int(kv["ffn"]), "p": float(kv["p"]), "in": [], "out": []}
            cases.append(cur)
        else:
            cur[p[0]].append((p[1], tuple(int(v) for v in p[2:-1]), float(p[-1])))
    return cases


CASES = _cases()


@pytest.mark.parametrize("recompute", [False, True])
@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_single_token_cases_exact(case, recompute):
    """The hand-worked cases, zero-padded to hidden = ffn = 128 (the fused path's granularity)."""
    H = ffn = 128
    glu = case["act"] == "swiglu"
    F1 = 2 * ffn if glu else ffn

    def row(r):          # SwiGLU: the up half of W1 / dW1 starts at row ffn
        return r - case["ffn"] + ffn if (glu and r >= case["ffn"]) else r

    t = {"x": np.zeros((1, H)), "w1": np.zeros((1, F1, H)), "w2": np.zeros((1, H, ffn)), "dy": np.zeros((1, H))}
    for name, idx, v in case["in"]:
        idx = (idx[0], row(idx[1]), idx[2]) if name == "w1" else idx
        t[name][idx] = v
    want = {"y": np.zeros((1, H)), "dx": np.zeros((1, H)), "dprobs": np.zeros(1), "dw1": np.zeros((1, F1, H)),
            "dw2": np.zeros((1, H, ffn))}
    for name, idx, v in case["out"]:
        name = "dprobs" if name == "dprob" else name
        idx = (idx[0], row(idx[1]), idx[2]) if name == "dw1" else idx
        want[name][idx] = v
    print(f"one-token case {case['name']} recompute={recompute}", flush=True)
    dev = {k: dev_bf16(F.f64_to_bf16_bits(v).reshape(-1, v.shape[-1])).view(*v.shape) for k, v in t.items()}
    rec = g.recipe("mxfp8")
    w1q, w2q = g.weight_quantize(dev["w1"], rec), g.weight_quantize(dev["w2"], rec)
    splits = dev_splits([1])
    probs = dev_f32(np.array([case["p"]], np.float32))
    y, ctx = g.grouped_mlp_forward(dev["x"], splits, w1q, w2q, probs, case["act"], rec, recompute=recompute)
    out = g.grouped_mlp_backward(dev["dy"], splits, w1q, w2q, probs, ctx)
    torch.cuda.synchronize()
    got = {"y": y, "dx": out["dx"], "dprobs": out["dprobs"], "dw1": out["dw1"], "dw2": out["dw2"]}
    for k, v in got.items():
        host = v.detach().cpu().double().numpy()
        bad = np.argwhere(host != want[k])
        assert bad.size == 0, f"{k}: {len(bad)} entries differ, first {bad[:3].tolist()}: " \
                              f"got {host[tuple(bad[0])]}, want {want[k][tuple(bad[0])]}"


# ----------------------------------------------------------------------------- NVFP4 blocks at inexact S
def test_nvfp4_inexact_blocks_exact():
    """Each hand-worked block is one row (padded with a zero block to 32 elements) and its own
    group, cast row-wise with the block's group amax given."""
    blocks, cur = [], None
    for line in read_golden("nvfp4_blocks_inexact.txt"):
        p = line.split()
        if p[0] == "block":
            cur = {"amax": float(p[1]), "code": int(p[3], 16), "vals": [], "nib": []}
            blocks.append(cur)
        else:
            cur["vals"].append(float(p[0]))
            cur["nib"].append(int(p[1], 16))
    G = len(blocks)
    x = np.zeros((G, 32), np.float32)
    for i, b in enumerate(blocks):
        x[i, :16] = b["vals"]
    amax = np.array([b["amax"] for b in blocks], np.float32)
    rec = g.recipe("nvfp4", 0)
    q = g.group_quantize_with_amax(dev_bf16(to_bf16_bits(x)), dev_splits([1] * G), rec, dev_f32(amax),
                                   dev_f32(amax), True, False)
    torch.cuda.synchronize()
    data = u8(q.bufs["row_data"])[:G * 16].reshape(G, 16)
    scales = u8(q.bufs["row_scale"])[:G * 2].reshape(G, 2)
    nib = F.unpack_fp4(data)
    for i, b in enumerate(blocks):
        assert int(scales[i, 0]) == b["code"], (i, hex(int(scales[i, 0])), hex(b["code"]))
        assert nib[i, :16].tolist() == b["nib"], (i, nib[i, :16].tolist(), b["nib"])
        assert int(scales[i, 1]) == 0 and not nib[i, 16:].any()


# ----------------------------------------------------------------------------- exhaustive NVFP4 casts
# Group amaxes: the data's own amax, one whose global scale is inexact (5), a small one (2^-20:
# scale codes saturate for most blocks), a huge one (global scale below 1, many blocks cast to
# zero) and one whose global scale overflows fp32 and is clipped to FLT_MAX (1e-36; then
# S / dec(q) overflows too for blocks below 6 / FLT_MAX and is clipped the same way).
AMAXES = [None, 5.0, 2.0 ** -20, 3.0e38, 1.0e-36]


def _sweep_input(order, seed, limit_bits=None):
    """Every finite bf16 pattern (or those below a magnitude) as rows of 256, sorted by magnitude
    (blocks of similar values) or shuffled."""
    v = all_bf16_finite()
    if limit_bits is not None:
        v = v[(v & 0x7FFF) < limit_bits]
    if order == "sorted":
        v = v[np.argsort(v & 0x7FFF, kind="stable")]
    else:
        v = np.random.default_rng(seed).permutation(v)
    K = 256
    M = -(-v.size // K)
    x = np.zeros(M * K, np.uint16)
    x[:v.size] = v
    return x.reshape(M, K)


def _nv_values_bf16(packed, scales):
    """bf16 bits of dec(E2M1) * dec(E4M3) for the oracle's packed codes [R, C/2] and scales [R, C/16]."""
    nib = F.unpack_fp4(packed)
    vals = F.e2m1_decode(nib) * np.repeat(F.e4m3_decode(scales), 16, axis=-1)
    return F.f64_to_bf16_bits(vals)


def _unpanel16(buf, R, C):
    """bf16 operand panels (2-byte elements, 32 per 64-byte row) -> [R, C] uint16."""
    return np.ascontiguousarray(unpanel(np.asarray(buf).reshape(-1)[:2 * R * C], R, 2 * C)).view(np.uint16)


# The Hadamard transform sums 16 values: inputs of magnitude 2^124 and above can overflow fp32 in
# it, which is outside the casts' domain (finite inputs with a finite transform), so the
# column-wise sweep takes the patterns below 2^120 (bf16 bits 0x7B80).
RHT_LIMIT = 0x7B80


@pytest.mark.parametrize("direction", ["row", "col"])
@pytest.mark.parametrize("order", ["sorted", "shuffled"])
def test_nvfp4_every_bf16_pattern_activation_casts(order, direction):
    """All finite bf16 patterns, once per group amax in AMAXES (one group each), cast row-wise
    (pre-RHT amax, no transform) or column-wise (16x16 RHT along tokens, post-RHT amax)."""
    col = direction == "col"
    parts = [_sweep_input(order, seed, RHT_LIMIT if col else None) for seed in range(len(AMAXES))]
    x = np.concatenate(parts)
    splits = [p.shape[0] for p in parts]
    M, K = x.shape
    mask = 0x9A5F
    with np.errstate(all="ignore"):
        pre, post = R.group_hadamard_amax(x, splits, mask)
    own = post if col else pre
    amax = np.array([own[i] if a is None else a for i, a in enumerate(AMAXES)], np.float32)
    print(f"nvfp4 exhaustive sweep {direction} order={order}: M={M} K={K} groups={splits} amax={amax}", flush=True)
    rec = g.recipe("nvfp4", mask)
    # the bf16 GEMM panels too (the form the fused MLP's GEMMs read): every scale code and nibble
    # the sweep produces goes through the hardware E2M1 expansion
    q = g.alloc_grouped_q(rec, M, K, len(splits), not col, col)
    key = "col_bf16" if col else "row_bf16"
    q.bufs[key] = torch.zeros(2 * K * (g.col_rows_bound(M, len(splits)) if col else M), dtype=torch.uint8,
                              device="cuda")
    q = g.group_quantize_with_amax(dev_bf16(x), dev_splits(splits), rec, dev_f32(amax), dev_f32(amax),
                                   not col, col, out=q)
    torch.cuda.synchronize()
    ref = Q.nvfp4_group_quantize_with_amax(x, splits, amax, amax, mask, row=not col, col=col)
    if col:
        P = col_total(splits)
        assert_bytes_equal(u8(q.bufs["col_data"])[:K * P // 2], ref["col_data"], "col data")
        assert_bytes_equal(u8(q.bufs["col_scale"])[:K * P // 16], ref["col_scale"], "col scales")
        panels, off = u8(q.bufs[key]), 0
        for gi, (packed, sc) in enumerate(ref["col_groups"]):
            Pg = -(-splits[gi] // 128) * 128
            assert_bytes_equal(_unpanel16(panels[2 * off:2 * (off + K * Pg)], K, Pg), _nv_values_bf16(packed, sc),
                               f"col bf16 panels of group {gi}")
            off += K * Pg
    else:
        assert_bytes_equal(u8(q.bufs["row_data"])[:M * K // 2], ref["row_data"], "row data")
        assert_bytes_equal(u8(q.bufs["row_scale"])[:M * K // 16], ref["row_scale"], "row scales")
        assert_bytes_equal(_unpanel16(u8(q.bufs[key]), M, K),
                           _nv_values_bf16(ref["row_data"].reshape(M, K // 2), ref["row_scale"]), "row bf16 panels")


def test_nvfp4_every_bf16_pattern_weight_casts():
    """Weight casts have no Hadamard transform and one amax per expert (that of its data).  Every
    finite bf16 pattern is cast by expert 0 (amax = the largest bf16), and the patterns of at most
    1, at most 2^-60 and at most 2^60 in magnitude by experts 1-3, row-wise (blocks along K) and
    column-wise (blocks along N)."""
    v = all_bf16_finite()
    mag = F.bf16_bits_to_f64(v & 0x7FFF)
    N, K = 512, 128
    mats = []
    for sel in (np.ones(v.size, bool), mag <= 1.0, mag <= 2.0 ** -60, mag <= 2.0 ** 60):
        s = np.random.default_rng(int(sel.sum())).permutation(v[sel])
        s = np.resize(s, N * K)                      # repeats fill the matrix
        mats.append(s.reshape(N, K))
    w = np.stack(mats)
    E = w.shape[0]
    rec = g.recipe("nvfp4")
    print(f"nvfp4 weight-cast sweep: {E} experts of [{N}, {K}]", flush=True)
    q = g.weight_quantize(dev_bf16(w.reshape(E * N, K)).view(E, N, K), rec)
    torch.cuda.synchronize()
    ref, _ = O.quantize_weight(w, O.Recipe("nvfp4"))
    assert_bytes_equal(f32bits(q.bufs["amax_pre"]), ref["amax"].view(np.uint32), "weight amax")
    assert_bytes_equal(u8(q.bufs["row_data"]), np.stack([r[0] for r in ref["row"]]), "row data")
    assert_bytes_equal(u8(q.bufs["row_scale"]), np.stack([r[1] for r in ref["row"]]), "row scales")
    assert_bytes_equal(u8(q.bufs["col_data"]), np.stack([r[0] for r in ref["colT"]]), "col data")
    assert_bytes_equal(u8(q.bufs["col_scale"]), np.stack([r[1] for r in ref["colT"]]), "col scales")


# ----------------------------------------------------------------------------- NVFP4 GEMM on exact operands
def _nv_operand(rng, rows, cols, scale_codes):
    """Random E2M1 nibbles [rows, cols] and E4M3 block scales [rows, cols / 16] drawn from
    scale_codes (so that every quantized value dec(c) dec(q) has at most 3 significant bits)."""
    nib = rng.integers(0, 16, size=(rows, cols)).astype(np.uint8)
    sc = rng.choice(np.array(scale_codes, np.uint8), size=(rows, cols // 16))
    return nib, sc


def _dequant(nib, sc, amax):
    return Q.nvfp4_dequant_rows(nib, sc, amax)


# Scale codes 0.5, 1 and 2 (E4M3 0x30, 0x38, 0x40); group amaxes 2688 / 2^j so that every global
# scale S = fp32(2688 / amax) is exactly 2^j: then each quantized value is a multiple of 2^-2 / S,
# each product of two a multiple of 2^-4 / (S_a S_b), every fp32 partial sum over K <= 512
# contraction elements stays below 2^21 of those units (exact), and the epilogue's
# fl(1 / S_a) fl(1 / S_b) is exact.  (For general scales that product of two rounded
# reciprocals adds at most about 1.5 fp32 ulps of relative error before the output rounding.)
EXACT_SCALES = [0x30, 0x38, 0x40]
EXACT_AMAX = [2688.0 / 2.0 ** j for j in (8, 4, 10, 6, 9)]


def test_gemm_nvfp4_fprop_exact_inputs_bitwise():
    rng = np.random.default_rng(3)
    splits, N, K = [96, 0, 300, 17], 256, 512
    M, E = sum(splits), len(splits)
    an, asc = _nv_operand(rng, M, K, EXACT_SCALES)
    a_amax = np.array(EXACT_AMAX[:E], np.float32)
    wn = [_nv_operand(rng, N, K, EXACT_SCALES) for _ in range(E)]
    w_amax = np.array(EXACT_AMAX[1:E + 1], np.float32)
    rec = g.recipe("nvfp4", 0)
    A = g.QTensor(g.NVFP4_RHT, {"row_data": torch.from_numpy(F.pack_fp4(an)).cuda(),
                                "row_scale": torch.from_numpy(asc).cuda(), "amax_pre": dev_f32(a_amax)})
    B = g.QTensor(g.NVFP4_RHT, {"row_data": torch.from_numpy(np.stack([F.pack_fp4(n) for n, _ in wn])).cuda(),
                                "row_scale": torch.from_numpy(np.stack([s for _, s in wn])).cuda(),
                                "amax_pre": dev_f32(w_amax)})
    sd = dev_splits(splits)
    c = g.grouped_gemm(g.GEMM_FPROP, rec, A, B, sd, M, N, K)
    c32 = g.grouped_gemm(g.GEMM_FPROP, rec, A, B, sd, M, N, K, out_dtype=g.OUT_FP32)
    torch.cuda.synchronize()
    ref, off = [], 0
    for e, m in enumerate(splits):
        ad = _dequant(an[off:off + m], asc[off:off + m], a_amax[e])
        ref.append(ad @ _dequant(*wn[e], w_amax[e]).T)
        off += m
    ref = np.concatenate(ref)
    assert np.array_equal(c32.cpu().numpy().astype(np.float64), ref), "fp32 output not exact"
    assert np.array_equal(bits16(c).reshape(M, N), F.f64_to_bf16_bits(ref))


def _panel(a):
    """[R, K] bytes (K a multiple of 64) -> the 64-byte K-panel layout of the GEMM operands."""
    R, K = a.shape
    return np.ascontiguousarray(a.reshape(R, K // 64, 64).transpose(1, 0, 2)).reshape(-1)


def _scale_words(codes):
    """E8M0 codes [R, K / 32] -> MFMA scale words [K / 128, R] (byte j: 32-block 4 w + j)."""
    R, nb = codes.shape
    c = codes.astype(np.uint32).reshape(R, nb // 4, 4)
    return np.ascontiguousarray((c[..., 0] | (c[..., 1] << 8) | (c[..., 2] << 16) | (c[..., 3] << 24)).T)


def test_gemm_mxfp8_every_code_exactly():
    """Every finite E4M3 code (each row of A cycles through all 254) under E8M0 block scales
    2^-24 .. 2^23 through the scaled MFMA, read back exactly: B is the identity (E4M3 1.0 under
    scale 2^0), so the fp32 output is dec(E4M3) 2^(X - 127) of each element of A (zeros compared
    by value) and the bf16 output its rounding."""
    M, N, K = 96, 256, 256
    finite = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    idx = (np.arange(K)[None, :] + 7 * np.arange(M)[:, None]) % finite.size
    a = finite[idx]
    a_codes = (103 + (np.arange(M)[:, None] + 5 * np.arange(K // 32)[None, :]) % 48).astype(np.uint8)
    b = np.zeros((N, K), np.uint8)
    b[np.arange(N), np.arange(N)] = 0x38                       # E4M3 1.0
    b_codes = np.full((N, K // 32), 127, np.uint8)             # 2^0
    rec = g.recipe("mxfp8")
    A = g.QTensor(g.MXFP8, {"row_data": torch.from_numpy(_panel(a)).cuda(),
                            "row_scale_mfma": torch.from_numpy(_scale_words(a_codes).view(np.int32)).cuda()})
    B = g.QTensor(g.MXFP8, {"row_data": torch.from_numpy(_panel(b)).cuda(),
                            "row_scale_mfma": torch.from_numpy(_scale_words(b_codes).view(np.int32)).cuda()})
    sd = dev_splits([M])
    c32 = g.grouped_gemm(g.GEMM_FPROP, rec, A, B, sd, M, N, K, out_dtype=g.OUT_FP32)
    c16 = g.grouped_gemm(g.GEMM_FPROP, rec, A, B, sd, M, N, K)
    torch.cuda.synchronize()
    want = F.e4m3_decode(a) * np.exp2(np.repeat(a_codes.astype(np.float64) - 127.0, 32, axis=1))
    assert np.array_equal(c32.cpu().numpy().astype(np.float64), want)
    assert np.array_equal(bits16(c16).reshape(M, N) & 0x7FFF, F.f64_to_bf16_bits(want) & 0x7FFF)
    assert np.array_equal(np.sign(c16.float().cpu().numpy()), np.sign(want))


def test_gemm_nvfp4_expands_every_code_exactly():
    """Every E2M1 code under every finite E4M3 block scale (codes 0..126, one per row of A) through
    the GEMM's expansion of packed operands, read back exactly: B is the identity (E2M1 1.0 under
    scale 1.0) and both group amaxes are 2688 (global scales 1), so the fp32 output is
    dec(E2M1) dec(E4M3) of each element of A (zeros compared by value)."""
    codes = np.arange(127, dtype=np.uint8)
    M, N, K = codes.size, 256, 256
    nib = (np.arange(M * K, dtype=np.int64).reshape(M, K) + np.arange(M)[:, None]) % 16
    nib = nib.astype(np.uint8)
    asc = np.repeat(codes[:, None], K // 16, axis=1)
    bn = np.zeros((N, K), np.uint8)
    bn[np.arange(N), np.arange(N)] = 2                       # E2M1 code 2 = 1.0
    bsc = np.full((N, K // 16), 0x38, np.uint8)              # E4M3 1.0
    amax = np.array([2688.0], np.float32)
    rec = g.recipe("nvfp4", 0)
    A = g.QTensor(g.NVFP4_RHT, {"row_data": torch.from_numpy(F.pack_fp4(nib)).cuda(),
                                "row_scale": torch.from_numpy(asc).cuda(), "amax_pre": dev_f32(amax)})
    B = g.QTensor(g.NVFP4_RHT, {"row_data": torch.from_numpy(F.pack_fp4(bn)[None]).cuda(),
                                "row_scale": torch.from_numpy(bsc[None]).cuda(), "amax_pre": dev_f32(amax)})
    c32 = g.grouped_gemm(g.GEMM_FPROP, rec, A, B, dev_splits([M]), M, N, K, out_dtype=g.OUT_FP32)
    torch.cuda.synchronize()
    want = F.e2m1_decode(nib) * F.e4m3_decode(asc).repeat(16, axis=1)
    assert np.array_equal(c32.cpu().numpy().astype(np.float64), want)


def test_gemm_nvfp4_wgrad_exact_inputs_bitwise():
    rng = np.random.default_rng(4)
    splits, Na, Nb = [40, 0, 300, 128], 256, 128
    E = len(splits)
    P = [-(-m // 128) * 128 for m in splits]
    ops = {}
    for name, rows in (("a", Na), ("b", Nb)):
        nib, sc, amax = [], [], np.array(EXACT_AMAX[:E] if name == "a" else EXACT_AMAX[-E:], np.float32)
        for m, p in zip(splits, P):
            n, s = _nv_operand(rng, rows, p, EXACT_SCALES)
            n[:, m:] = 0                              # padded tokens hold zeros
            nib.append(n)
            sc.append(s)
        ops[name] = (nib, sc, amax)
    rec = g.recipe("nvfp4", 0)

    def qt(name):
        nib, sc, amax = ops[name]
        return g.QTensor(g.NVFP4_RHT, {
            "col_data": torch.from_numpy(np.concatenate([F.pack_fp4(n).reshape(-1) for n in nib])).cuda(),
            "col_scale": torch.from_numpy(np.concatenate([s.reshape(-1) for s in sc])).cuda(),
            "amax_post": dev_f32(amax)})

    sd = dev_splits(splits)
    M = sum(splits)
    c = g.grouped_gemm(g.GEMM_WGRAD, rec, qt("a"), qt("b"), sd, M, Na, Nb)
    c32 = g.grouped_gemm(g.GEMM_WGRAD, rec, qt("a"), qt("b"), sd, M, Na, Nb, out_dtype=g.OUT_FP32)
    torch.cuda.synchronize()
    ref = np.stack([_dequant(ops["a"][0][e], ops["a"][1][e], ops["a"][2][e]) @
                    _dequant(ops["b"][0][e], ops["b"][1][e], ops["b"][2][e]).T if splits[e] else np.zeros((Na, Nb))
                    for e in range(E)])
    assert np.array_equal(c32.cpu().numpy().astype(np.float64), ref), "fp32 output not exact"
    assert np.array_equal(bits16(c).reshape(E, Na, Nb), F.f64_to_bf16_bits(ref))


# ----------------------------------------------------------------------------- dgrad orientation
@pytest.mark.parametrize("kind", ["mxfp8", "nvfp4"])
@pytest.mark.parametrize("splits,N,K", [([0, 37, 300, 129], 256, 384), ([700, 1, 0], 384, 640)])
def test_gemm_dgrad_orientation(kind, splits, N, K):
    """C [M, K] = A [M, N] . W^T, the fc1 / fc2 dgrad: A row-wise with blocks along N, and the
    weight's dgrad operand (W_e^T [K, N] per expert, blocks along N) as B, passed as an FPROP
    operand and through the DGRAD layout."""
    M, E, mask = sum(splits), len(splits), 0x1D2B
    print(f"gemm dgrad {kind} splits={splits} N={N} K={K}", flush=True)
    a = random_bf16((M, N), seed=M + 3 * N)
    w = random_bf16((E, N, K), seed=N + K + 1, std=1 / np.sqrt(N))
    rec = g.recipe(kind, mask)
    sd = dev_splits(splits)
    aq = g.group_quantize(dev_bf16(a), sd, rec, True, False)
    wq = g.weight_quantize(dev_bf16(w.reshape(E * N, K)).view(E, N, K), rec)
    wd = g.QTensor(wq.kind, {"row_data": wq.bufs["col_data"], "row_scale": wq.bufs["col_scale"],
                             "row_scale_mfma": wq.bufs.get("col_scale_mfma"), "amax_pre": wq.bufs.get("amax_pre"),
                             "row_bf16": wq.bufs.get("col_bf16")})
    c = g.grouped_gemm(g.GEMM_FPROP, rec, aq, wd, sd, M, K, N)
    # the DGRAD layout takes the weight as quantized (its dgrad operand) and must give the same bits
    c2 = g.grouped_gemm(g.GEMM_DGRAD, rec, aq, wq, sd, M, K, N)
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.int16), c2.view(torch.int16)), "DGRAD layout differs from FPROP on W^T"
    orec = O.Recipe(kind, mask)
    _, ad = O.quantize_activation(a, splits, orec, row=True, col=False)
    _, wdq = O.quantize_weight(w, orec)
    ref, off = [], 0
    for e, m in enumerate(splits):
        ref.append(ad["row"][off:off + m] @ wdq["colT"][e].T)
        off += m
    ref = np.concatenate(ref)
    got = F.bf16_bits_to_f64(bits16(c)).reshape(M, K)
    assert O.rel_fro(got, F.round_bf16(ref)) <= 1e-3
