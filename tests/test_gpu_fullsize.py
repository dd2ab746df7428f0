"""Full-size MXFP8 parity on the bench workload (8 experts, hidden 4096, ffn 1536, 32768 rows,
SwiGLU, recompute off), run through the same calls and launch configuration as bench.py.

The oracle cannot redo the whole step in seconds, so it evaluates samples that it can compute
on their own (oracle.mlp.mxfp8_rows, mxfp8_wgrad_entries): the first and the last expert's
quantized weights (bit-exact), the row- and column-wise casts of x at sampled rows and
features (bit-exact), y, dx and dprob at rows at both ends and in the middle of those experts'
groups, and sampled entries of both weight gradients (each needs two feature columns over
all of the group's tokens)."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_mxfp8_amd as g
from gpu_util import assert_bytes_equal, bits16, dev_bf16, dev_f32, dev_splits, u8, unpanel
from oracle import formats as F
from oracle import mlp as O
from oracle import quant as Q
from workloads import CONFIGS, make_workload, random_bf16

pytestmark = pytest.mark.gpu
TOL = 1e-2          # relative Frobenius error over the sampled values (fp32 vs fp64 accumulation)
GEMM_TOL = 1e-3     # grouped GEMM on identical quantized operands vs the fp64 product rounded to bf16
WGRAD_A_SEED = 4242


@pytest.fixture(scope="module")
def run():
    wl = make_workload(CONFIGS["mid"])
    cfg = wl.config
    E, H, ffn, F1 = cfg.experts, cfg.hidden, cfg.ffn, cfg.f1
    M = int(wl.m_splits.sum())
    print(f"full-size mid workload: splits={wl.m_splits.tolist()}", flush=True)
    rec = g.recipe("mxfp8")
    x, dy = dev_bf16(wl.x), dev_bf16(wl.dy)
    w1 = dev_bf16(wl.w1.reshape(E * F1, H)).view(E, F1, H)
    w2 = dev_bf16(wl.w2.reshape(E * H, ffn)).view(E, H, ffn)
    splits, probs = dev_splits(wl.m_splits), dev_f32(wl.probs)
    w1q, w2q = g.weight_quantize(w1, rec), g.weight_quantize(w2, rec)
    y, ctx = g.grouped_mlp_forward(x, splits, w1q, w2q, probs, cfg.activation, rec, recompute=False)
    out = g.grouped_mlp_backward(dy, splits, w1q, w2q, probs, ctx)
    xq = g.group_quantize(x, splits, rec, True, True)
    # whole-output GEMM checks in the launch shapes of the step: fc1 FPROP (x . W1^T, 7 rounds of
    # 256 workgroups) and a WGRAD of the fc1-wgrad shape (A [M, F1] with x, contraction over tokens)
    c_fprop = g.grouped_gemm(g.GEMM_FPROP, rec, xq, w1q, splits, M, F1, H)
    a_bits = random_bf16((M, F1), seed=WGRAD_A_SEED)
    aq = g.group_quantize(dev_bf16(a_bits), splits, rec, False, True)
    c_wgrad = g.grouped_gemm(g.GEMM_WGRAD, rec, aq, xq, splits, M, F1, H)
    torch.cuda.synchronize()
    print("full-size mid workload: fused step and the two GEMMs done", flush=True)
    r = {"wl": wl, "E": E, "H": H, "ffn": ffn, "F1": F1, "M": M, "a_bits": a_bits, "wq": {},
         "c_fprop": bits16(c_fprop).reshape(M, F1), "c_wgrad": bits16(c_wgrad).reshape(E, F1, H),
         "off": np.concatenate([[0], np.cumsum(wl.m_splits)]).astype(np.int64),
         "w1_row": u8(w1q.bufs["row_data"]), "w2_row": u8(w2q.bufs["row_data"]),
         "w1_col": u8(w1q.bufs["col_data"]), "xq_row": u8(xq.bufs["row_data"]), "xq_col": u8(xq.bufs["col_data"]),
         "y": bits16(y).reshape(M, H), "dx": bits16(out["dx"]).reshape(M, H),
         "dprobs": out["dprobs"].cpu().numpy(), "dw1": bits16(out["dw1"]).reshape(E, F1, H),
         "dw2": bits16(out["dw2"]).reshape(E, H, ffn)}
    return r


def _expert(r, e):
    """Oracle-quantized weights of expert e (codes and dequantized values), computed once."""
    if e not in r["wq"]:
        wl = r["wl"]
        rec = O.Recipe("mxfp8")
        q1, d1 = O.quantize_weight(wl.w1[e:e + 1], rec)
        q2, d2 = O.quantize_weight(wl.w2[e:e + 1], rec)
        r["wq"][e] = (q1, q2, {"row": d1["row"][0], "colT": d1["colT"][0]},
                      {"row": d2["row"][0], "colT": d2["colT"][0]})
    return r["wq"][e]


def _rows(r, e):
    o, m = int(r["off"][e]), int(r["wl"].m_splits[e])
    return np.unique(np.array([o, o + 1, o + m // 2, o + m - 2, o + m - 1]))


@pytest.mark.parametrize("e", [0, 7])
def test_fullsize_weights_and_x_casts(run, e):
    r = run
    E, H, ffn, F1, M = r["E"], r["H"], r["ffn"], r["F1"], r["M"]
    q1, q2, _, _ = _expert(r, e)
    print(f"expert {e}: weight casts", flush=True)
    assert_bytes_equal(unpanel(r["w1_row"][e * F1 * H:(e + 1) * F1 * H], F1, H), q1["row"][0][0], "W1 fprop data")
    assert_bytes_equal(unpanel(r["w2_row"][e * H * ffn:(e + 1) * H * ffn], H, ffn), q2["row"][0][0], "W2 fprop data")
    assert_bytes_equal(unpanel(r["w1_col"][e * F1 * H:(e + 1) * F1 * H], H, F1), q1["colT"][0][0], "W1 dgrad data")
    # row-wise x at sampled rows, column-wise x at sampled features of the group
    rows = _rows(r, e)
    xr = unpanel(r["xq_row"], M, H)[rows]
    qx, _ = Q.mxfp8_quantize_rows(F.bf16_bits_to_f64(r["wl"].x[rows]))
    assert_bytes_equal(xr, qx, "x row-wise data")
    P = [-(-int(m) // 128) * 128 for m in r["wl"].m_splits]
    base = H * sum(P[:e])
    col = unpanel(r["xq_col"][base:base + H * P[e]], H, P[e])
    o, m = int(r["off"][e]), int(r["wl"].m_splits[e])
    feats = [0, 1, 777, H - 1]
    t = np.zeros((len(feats), P[e]))
    t[:, :m] = F.bf16_bits_to_f64(r["wl"].x[o:o + m][:, feats]).T
    qc, _ = Q.mxfp8_quantize_rows(t)
    assert_bytes_equal(col[feats], qc, "x column-wise data")


@pytest.mark.parametrize("e", [0, 7])
def test_fullsize_sampled_rows(run, e):
    r = run
    wl = r["wl"]
    _, _, d1, d2 = _expert(r, e)
    rows = _rows(r, e)
    print(f"expert {e}: rows {rows.tolist()}", flush=True)
    ref = O.mxfp8_rows(wl.x[rows], wl.dy[rows], wl.probs[rows], d1, d2, wl.config.activation)
    errs = {"y": O.rel_fro(F.bf16_bits_to_f64(r["y"][rows]), F.round_bf16(ref["y_f64"])),
            "dx": O.rel_fro(F.bf16_bits_to_f64(r["dx"][rows]), F.round_bf16(ref["dx_f64"])),
            "dprob": O.rel_fro(r["dprobs"][rows].astype(np.float64), ref["dprob"])}
    print(f"expert {e}:", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for k, v in errs.items():
        assert v <= TOL, (k, v)


@pytest.mark.parametrize("e", [0, 7])
def test_fullsize_sampled_weight_gradients(run, e):
    r = run
    wl = r["wl"]
    H, ffn, F1 = r["H"], r["ffn"], r["F1"]
    _, _, d1, d2 = _expert(r, e)
    o, m = int(r["off"][e]), int(wl.m_splits[e])
    dw1_idx = [(0, 0), (ffn - 1, H - 1), (ffn, 17), (F1 - 1, 1000), (100, 2048), (2000, 5)]
    dw2_idx = [(0, 0), (H - 1, ffn - 1), (123, 456), (4000, 1500), (2048, 64)]
    print(f"expert {e}: {len(dw1_idx)} dW1 and {len(dw2_idx)} dW2 entries over {m} tokens", flush=True)
    ref1, ref2 = O.mxfp8_wgrad_entries(wl.x[o:o + m], wl.dy[o:o + m], wl.probs[o:o + m], d1, d2,
                                       wl.config.activation, dw1_idx, dw2_idx)
    got1 = F.bf16_bits_to_f64(np.array([r["dw1"][e, f, k] for f, k in dw1_idx], np.uint16))
    got2 = F.bf16_bits_to_f64(np.array([r["dw2"][e, n, f] for n, f in dw2_idx], np.uint16))
    err1 = O.rel_fro(got1, F.round_bf16(ref1))
    err2 = O.rel_fro(got2, F.round_bf16(ref2))
    print(f"expert {e}: dW1 {err1:.2e} dW2 {err2:.2e}", flush=True)
    assert err1 <= TOL and err2 <= TOL, (err1, err2)
    # every entry: within a few bf16 steps of the oracle's value (relative to the entry scale)
    for got, ref in ((got1, ref1), (got2, ref2)):
        scale = np.sqrt(np.mean(ref * ref))
        assert np.all(np.abs(got - ref) <= 2.0 ** -6 * np.abs(ref) + 1e-2 * scale), (got, ref)


@pytest.mark.parametrize("e", range(8))
def test_fullsize_fc1_fprop_whole_output(run, e):
    """Every element of expert e's rows of h = Q(x) Q(W1)^T from gmlp_grouped_gemm (the fc1 launch of
    the step: 8 experts of ~4096 rows, 12 x 128 tile pairs per expert, 7 rounds of 256 workgroups)
    against the fp64 product of the oracle's dequantized operands, rounded to bf16."""
    r = run
    wl = r["wl"]
    o, m = int(r["off"][e]), int(wl.m_splits[e])
    _, _, d1, _ = _expert(r, e)
    print(f"expert {e}: fc1 FPROP, {m} rows", flush=True)
    xd = Q.mxfp8_dequant_rows(*Q.mxfp8_quantize_rows(F.bf16_bits_to_f64(wl.x[o:o + m])))
    ref = xd @ d1["row"].T
    err = O.rel_fro(F.bf16_bits_to_f64(r["c_fprop"][o:o + m]), F.round_bf16(ref))
    print(f"expert {e}: fc1 FPROP relative Frobenius error {err:.2e}", flush=True)
    assert err <= GEMM_TOL


@pytest.mark.parametrize("e", range(8))
def test_fullsize_fc1_wgrad_whole_output(run, e):
    """Every element of expert e's [F1, H] slice of Qc(A)^T Qc(x) (contraction over the expert's
    tokens, column-wise operands zero padded to 128 tokens) against the oracle's fp64 product."""
    r = run
    wl = r["wl"]
    o, m = int(r["off"][e]), int(wl.m_splits[e])
    print(f"expert {e}: fc1-shaped WGRAD over {m} tokens", flush=True)
    rec = O.Recipe("mxfp8")
    _, ad = O.quantize_activation(r["a_bits"][o:o + m], [m], rec, row=False, col=True)
    _, xd = O.quantize_activation(wl.x[o:o + m], [m], rec, row=False, col=True)
    ref = ad["col"][0] @ xd["col"][0].T
    err = O.rel_fro(F.bf16_bits_to_f64(r["c_wgrad"][e]), F.round_bf16(ref))
    print(f"expert {e}: WGRAD relative Frobenius error {err:.2e}", flush=True)
    assert err <= GEMM_TOL
