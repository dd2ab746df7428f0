"""Full-size parity on the three other workloads, run through the same calls as bench.py:

* nvfp4: 8 experts, hidden 5120, ffn 2048, 24576 rows split equally, NVFP4 + 16x16 RHT,
  prob-scaled SReLU, backward with activation recompute on and off;
* zipf:  64 experts, hidden 2048, ffn 1408, 49152 rows with Zipf(1.2) counts and 4 empty
  experts, MXFP8 SwiGLU;
* large: 128 experts, hidden 7168, ffn 2048, 65536 rows with Dirichlet(0.5) counts (empty
  experts and groups of fewer than 32 rows), stacked weights, MXFP8 SwiGLU.

The oracle cannot redo a whole step in seconds, so it checks what it can compute on its own:
- every group is independent, so one expert's slice of the full result equals the oracle's
  forward + backward of that expert alone (whole-group check of y, dx, dprob, dW1, dW2);
- MXFP8 rows and weight-gradient entries are row- / column-local (oracle.mlp.mxfp8_rows,
  mxfp8_wgrad_entries), which samples the largest experts;
- casts of x are compared bit for bit on sampled experts (NVFP4: with that group's pre- and
  post-RHT amax, themselves bit-exact);
- empty experts give exactly zero weight gradients, everything is finite, and recompute on/off
  are bitwise equal over the whole output (NVFP4).
"""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_mxfp8_amd as g
from gpu_util import assert_bytes_equal, bits16, dev_bf16, dev_f32, dev_splits, f32bits, u8, unpanel
from oracle import formats as F
from oracle import mlp as O
from oracle import quant as Q
from oracle import rht as R
from workloads import CONFIGS, expert_weights, iter_expert_weights, make_workload, random_bf16

pytestmark = pytest.mark.gpu
TOL = 2e-2              # end-to-end relative Frobenius error (fused output and gradients)
ROW_TOL = 1e-2          # sampled rows / entries of MXFP8 (fp32 vs fp64 accumulation only)
GEMM_TOL = 1e-3         # grouped GEMM on identical quantized operands vs the fp64 product rounded to bf16
LARGE_WGRAD_A_SEED = 777

_STATE = {}


def _pad(m):
    return -(-int(m) // 128) * 128


def _upload_weights(cfg):
    """Stacked bf16 weights on the device, drawn chunk by chunk of experts (the full host draw of the
    large workload would hold 11 GB of bf16 plus its fp32 draw)."""
    E, F1, H, ffn = cfg.experts, cfg.f1, cfg.hidden, cfg.ffn
    w1 = torch.empty((E, F1, H), dtype=torch.bfloat16, device="cuda")
    w2 = torch.empty((E, H, ffn), dtype=torch.bfloat16, device="cuda")
    for idx, a, b in iter_expert_weights(cfg, 0):
        n = len(idx)
        w1[idx[0]:idx[-1] + 1].copy_(dev_bf16(a.reshape(n * F1, H)).view(n, F1, H))
        w2[idx[0]:idx[-1] + 1].copy_(dev_bf16(b.reshape(n * H, ffn)).view(n, H, ffn))
        print(f"{cfg.name}: weights of experts {idx[0]}..{idx[-1]} on the device", flush=True)
    return w1, w2


def _host(t):
    return bits16(t) if t.dtype == torch.bfloat16 else t.detach().cpu().numpy()


def state(name):
    """Run the config's fused forward + backward once per module (one config held at a time)."""
    if _STATE.get("name") == name:
        return _STATE
    _STATE.clear()
    torch.cuda.empty_cache()
    cfg = CONFIGS[name]
    wl = make_workload(cfg, with_weights=False)
    E, H, ffn, F1 = cfg.experts, cfg.hidden, cfg.ffn, cfg.f1
    M = int(wl.m_splits.sum())
    print(f"{name}: splits={wl.m_splits.tolist()}", flush=True)
    rec = g.recipe(cfg.recipe, wl.sign_mask)
    x, dy = dev_bf16(wl.x), dev_bf16(wl.dy)
    splits, probs = dev_splits(wl.m_splits), dev_f32(wl.probs)
    w1, w2 = _upload_weights(cfg)
    w1q, w2q = g.weight_quantize(w1, rec), g.weight_quantize(w2, rec)
    del w1, w2
    runs = {}
    for recompute in ([False, True] if cfg.recipe == "nvfp4" else [False]):
        # NVFP4: the recompute run takes the fc2-input amax in the fc1 epilogue (fc2_amax_in_fc1), the
        # other in a pass over h; the two runs are compared bitwise below
        fused = cfg.recipe == "nvfp4" and recompute
        y, ctx = g.grouped_mlp_forward(x, splits, w1q, w2q, probs, cfg.activation, rec, recompute=recompute,
                                       fc2_amax_in_fc1=fused)
        fwd_counts = g.last_launch_counts()
        fused_amax_ok = None
        if fused:
            # the fc2 input's amax from the fc1 GEMM's epilogue vs the standalone pass on the same a
            h, pre, post = g.forward_saved(ctx)
            r_ = torch.relu(h.float())
            a_ = (r_ * r_ * probs[:, None]).to(torch.bfloat16)
            del r_
            rpre, rpost = g.group_hadamard_amax(a_, splits, wl.sign_mask)
            fused_amax_ok = (torch.equal(pre.view(torch.int32), rpre.view(torch.int32)) and
                             torch.equal(post.view(torch.int32), rpost.view(torch.int32)))
            del a_
        out = g.grouped_mlp_backward(dy, splits, w1q, w2q, probs, ctx)
        bwd_counts = g.last_launch_counts()
        torch.cuda.synchronize()
        finite = all(bool(torch.isfinite(t.float()).all()) for t in (y, out["dx"], out["dprobs"], out["dw1"],
                                                                      out["dw2"]))
        empty = [e for e in range(E) if wl.m_splits[e] == 0]
        empty_zero = all(not bool(out["dw1"][e].any()) and not bool(out["dw2"][e].any()) for e in empty)
        host = {"y": _host(y).reshape(M, H), "dx": _host(out["dx"]).reshape(M, H), "dprobs": _host(out["dprobs"]),
                "finite": finite, "empty": empty, "empty_zero": empty_zero,
                "fwd_counts": fwd_counts, "bwd_counts": bwd_counts, "dev": {k: out[k] for k in ("dw1", "dw2")},
                "fused_amax_ok": fused_amax_ok}
        host["dev"]["y"], host["dev"]["dx"], host["dev"]["dprobs"] = y, out["dx"], out["dprobs"]
        runs[recompute] = host
        del ctx
        print(f"{name}: forward + backward done (recompute={recompute})", flush=True)
    xq = g.group_quantize(x, splits, rec, True, True)
    wgrad = {}
    if name == "large":
        # whole-output check of an fc1-wgrad-shaped GEMM (A [M, F1] with x, contraction over each
        # expert's tokens) on the three largest experts, in the launch shape of the step
        order = sorted(range(E), key=lambda e: (-int(wl.m_splits[e]), e))[:3]
        a_bits = random_bf16((M, F1), seed=LARGE_WGRAD_A_SEED)
        aq = g.group_quantize(dev_bf16(a_bits), splits, rec, False, True)
        c = g.grouped_gemm(g.GEMM_WGRAD, rec, aq, xq, splits, M, F1, H)
        torch.cuda.synchronize()
        wgrad = {"experts": order, "a_bits": a_bits, "c": {e: bits16(c[e]) for e in order}}
        del aq, c
        print(f"{name}: fc1-shaped WGRAD done; checking experts {order}", flush=True)
    torch.cuda.synchronize()
    _STATE.update(wgrad=wgrad, name=name, wl=wl, cfg=cfg, E=E, H=H, ffn=ffn, F1=F1, M=M, runs=runs, rec=rec,
                  off=np.concatenate([[0], np.cumsum(wl.m_splits)]).astype(np.int64),
                  xq={k: u8(v) if k not in ("amax_pre", "amax_post") else f32bits(v) for k, v in xq.bufs.items()
                      if k in ("row_data", "row_scale", "col_data", "col_scale", "amax_pre", "amax_post")},
                  wq={})
    del xq, w1q, w2q
    return _STATE


def _weights_q(s, e):
    """Oracle-quantized weights of expert e: ((wq1, wq2) as O.forward takes them, bf16 bits)."""
    if e not in s["wq"]:
        a, b = expert_weights(s["cfg"], 0, [e])
        orec = O.Recipe(s["cfg"].recipe, s["wl"].sign_mask)
        s["wq"][e] = (O.quantize_weight(a, orec), O.quantize_weight(b, orec), a, b)
    return s["wq"][e]


def _expert_full(s, e, recompute=False):
    """One expert's rows of the fused output and its weight gradients vs the oracle's forward + backward
    of that expert alone."""
    wl, cfg = s["wl"], s["cfg"]
    o, m = int(s["off"][e]), int(wl.m_splits[e])
    wq1, wq2, a, b = _weights_q(s, e)
    print(f"{cfg.name}: expert {e} ({m} rows), oracle forward + backward", flush=True)
    orec = O.Recipe(cfg.recipe, wl.sign_mask)
    fwd = O.forward(wl.x[o:o + m], [m], a, b, wl.probs[o:o + m], cfg.activation, orec, wq1=wq1, wq2=wq2)
    bwd = O.backward(fwd, wl.dy[o:o + m])
    run = s["runs"][recompute]
    dw1 = bits16(run["dev"]["dw1"][e])
    dw2 = bits16(run["dev"]["dw2"][e])
    errs = {"y": O.rel_fro(F.bf16_bits_to_f64(run["y"][o:o + m]), F.round_bf16(fwd["y_f64"])),
            "dx": O.rel_fro(F.bf16_bits_to_f64(run["dx"][o:o + m]), F.round_bf16(bwd["dx_f64"])),
            "dprob": O.rel_fro(run["dprobs"][o:o + m].astype(np.float64), bwd["dprob"]),
            "dw1": O.rel_fro(F.bf16_bits_to_f64(dw1).reshape(-1), F.round_bf16(bwd["dw1_f64"][0]).reshape(-1)),
            "dw2": O.rel_fro(F.bf16_bits_to_f64(dw2).reshape(-1), F.round_bf16(bwd["dw2_f64"][0]).reshape(-1))}
    print(f"{cfg.name}: expert {e}:", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for k, v in errs.items():
        assert v <= TOL, (k, v)
    return fwd


def _sampled_rows(s, e):
    """MXFP8: y, dx, dprob at rows at both ends and in the middle of expert e's group, and sampled
    weight-gradient entries (each over all of the group's tokens)."""
    wl, cfg = s["wl"], s["cfg"]
    H, ffn, F1 = s["H"], s["ffn"], s["F1"]
    o, m = int(s["off"][e]), int(wl.m_splits[e])
    wq1, wq2, _, _ = _weights_q(s, e)
    d1 = {"row": wq1[1]["row"][0], "colT": wq1[1]["colT"][0]}
    d2 = {"row": wq2[1]["row"][0], "colT": wq2[1]["colT"][0]}
    rows = np.unique(np.array([o, o + 1, o + m // 2, o + m - 2, o + m - 1]))
    print(f"{cfg.name}: expert {e} ({m} rows): rows {rows.tolist()}", flush=True)
    run = s["runs"][False]
    ref = O.mxfp8_rows(wl.x[rows], wl.dy[rows], wl.probs[rows], d1, d2, cfg.activation)
    errs = {"y": O.rel_fro(F.bf16_bits_to_f64(run["y"][rows]), F.round_bf16(ref["y_f64"])),
            "dx": O.rel_fro(F.bf16_bits_to_f64(run["dx"][rows]), F.round_bf16(ref["dx_f64"])),
            "dprob": O.rel_fro(run["dprobs"][rows].astype(np.float64), ref["dprob"])}
    rng = np.random.default_rng(e)
    dw1_idx = [(0, 0), (ffn - 1, H - 1), (ffn, 17), (F1 - 1, H // 2)] + \
        [(int(rng.integers(F1)), int(rng.integers(H))) for _ in range(2)]
    dw2_idx = [(0, 0), (H - 1, ffn - 1), (H // 3, ffn // 2)] + \
        [(int(rng.integers(H)), int(rng.integers(ffn))) for _ in range(2)]
    ref1, ref2 = O.mxfp8_wgrad_entries(wl.x[o:o + m], wl.dy[o:o + m], wl.probs[o:o + m], d1, d2,
                                       cfg.activation, dw1_idx, dw2_idx)
    dw1 = run["dev"]["dw1"][e]
    dw2 = run["dev"]["dw2"][e]
    got1 = F.bf16_bits_to_f64(bits16(dw1[[f for f, _ in dw1_idx], [k for _, k in dw1_idx]]))
    got2 = F.bf16_bits_to_f64(bits16(dw2[[n for n, _ in dw2_idx], [f for _, f in dw2_idx]]))
    errs["dw1"] = O.rel_fro(got1, F.round_bf16(ref1))
    errs["dw2"] = O.rel_fro(got2, F.round_bf16(ref2))
    print(f"{cfg.name}: expert {e}:", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for k, v in errs.items():
        assert v <= ROW_TOL, (k, v)


def _mx_x_casts(s, e):
    """MXFP8 row-wise x at sampled rows and column-wise x at sampled features of expert e: bit-exact."""
    wl, H, M = s["wl"], s["H"], s["M"]
    o, m = int(s["off"][e]), int(wl.m_splits[e])
    rows = np.unique(np.array([o, o + m // 2, o + m - 1]))
    xr = unpanel(s["xq"]["row_data"], M, H)[rows]
    qx, _ = Q.mxfp8_quantize_rows(F.bf16_bits_to_f64(wl.x[rows]))
    assert_bytes_equal(xr, qx, "x row-wise data")
    P = [_pad(v) for v in wl.m_splits]
    base = H * sum(P[:e])
    col = unpanel(s["xq"]["col_data"][base:base + H * P[e]], H, P[e])
    feats = [0, 1, H // 3, H - 1]
    t = np.zeros((len(feats), P[e]))
    t[:, :m] = F.bf16_bits_to_f64(wl.x[o:o + m][:, feats]).T
    qc, _ = Q.mxfp8_quantize_rows(t)
    assert_bytes_equal(col[feats], qc, "x column-wise data")


def _by_size(wl):
    nz = [e for e in range(len(wl.m_splits)) if wl.m_splits[e] > 0]
    order = sorted(nz, key=lambda e: (int(wl.m_splits[e]), e))
    return order[0], order[-1]


def _median_expert(wl):
    nz = [e for e in range(len(wl.m_splits)) if wl.m_splits[e] > 0]
    order = sorted(nz, key=lambda e: (int(wl.m_splits[e]), e))
    return order[len(order) // 2]


# ----------------------------------------------------------------------------- NVFP4 + RHT, SReLU
def test_nvfp4_recompute_on_off_bitwise():
    s = state("nvfp4")
    a, b = s["runs"][False], s["runs"][True]
    assert a["finite"] and b["finite"]
    for k in ("y", "dx", "dprobs", "dw1", "dw2"):
        ta, tb = a["dev"][k], b["dev"][k]
        view = torch.int16 if ta.dtype == torch.bfloat16 else torch.int32
        assert torch.equal(ta.view(view), tb.view(view)), k
    # recompute casts the rebuilt fc2 input with the forward's amax: no extra Hadamard-amax pass
    assert a["bwd_counts"]["hadamard_amax"] == b["bwd_counts"]["hadamard_amax"] == 2
    # the recompute run took the fc2-input amax in the fc1 GEMM's epilogue: bit for bit the
    # standalone pass's, and only x got an amax pass of its own
    assert b["fused_amax_ok"]
    assert a["fwd_counts"]["hadamard_amax"] == 2 and b["fwd_counts"]["hadamard_amax"] == 1
    assert b["bwd_counts"]["nvfp4_quantize"] == a["bwd_counts"]["nvfp4_quantize"] + 1


@pytest.mark.parametrize("e", [0, 5])
def test_nvfp4_x_amax_and_casts(e):
    s = state("nvfp4")
    wl, H = s["wl"], s["H"]
    o, m = int(s["off"][e]), int(wl.m_splits[e])
    xg = wl.x[o:o + m]
    pre, post = R.group_hadamard_amax(xg, [m], wl.sign_mask)
    assert_bytes_equal(s["xq"]["amax_pre"][e:e + 1], pre.view(np.uint32), "pre-RHT amax")
    assert_bytes_equal(s["xq"]["amax_post"][e:e + 1], post.view(np.uint32), "post-RHT amax")
    ref = Q.nvfp4_group_quantize_with_amax(xg, [m], pre, post, wl.sign_mask)
    assert_bytes_equal(s["xq"]["row_data"][o * H // 2:(o + m) * H // 2], ref["row_data"], "row data")
    assert_bytes_equal(s["xq"]["row_scale"][o * H // 16:(o + m) * H // 16], ref["row_scale"], "row scales")
    P = [_pad(v) for v in wl.m_splits]
    c0 = H * sum(P[:e])
    assert_bytes_equal(s["xq"]["col_data"][c0 // 2:(c0 + H * P[e]) // 2], ref["col_data"], "col data")
    assert_bytes_equal(s["xq"]["col_scale"][c0 // 16:(c0 + H * P[e]) // 16], ref["col_scale"], "col scales")


def test_nvfp4_expert_matches_oracle():
    s = state("nvfp4")
    _expert_full(s, 7, recompute=True)


# ----------------------------------------------------------------------------- 64 experts, Zipf counts
def test_zipf_empty_experts_and_finite():
    s = state("zipf")
    r = s["runs"][False]
    assert len(r["empty"]) == 4, r["empty"]
    assert r["finite"] and r["empty_zero"]


def test_zipf_smallest_expert_matches_oracle():
    s = state("zipf")
    small, _ = _by_size(s["wl"])
    _mx_x_casts(s, small)
    _expert_full(s, small)


def test_zipf_largest_expert_sampled():
    s = state("zipf")
    _, big = _by_size(s["wl"])
    _mx_x_casts(s, big)
    _sampled_rows(s, big)


# ----------------------------------------------------------------------------- 128 experts, Dirichlet counts
def test_large_empty_experts_and_finite():
    s = state("large")
    r = s["runs"][False]
    assert r["finite"] and r["empty_zero"], r["empty"]


def test_large_smallest_expert_matches_oracle():
    s = state("large")
    small, _ = _by_size(s["wl"])
    _mx_x_casts(s, small)
    _expert_full(s, small)


def test_large_largest_expert_sampled():
    s = state("large")
    _, big = _by_size(s["wl"])
    _mx_x_casts(s, big)
    _sampled_rows(s, big)


def test_large_median_expert_matches_oracle():
    """The median-size non-empty expert, whole: y, dx, dprob and both weight gradients."""
    s = state("large")
    e = _median_expert(s["wl"])
    _mx_x_casts(s, e)
    _expert_full(s, e)


@pytest.mark.parametrize("rank", [0, 1, 2])
def test_large_fc1_wgrad_largest_experts_whole(rank):
    """Every element of the rank-th largest expert's [F1, H] = [4096, 7168] slice of an
    fc1-wgrad-shaped grouped GEMM against the oracle's fp64 product of the column-wise operands."""
    s = state("large")
    wl, w = s["wl"], s["wgrad"]
    e = w["experts"][rank]
    o, m = int(s["off"][e]), int(wl.m_splits[e])
    print(f"large: WGRAD of expert {e} over {m} tokens", flush=True)
    rec = O.Recipe("mxfp8")
    _, ad = O.quantize_activation(w["a_bits"][o:o + m], [m], rec, row=False, col=True)
    _, xd = O.quantize_activation(wl.x[o:o + m], [m], rec, row=False, col=True)
    ref = ad["col"][0] @ xd["col"][0].T
    err = O.rel_fro(F.bf16_bits_to_f64(w["c"][e]).reshape(ref.shape), F.round_bf16(ref))
    print(f"large: expert {e} WGRAD relative Frobenius error {err:.2e}", flush=True)
    assert err <= GEMM_TOL
