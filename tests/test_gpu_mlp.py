"""GPU parity of the fused grouped MLP forward + backward with the oracle (relative Frobenius
<= 2e-2), recompute on/off bitwise equality, determinism and the launch plan."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_mxfp8_amd as g
from gpu_util import bits16, dev_bf16, dev_f32, dev_splits
from oracle import formats as F
from oracle import mlp as O
from workloads import make_workload, small_case

pytestmark = pytest.mark.gpu
TOL = 2e-2


def _upload(wl):
    E, H, ffn = wl.config.experts, wl.config.hidden, wl.config.ffn
    F1 = wl.config.f1
    d = {"x": dev_bf16(wl.x), "splits": dev_splits(wl.m_splits), "probs": dev_f32(wl.probs),
         "w1": dev_bf16(wl.w1.reshape(E * F1, H)).view(E, F1, H),
         "w2": dev_bf16(wl.w2.reshape(E * H, ffn)).view(E, H, ffn)}
    if wl.dy is not None:
        d["dy"] = dev_bf16(wl.dy)
    return d


def _run(wl, d, kind, recompute, backward=True, wgrad_dtype=g.OUT_BF16, out=None):
    rec = g.recipe(kind, wl.sign_mask)
    w1q = g.weight_quantize(d["w1"], rec)
    w2q = g.weight_quantize(d["w2"], rec)
    y, ctx = g.grouped_mlp_forward(d["x"], d["splits"], w1q, w2q, d["probs"], wl.config.activation, rec,
                                   recompute=recompute)
    res = {"y": y, "fwd_counts": g.last_launch_counts()}
    if backward:
        res.update(g.grouped_mlp_backward(d["dy"], d["splits"], w1q, w2q, d["probs"], ctx,
                                          wgrad_dtype=wgrad_dtype, out=out))
        res["bwd_counts"] = g.last_launch_counts()
    torch.cuda.synchronize()
    return res


def _f64(t):
    return F.bf16_bits_to_f64(bits16(t)) if t.dtype == torch.bfloat16 else t.detach().cpu().double().numpy()


def _compare(out, wl, kind, backward=True):
    rec = O.Recipe(kind, wl.sign_mask)
    fwd = O.forward(wl.x, wl.m_splits, wl.w1, wl.w2, wl.probs, wl.config.activation, rec)
    errs = {"y": O.rel_fro(_f64(out["y"]).reshape(fwd["y_f64"].shape), F.round_bf16(fwd["y_f64"]))}
    if backward:
        bwd = O.backward(fwd, wl.dy)
        errs["dx"] = O.rel_fro(_f64(out["dx"]).reshape(bwd["dx_f64"].shape), F.round_bf16(bwd["dx_f64"]))
        errs["dprobs"] = O.rel_fro(out["dprobs"].cpu().double().numpy(), bwd["dprob"])
        errs["dw1"] = O.rel_fro(_f64(out["dw1"]).reshape(bwd["dw1_f64"].shape), F.round_bf16(bwd["dw1_f64"]))
        errs["dw2"] = O.rel_fro(_f64(out["dw2"]).reshape(bwd["dw2_f64"].shape), F.round_bf16(bwd["dw2_f64"]))
        for e, m in enumerate(wl.m_splits):
            if m == 0:
                assert not _f64(out["dw1"])[e].any() and not _f64(out["dw2"])[e].any()
    print(kind, wl.config.activation, {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for k, v in errs.items():
        assert v <= TOL, (k, v)
    return errs


# The tanh-clamped squared ReLU with clamp scale 2 (h has a standard deviation near 1 here, so the
# clamp bends a fair share of the values without flattening them) and QGeGLU.
TANH_SRELU = ("tanh_srelu", 2.0)
CASES = [("mxfp8", "swiglu"), ("nvfp4", "srelu"), ("mxfp8", "srelu"), ("nvfp4", "swiglu"),
         ("mxfp8", TANH_SRELU), ("nvfp4", TANH_SRELU), ("mxfp8", "qgeglu"), ("nvfp4", "qgeglu")]
CASE_IDS = [f"{k}-{a if isinstance(a, str) else a[0]}" for k, a in CASES]


@pytest.mark.parametrize("kind,act", CASES, ids=CASE_IDS)
def test_mlp_forward_backward_matches_oracle(kind, act):
    print(f"mlp {kind} {act}", flush=True)
    wl = small_case([0, 37, 300, 129, 5], 512, 384, activation=act, recipe=kind, seed=1, w_std=0.05)
    out = _run(wl, _upload(wl), kind, recompute=False)
    _compare(out, wl, kind)


@pytest.mark.parametrize("kind,act", CASES, ids=CASE_IDS)
def test_recompute_on_off_bitwise(kind, act):
    """Rebuilding the fc2 input in backward gives bitwise-equal output and gradients."""
    print(f"recompute {kind} {act}", flush=True)
    wl = small_case([64, 0, 200, 300], 256, 256, activation=act, recipe=kind, seed=2, w_std=0.05)
    d = _upload(wl)
    a = _run(wl, d, kind, recompute=False)
    b = _run(wl, d, kind, recompute=True)
    for k in ("y", "dx", "dprobs", "dw1", "dw2"):
        assert torch.equal(a[k].view(torch.int16) if a[k].dtype == torch.bfloat16 else a[k].view(torch.int32),
                           b[k].view(torch.int16) if b[k].dtype == torch.bfloat16 else b[k].view(torch.int32)), k
    if kind == "nvfp4":
        # the recompute backward casts the rebuilt input with the forward's amax: no third amax pass
        assert b["bwd_counts"]["hadamard_amax"] == 2 and a["bwd_counts"]["hadamard_amax"] == 2
        assert b["bwd_counts"]["nvfp4_quantize"] == 3 and a["bwd_counts"]["nvfp4_quantize"] == 2
        # forward: x's amax pass and the fc2 input's
        assert a["fwd_counts"]["hadamard_amax"] == b["fwd_counts"]["hadamard_amax"] == 2


def _fc2_input_amax_reference(ctx, probs, splits, sign_mask):
    """gmlp_group_hadamard_amax on the fc2 input a = bf16(relu(h)^2 p), formed by torch from the h
    the forward saved (fp32 products, round to nearest even, as the kernels form it)."""
    h, pre, post = g.forward_saved(ctx)
    r = torch.relu(h.float())
    a = (r * r * probs[:, None]).to(torch.bfloat16)
    rpre, rpost = g.group_hadamard_amax(a, splits, sign_mask)
    return pre, post, rpre, rpost


@pytest.mark.parametrize("recompute", [False, True])
@pytest.mark.parametrize("splits", [[0, 37, 300, 129, 5], [512, 256, 1]])
def test_nvfp4_fused_fc2_amax_matches_standalone_pass(splits, recompute):
    """NVFP4 with squared ReLU and fc2_amax_in_fc1: the fc1 GEMM's epilogue takes the fc2 input's
    per-group pre- and post-RHT amax ("Reduce NVFP4 quantization work ...", Changes: the
    Hadamard-fused fc1 kernel returns both); they equal, bit for bit, the standalone Hadamard-amax
    pass on the same fc2 input, the forward launches only x's amax pass, and y is bitwise the
    default forward's (which takes the amax in a pass over h).  (ffn 384: the second column tile
    of each row band is half empty.)"""
    print(f"fused fc2 amax splits={splits} recompute={recompute}", flush=True)
    wl = small_case(splits, 256, 384, activation="srelu", recipe="nvfp4", seed=9, w_std=0.05)
    d = _upload(wl)
    rec = g.recipe("nvfp4", wl.sign_mask)
    w1q, w2q = g.weight_quantize(d["w1"], rec), g.weight_quantize(d["w2"], rec)
    y0, ctx0 = g.grouped_mlp_forward(d["x"], d["splits"], w1q, w2q, d["probs"], "srelu", rec, recompute=recompute)
    counts0 = g.last_launch_counts()
    y, ctx = g.grouped_mlp_forward(d["x"], d["splits"], w1q, w2q, d["probs"], "srelu", rec, recompute=recompute,
                                   fc2_amax_in_fc1=True)
    counts = g.last_launch_counts()
    pre, post, rpre, rpost = _fc2_input_amax_reference(ctx, d["probs"], d["splits"], wl.sign_mask)
    _, pre0, post0 = g.forward_saved(ctx0)
    torch.cuda.synchronize()
    assert counts["hadamard_amax"] == 1 and counts0["hadamard_amax"] == 2, (counts, counts0)
    assert torch.equal(pre.view(torch.int32), rpre.view(torch.int32)), (pre, rpre)
    assert torch.equal(post.view(torch.int32), rpost.view(torch.int32)), (post, rpost)
    assert torch.equal(pre0.view(torch.int32), pre.view(torch.int32))
    assert torch.equal(post0.view(torch.int32), post.view(torch.int32))
    assert torch.equal(y0.view(torch.int16), y.view(torch.int16))
    assert float(post.max()) > 0 and all(float(pre[e]) == 0 for e in range(len(splits)) if splits[e] == 0)


@pytest.mark.parametrize("recompute", [False, True])
def test_nvfp4_fused_fc2_amax_tanh_srelu(recompute):
    """The tanh-clamped squared ReLU takes the same fused route ("Reduce NVFP4 quantization work ...",
    Changes: ScaledTanhSReLU through the Hadamard-fused fc1 kernel with tanh_clamp_scale): the fc1
    epilogue's pre- and post-RHT amax equal, bit for bit, those of the default forward's pass over h
    (the same activation function), with one amax launch fewer, and y and the gradients are bitwise
    the default forward's."""
    print(f"fused fc2 amax tanh_srelu recompute={recompute}", flush=True)
    wl = small_case([0, 37, 300, 129, 5], 256, 384, activation=TANH_SRELU, recipe="nvfp4", seed=9, w_std=0.05)
    d = _upload(wl)
    rec = g.recipe("nvfp4", wl.sign_mask)
    w1q, w2q = g.weight_quantize(d["w1"], rec), g.weight_quantize(d["w2"], rec)
    y0, ctx0 = g.grouped_mlp_forward(d["x"], d["splits"], w1q, w2q, d["probs"], TANH_SRELU, rec, recompute=recompute)
    counts0 = g.last_launch_counts()
    y, ctx = g.grouped_mlp_forward(d["x"], d["splits"], w1q, w2q, d["probs"], TANH_SRELU, rec, recompute=recompute,
                                   fc2_amax_in_fc1=True)
    counts = g.last_launch_counts()
    _, pre0, post0 = g.forward_saved(ctx0)
    _, pre, post = g.forward_saved(ctx)
    b0 = g.grouped_mlp_backward(d["dy"], d["splits"], w1q, w2q, d["probs"], ctx0)
    b1 = g.grouped_mlp_backward(d["dy"], d["splits"], w1q, w2q, d["probs"], ctx)
    torch.cuda.synchronize()
    assert counts["hadamard_amax"] == 1 and counts0["hadamard_amax"] == 2, (counts, counts0)
    assert torch.equal(pre0.view(torch.int32), pre.view(torch.int32)), (pre0, pre)
    assert torch.equal(post0.view(torch.int32), post.view(torch.int32)), (post0, post)
    assert torch.equal(y0.view(torch.int16), y.view(torch.int16))
    for k in ("dx", "dprobs", "dw1", "dw2"):
        view = torch.int16 if b0[k].dtype == torch.bfloat16 else torch.int32
        assert torch.equal(b0[k].view(view), b1[k].view(view)), k
    assert float(post.max()) > 0 and float(pre[0]) == 0


@pytest.mark.parametrize("act", ["srelu", TANH_SRELU, "swiglu", "qgeglu"],
                         ids=["srelu", "tanh_srelu", "swiglu", "qgeglu"])
def test_nvfp4_fc2_input_amax_matches_the_oracle_activation(act):
    """The NVFP4 forward keeps the fc2 input's per-group amax for the recompute cast.  Against the
    oracle's activation of the same saved h (fp64, then p, then bf16): the pre-RHT amax, which is
    one of the a values, within one bf16 ulp (the kernels evaluate the activation in fp32 with the
    hardware exp2, reciprocal and the library tanh), the post-RHT amax within 2^-5."""
    from oracle.rht import group_hadamard_amax
    print(f"fc2 input amax {act}", flush=True)
    wl = small_case([0, 37, 300, 129, 5], 256, 384, activation=act, recipe="nvfp4", seed=13, w_std=0.05)
    d = _upload(wl)
    rec = g.recipe("nvfp4", wl.sign_mask)
    w1q, w2q = g.weight_quantize(d["w1"], rec), g.weight_quantize(d["w2"], rec)
    _, ctx = g.grouped_mlp_forward(d["x"], d["splits"], w1q, w2q, d["probs"], act, rec, recompute=True)
    h, pre, post = g.forward_saved(ctx)
    torch.cuda.synchronize()
    hv = F.bf16_bits_to_f64(bits16(h))
    a = F.round_bf16(O.act_forward(hv, act) * wl.probs.astype(np.float64)[:, None])
    rpre, rpost = group_hadamard_amax(F.f64_to_bf16_bits(a), wl.m_splits, wl.sign_mask)
    pre, post = pre.cpu().numpy(), post.cpu().numpy()
    for e, m in enumerate(wl.m_splits):
        if m == 0:
            assert pre[e] == 0 and post[e] == 0 and rpre[e] == 0
            continue
        assert abs(pre[e] - rpre[e]) <= 2.0 ** -7 * rpre[e], (e, pre[e], rpre[e])
        assert abs(post[e] - rpost[e]) <= 2.0 ** -5 * rpost[e], (e, post[e], rpost[e])


def test_backward_rejects_a_ctx_written_with_other_settings():
    """The backward and the deferred wgrad call check their settings against those the forward
    (and the deferring backward) wrote their buffers with: a recompute flag, a weight-gradient flag
    or a workspace that does not match is an error, not a read of the buffer in another layout."""
    import dataclasses
    wl = small_case([64, 0, 100], 128, 128, activation="srelu", recipe="nvfp4", seed=9, w_std=0.05)
    d = _upload(wl)
    rec = g.recipe("nvfp4", wl.sign_mask)
    w1q, w2q = g.weight_quantize(d["w1"], rec), g.weight_quantize(d["w2"], rec)
    _, ctx = g.grouped_mlp_forward(d["x"], d["splits"], w1q, w2q, d["probs"], "srelu", rec, recompute=False)
    with pytest.raises(g.GmlpError, match="ctx: written by a forward with a different recompute"):
        g.grouped_mlp_backward(d["dy"], d["splits"], w1q, w2q, d["probs"], dataclasses.replace(ctx, recompute=True))
    _, ctx2 = g.grouped_mlp_forward(d["x"], d["splits"], w1q, w2q, d["probs"], "srelu", rec,
                                    weight_requires_grad=False)
    with pytest.raises(g.GmlpError, match="saved no weight-gradient operands"):
        g.grouped_mlp_backward(d["dy"], d["splits"], w1q, w2q, d["probs"],
                               dataclasses.replace(ctx2, weight_requires_grad=True))
    part = g.grouped_mlp_backward(d["dy"], d["splits"], w1q, w2q, d["probs"], ctx, defer_wgrad=True)
    # the deferred operands are in part's workspace; a backward that does not defer reuses it
    g.grouped_mlp_backward(d["dy"], d["splits"], w1q, w2q, d["probs"], ctx, ws=part["deferred"].ws)
    with pytest.raises(g.GmlpError, match="ws: last written by a call that left no deferred"):
        g.grouped_mlp_wgrad(part["deferred"])
    torch.cuda.synchronize()


def test_tanh_srelu_needs_a_positive_clamp_scale():
    wl = small_case([64, 64], 128, 128, activation="srelu", recipe="mxfp8", seed=9, w_std=0.05)
    d = _upload(wl)
    rec = g.recipe("mxfp8")
    w1q, w2q = g.weight_quantize(d["w1"], rec), g.weight_quantize(d["w2"], rec)
    for c in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(g.GmlpError, match="clamp scale"):
            g.grouped_mlp_forward(d["x"], d["splits"], w1q, w2q, d["probs"], ("tanh_srelu", c), rec)


def test_fc2_amax_in_fc1_needs_nvfp4_srelu():
    wl = small_case([64, 64], 128, 128, activation="swiglu", recipe="nvfp4", seed=9, w_std=0.05)
    d = _upload(wl)
    rec = g.recipe("nvfp4", 1)
    w1q, w2q = g.weight_quantize(d["w1"], rec), g.weight_quantize(d["w2"], rec)
    with pytest.raises(g.GmlpError, match="squared-ReLU"):
        g.grouped_mlp_forward(d["x"], d["splits"], w1q, w2q, d["probs"], "swiglu", rec, fc2_amax_in_fc1=True)


def test_deterministic_and_fp32_wgrad():
    wl = small_case([100, 1, 300], 256, 256, activation="swiglu", recipe="mxfp8", seed=3, w_std=0.05)
    d = _upload(wl)
    a = _run(wl, d, "mxfp8", recompute=False)
    b = _run(wl, d, "mxfp8", recompute=False)
    for k in ("y", "dx", "dprobs", "dw1", "dw2"):
        assert torch.equal(a[k], b[k]), k
    c = _run(wl, d, "mxfp8", recompute=False, wgrad_dtype=g.OUT_FP32)
    assert c["dw1"].dtype == torch.float32
    assert O.rel_fro(c["dw1"].double().cpu().numpy(), _f64(a["dw1"])) <= 1e-2


@pytest.mark.parametrize("kind,act", [("mxfp8", "swiglu"), ("nvfp4", "srelu")])
def test_backward_accumulates_weight_gradients_into_fp32_main_grad(kind, act):
    """wgrad_dtype OUT_FP32_ACCUMULATE adds the weight gradients to the fp32 main_grads passed in:
    bit for bit the fp32 sum of the stored values and the plain fp32 gradients (an empty expert's
    slices unchanged), dx and dprobs as without it, and within tolerance of the oracle's
    fp32(main_grad + dW)."""
    wl = small_case([100, 0, 300, 41], 256, 256, activation=act, recipe=kind, seed=9, w_std=0.05)
    d = _upload(wl)
    plain = _run(wl, d, kind, recompute=True, wgrad_dtype=g.OUT_FP32)
    rng = np.random.default_rng(10)
    m0 = {k: (rng.standard_normal(tuple(plain[k].shape)) * plain[k].std().item()).astype(np.float32)
          for k in ("dw1", "dw2")}
    main = {k: torch.from_numpy(v).to("cuda") for k, v in m0.items()}
    acc = _run(wl, d, kind, recompute=True, wgrad_dtype=g.OUT_FP32_ACCUMULATE, out=dict(main))
    rec = O.Recipe(kind, wl.sign_mask)
    bwd = O.backward(O.forward(wl.x, wl.m_splits, wl.w1, wl.w2, wl.probs, act, rec), wl.dy)
    for k in ("dw1", "dw2"):
        assert acc[k].data_ptr() == main[k].data_ptr(), "the main_grad is updated in place"
        got = acc[k].cpu().numpy()
        want = m0[k] + plain[k].cpu().numpy()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), k
        assert np.array_equal(got[1].view(np.uint32), m0[k][1].view(np.uint32)), "empty expert changed"
        err = O.rel_fro(got.astype(np.float64), O.accumulate_main_grad(m0[k], bwd[k + "_f64"]))
        print(kind, act, k, f"{err:.2e}", flush=True)
        assert err <= TOL, (k, err)
    for k in ("y", "dx", "dprobs"):
        assert torch.equal(acc[k], plain[k]), k


@pytest.mark.parametrize("kind,act,recompute", [("mxfp8", "swiglu", True), ("mxfp8", "srelu", False),
                                                ("nvfp4", "srelu", True), ("nvfp4", "swiglu", False)])
def test_deferred_wgrad_matches_one_backward_bitwise(kind, act, recompute):
    """A backward with defer_wgrad leaves dw1, dw2 to a later grouped_mlp_wgrad call: dx and dprobs
    as from one backward with two fewer GEMM launches; the later call (split scan + the two wgrad
    GEMMs), made after other work on the stream, gives bitwise the same weight gradients, and
    can be repeated, in fp32 or accumulated into an fp32 main_grad."""
    wl = small_case([100, 0, 300, 41], 256, 256, activation=act, recipe=kind, seed=12, w_std=0.05)
    d = _upload(wl)
    rec = g.recipe(kind, wl.sign_mask)
    w1q, w2q = g.weight_quantize(d["w1"], rec), g.weight_quantize(d["w2"], rec)
    _, ctx = g.grouped_mlp_forward(d["x"], d["splits"], w1q, w2q, d["probs"], act, rec, recompute=recompute)
    full = g.grouped_mlp_backward(d["dy"], d["splits"], w1q, w2q, d["probs"], ctx)
    full_counts = g.last_launch_counts()
    part = g.grouped_mlp_backward(d["dy"], d["splits"], w1q, w2q, d["probs"], ctx, defer_wgrad=True)
    part_counts = g.last_launch_counts()
    assert part["dw1"] is None and part["dw2"] is None
    assert part_counts["gemm"] == full_counts["gemm"] - 2
    # other work in between: a forward with buffers of its own
    g.grouped_mlp_forward(d["x"], d["splits"], w1q, w2q, d["probs"], act, rec, recompute=recompute)
    late = g.grouped_mlp_wgrad(part["deferred"])
    wg_counts = g.last_launch_counts()
    assert wg_counts["gemm"] == 2 and wg_counts["scan"] == 1 and sum(wg_counts.values()) == 3
    fp = g.grouped_mlp_wgrad(part["deferred"], wgrad_dtype=g.OUT_FP32)
    main = {k: torch.full(tuple(full[k].shape), 0.5, dtype=torch.float32, device="cuda") for k in ("dw1", "dw2")}
    acc = g.grouped_mlp_wgrad(part["deferred"], wgrad_dtype=g.OUT_FP32_ACCUMULATE, out=dict(main))
    torch.cuda.synchronize()
    for k in ("dx", "dprobs"):
        assert torch.equal(part[k], full[k]), k
    for k in ("dw1", "dw2"):
        assert torch.equal(late[k].view(torch.int16), full[k].view(torch.int16)), k
        assert torch.equal(acc[k], 0.5 + fp[k]), k
        assert torch.equal(fp[k].to(torch.bfloat16).view(torch.int16), full[k].view(torch.int16)), k


def test_tiny_config_forward():
    """2 experts, hidden 128, ffn 128, m_splits [64, 128], MXFP8 SwiGLU, forward only."""
    wl = make_workload("tiny")
    out = _run(wl, _upload(wl), "mxfp8", recompute=False, backward=False)
    _compare(out, wl, "mxfp8", backward=False)


def test_all_tokens_in_one_expert_and_empty_experts():
    wl = small_case([0, 0, 513, 0], 256, 256, activation="srelu", recipe="nvfp4", seed=4, w_std=0.05)
    out = _run(wl, _upload(wl), "nvfp4", recompute=True)
    _compare(out, wl, "nvfp4")


def test_nvfp4_weights_with_or_without_bf16_panels_bitwise():
    """Weights given as packed NVFP4 only (the GEMMs expand them into their workspace) or with the
    bf16 panels written at quantize time give bitwise-equal outputs and gradients."""
    wl = small_case([37, 0, 200, 64], 256, 384, activation="swiglu", recipe="nvfp4", seed=6, w_std=0.05)
    d = _upload(wl)
    rec = g.recipe("nvfp4", wl.sign_mask)
    E, H, ffn, F1 = 4, 256, 384, 768
    res = []
    for panels in (True, False):
        w1q = g.weight_quantize(d["w1"], rec, out=g.alloc_weight_q(rec, E, F1, H, bf16_panels=panels))
        w2q = g.weight_quantize(d["w2"], rec, out=g.alloc_weight_q(rec, E, H, ffn, bf16_panels=panels))
        y, ctx = g.grouped_mlp_forward(d["x"], d["splits"], w1q, w2q, d["probs"], "swiglu", rec)
        out = g.grouped_mlp_backward(d["dy"], d["splits"], w1q, w2q, d["probs"], ctx)
        out["y"] = y
        torch.cuda.synchronize()
        res.append(out)
    for k in ("y", "dx", "dprobs", "dw1", "dw2"):
        a, b = res[0][k], res[1][k]
        view = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
        assert torch.equal(a.view(view), b.view(view)), k
