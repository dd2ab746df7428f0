"""Pins for the oracle's grouped GEMMs, activations and forward / backward (CPU only)."""
import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import mlp as O
from workloads import small_case


def test_grouped_gemm_brute_force_loops():
    rng = np.random.default_rng(20)
    splits = [0, 1, 31, 33, 0, 64]
    n, k = 5, 9
    a = rng.integers(-3, 4, size=(sum(splits), k)).astype(np.float64)
    b = rng.integers(-3, 4, size=(len(splits), n, k)).astype(np.float64)
    got = O.grouped_gemm_nt(O._split_rows(a, splits), list(b))
    off = 0
    for g, m in enumerate(splits):
        want = np.zeros((m, n))
        for i in range(m):
            for j in range(n):
                s = 0.0
                for t in range(k):
                    s += a[off + i, t] * b[g, j, t]
                want[i, j] = s
        assert np.array_equal(got[g], want)
        off += m


def test_one_expert_is_a_dense_gemm():
    rng = np.random.default_rng(21)
    a = rng.standard_normal((40, 64))
    b = rng.standard_normal((24, 64))
    got = O.grouped_gemm_nt([a], [b])[0]
    want = torch.nn.functional.linear(torch.from_numpy(a), torch.from_numpy(b)).numpy()
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


TANH_SRELU_3 = (O.TANH_SRELU, 3.0)


@pytest.mark.parametrize("act", [O.SWIGLU, O.SRELU, TANH_SRELU_3, O.QGEGLU], ids=["swiglu", "srelu", "tanh_srelu",
                                                                                    "qgeglu"])
def test_activation_derivatives_by_central_differences(act):
    rng = np.random.default_rng(22)
    f = 6
    n1 = 2 * f if O.is_glu(act) else f
    relu_kind = O.act_kind(act)[0] in (O.SRELU, O.TANH_SRELU)
    h = rng.standard_normal((4, n1)) * 2
    h[0, 0] = 0.0
    h[1, 1] = -1.5
    p = rng.random(4)
    da = rng.standard_normal((4, f))
    dh, dprob = O.act_backward(h, da, p, act)
    eps = 1e-6

    def loss(hh, pp):
        return np.sum(da * O.act_forward(hh, act) * pp[:, None])

    for i in range(4):
        for j in range(n1):
            if relu_kind and abs(h[i, j]) < 1e-3:
                continue
            hp, hm = h.copy(), h.copy()
            hp[i, j] += eps
            hm[i, j] -= eps
            num = (loss(hp, p) - loss(hm, p)) / (2 * eps)
            assert abs(num - dh[i, j]) < 1e-6 * max(1, abs(num))
        pp, pm = p.copy(), p.copy()
        pp[i] += eps
        pm[i] -= eps
        num = (loss(h, pp) - loss(h, pm)) / (2 * eps)
        assert abs(num - dprob[i]) < 1e-6 * max(1, abs(num))
    if relu_kind:
        assert dh[1, 1] == 0.0 and dh[0, 0] == 0.0


def test_tanh_srelu_closed_forms():
    """c tanh(relu(h)^2 / c): tanh(ln(3) / 2) = 1/2 exactly, so relu(h)^2 = c ln(3) / 2 gives c / 2;
    no output for h <= 0; the clamp c for large h; the plain squared ReLU as c grows (tanh(x) = x to
    fp64 precision for x below 2^-27, and c a power of two makes (s / c) c exact)."""
    c = 2.0 / np.log(3.0)                          # relu(1)^2 / c = ln(3) / 2
    h = np.array([[1.0, 0.0, -2.0, 10.0]])
    got = O.act_forward(h, (O.TANH_SRELU, c))
    assert abs(got[0, 0] - c / 2) < 1e-15
    assert got[0, 1] == 0.0 and got[0, 2] == 0.0
    assert got[0, 3] == c                          # tanh(100 / c) rounds to 1
    big = 2.0 ** 80
    hh = np.random.default_rng(5).standard_normal((3, 8)) * 4
    assert np.array_equal(O.act_forward(hh, (O.TANH_SRELU, big)), O.act_forward(hh, O.SRELU))
    # dprob is the activation itself, da = 1
    _, dprob = O.act_backward(h, np.ones_like(h), np.ones(1), (O.TANH_SRELU, c))
    assert abs(dprob[0] - (c / 2 + c)) < 1e-14


def test_qgeglu_closed_forms_and_the_gelu_it_approximates():
    """gate sigmoid(1.702 gate) up: sigmoid(ln 3) = 3/4 exactly; gate 0 gives 0; it is SwiGLU at
    1.702 gate divided by 1.702; and g sigmoid(1.702 g) stays within 0.021 of the exact GELU
    g Phi(g) (Phi from scipy), which the constants 1 and 2 miss by twice that or more."""
    from scipy.special import ndtr
    g0 = np.log(3.0) / O.QUICK_GELU_K
    h = np.array([[g0, 0.0, 2.0, 5.0]])            # gate = [g0, 0], up = [2, 5]
    got = O.act_forward(h, O.QGEGLU)
    assert abs(got[0, 0] - g0 * 0.75 * 2.0) < 1e-15
    assert got[0, 1] == 0.0
    hh = np.random.default_rng(6).standard_normal((4, 10)) * 3
    sw = np.concatenate([hh[:, :5] * O.QUICK_GELU_K, hh[:, 5:]], axis=1)
    assert np.allclose(O.act_forward(hh, O.QGEGLU), O.act_forward(sw, O.SWIGLU) / O.QUICK_GELU_K,
                       rtol=1e-13, atol=1e-15)
    g = np.linspace(-8, 8, 4001)
    ones = np.ones_like(g)
    quick = O.act_forward(np.stack([g, ones], axis=1), O.QGEGLU)[:, 0]
    err = np.max(np.abs(quick - g * ndtr(g)))
    assert 0.015 < err < 0.021
    for k in (1.0, 2.0):
        assert np.max(np.abs(g / (1 + np.exp(-k * g)) - g * ndtr(g))) > 0.035


def _torch_reference(wl, act):
    """fp64 autograd of the unquantized grouped MLP (no rounding anywhere)."""
    x = torch.from_numpy(F.bf16_bits_to_f64(wl.x)).requires_grad_()
    w1 = torch.from_numpy(F.bf16_bits_to_f64(wl.w1)).requires_grad_()
    w2 = torch.from_numpy(F.bf16_bits_to_f64(wl.w2)).requires_grad_()
    p = torch.from_numpy(wl.probs.astype(np.float64)).requires_grad_()
    ys, off = [], 0
    for g, m in enumerate(wl.m_splits.tolist()):
        h = x[off:off + m] @ w1[g].T
        kind, c = O.act_kind(act)
        if kind == O.SWIGLU:
            f = h.shape[1] // 2
            a = torch.nn.functional.silu(h[:, :f]) * h[:, f:]
        elif kind == O.QGEGLU:
            f = h.shape[1] // 2
            a = h[:, :f] * torch.sigmoid(1.702 * h[:, :f]) * h[:, f:]
        elif kind == O.TANH_SRELU:
            a = c * torch.tanh(torch.relu(h) ** 2 / c)
        else:
            a = torch.relu(h) ** 2
        ys.append((a * p[off:off + m, None]) @ w2[g].T)
        off += m
    y = torch.cat(ys)
    dy = torch.from_numpy(F.bf16_bits_to_f64(wl.dy))
    (y * dy).sum().backward()
    return y.detach().numpy(), x.grad.numpy(), p.grad.numpy(), w1.grad.numpy(), w2.grad.numpy()


@pytest.mark.parametrize("recipe,act,tol", [(O.MXFP8, O.SWIGLU, 0.12), (O.NVFP4, O.SRELU, 0.35),
                                             (O.MXFP8, O.SRELU, 0.12), (O.NVFP4, O.SWIGLU, 0.35),
                                             (O.MXFP8, (O.TANH_SRELU, 2.0), 0.12), (O.NVFP4, O.QGEGLU, 0.35),
                                             (O.NVFP4, (O.TANH_SRELU, 2.0), 0.35), (O.MXFP8, O.QGEGLU, 0.12)])
def test_forward_backward_close_to_unquantized_autograd(recipe, act, tol):
    """Within the quantization-format error of torch fp64 autograd of the same MLP.

    Catches transposed operands, swapped gate/up halves, a missing prob or a wrong
    derivative anywhere in the oracle's forward or backward: each of those is O(1) off.
    """
    wl = small_case([0, 37, 64, 5, 90], 64, 96, activation=act, recipe=recipe, seed=3)
    rec = O.Recipe(recipe, wl.sign_mask)
    fwd = O.forward(wl.x, wl.m_splits, wl.w1, wl.w2, wl.probs, act, rec)
    bwd = O.backward(fwd, wl.dy)
    y, dx, dp, dw1, dw2 = _torch_reference(wl, act)
    assert O.rel_fro(fwd["y_f64"], y) < tol
    assert O.rel_fro(bwd["dx_f64"], dx) < tol * 1.5
    assert O.rel_fro(bwd["dprob"], dp) < tol
    assert O.rel_fro(bwd["dw1_f64"], dw1) < tol * 1.5
    assert O.rel_fro(bwd["dw2_f64"], dw2) < tol
    # empty expert: zero weight gradient
    assert np.all(bwd["dw1_f64"][0] == 0) and np.all(bwd["dw2_f64"][0] == 0)


def test_recompute_regenerates_the_activation_bitwise():
    """Rebuilding a from the saved bf16 h gives the forward's a and the same column-wise cast."""
    wl = small_case([33, 0, 70], 64, 64, activation=O.SRELU, recipe=O.NVFP4, seed=4)
    rec = O.Recipe(O.NVFP4, wl.sign_mask)
    fwd = O.forward(wl.x, wl.m_splits, wl.w1, wl.w2, wl.probs, O.SRELU, rec)
    a2 = F.round_bf16(O.act_forward(fwd["h"], O.SRELU) * fwd["probs"][:, None])
    a2_bits = F.f64_to_bf16_bits(a2)
    assert np.array_equal(a2_bits, fwd["a_bits"])
    # quantize the regenerated tensor with the forward's saved amax: identical column-wise data
    q2, _ = O.quantize_activation(a2_bits, fwd["m_splits"], rec, row=False, col=True,
                                  amax=(fwd["aq"]["amax_pre"], fwd["aq"]["amax_post"]))
    assert np.array_equal(q2["col_data"], fwd["aq"]["col_data"])
    assert np.array_equal(q2["col_scale"], fwd["aq"]["col_scale"])


def test_swiglu_halves_and_prob_placement():
    h = np.array([[1.0, -2.0, 3.0, 0.5]])       # gate = [1, -2], up = [3, 0.5]
    got = O.act_forward(h, O.SWIGLU)
    sig = lambda z: 1 / (1 + np.exp(-z))
    assert np.allclose(got, [[1 * sig(1) * 3, -2 * sig(-2) * 0.5]], rtol=1e-15)
    assert np.array_equal(O.act_forward(np.array([[-1.0, 2.0]]), O.SRELU), [[0.0, 4.0]])


@pytest.mark.parametrize("act", [O.SWIGLU, O.SRELU])
def test_sampled_rows_and_wgrad_entries_match_the_full_oracle(act):
    """The sampled evaluators used at full size (rows on their own, weight-gradient entries from
    two feature columns over a group's tokens) give the full unfused oracle's values: the same
    rounded h, a, da, dh and dprob, and y, dx, dW1, dW2 to fp64 summation-order noise."""
    splits = [70, 0, 161]
    wl = small_case(splits, 64, 96, activation=act, recipe=O.MXFP8, seed=11)
    rec = O.Recipe(O.MXFP8)
    fwd = O.forward(wl.x, splits, wl.w1, wl.w2, wl.probs, act, rec)
    bwd = O.backward(fwd, wl.dy)
    F1, ffn, H = wl.w1.shape[1], wl.w2.shape[2], wl.w1.shape[2]
    off = np.concatenate([[0], np.cumsum(splits)])
    for e in (0, 2):
        d1 = {"row": fwd["wq1"][1]["row"][e], "colT": fwd["wq1"][1]["colT"][e]}
        d2 = {"row": fwd["wq2"][1]["row"][e], "colT": fwd["wq2"][1]["colT"][e]}
        rows = np.array([off[e], off[e] + 1, off[e] + 33, off[e + 1] - 1])
        r = O.mxfp8_rows(wl.x[rows], wl.dy[rows], wl.probs[rows], d1, d2, act)
        for k, full in (("h", fwd["h"]), ("a", fwd["a"]), ("da", bwd["da"]), ("dh", bwd["dh"])):
            assert np.array_equal(r[k], full[rows]), k
        np.testing.assert_allclose(r["dprob"], bwd["dprob"][rows], rtol=1e-6, atol=1e-9)
        np.testing.assert_allclose(r["y_f64"], fwd["y_f64"][rows], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(r["dx_f64"], bwd["dx_f64"][rows], rtol=1e-10, atol=1e-12)
        i1 = [(0, 0), (F1 - 1, H - 1), (ffn // 2, 7), (F1 // 2 + 3, 40)]
        i2 = [(0, 0), (H - 1, ffn - 1), (5, 50)]
        w1e, w2e = O.mxfp8_wgrad_entries(wl.x[off[e]:off[e + 1]], wl.dy[off[e]:off[e + 1]],
                                         wl.probs[off[e]:off[e + 1]], d1, d2, act, i1, i2)
        np.testing.assert_allclose(w1e, [bwd["dw1_f64"][e, f, k] for f, k in i1], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(w2e, [bwd["dw2_f64"][e, n, f] for n, f in i2], rtol=1e-10, atol=1e-12)


def test_main_grad_accumulation_is_one_fp32_rounding():
    """fp32(main_grad + dW): for fp32 gradients it is IEEE fp32 addition (numpy's float32 add),
    bit for bit, across wide exponent ranges and cancellation; an fp64 gradient is rounded once,
    with ties to even, and never through bf16."""
    rng = np.random.default_rng(21)
    n = 20000
    main = (rng.standard_normal(n) * np.exp2(rng.integers(-40, 41, n))).astype(np.float32)
    dw = (rng.standard_normal(n) * np.exp2(rng.integers(-40, 41, n))).astype(np.float32)
    dw[:1000] = -main[:1000]                                    # exact cancellation
    dw[1000:2000] = 0.0                                         # an empty expert's zero gradient
    got = O.accumulate_main_grad(main, dw).astype(np.float32)
    assert np.array_equal(got.view(np.uint32)[1000:], (main + dw).view(np.uint32)[1000:])
    assert np.all(got[:1000] == 0.0)
    assert np.array_equal(got[1000:2000], main[1000:2000])
    # one rounding of the exact sum: 1 + 2^-24 is a tie (to even: 1), a hair above it rounds up
    assert O.accumulate_main_grad(1.0, 2.0 ** -24) == 1.0
    assert O.accumulate_main_grad(1.0, 2.0 ** -24 + 2.0 ** -40) == 1.0 + 2.0 ** -23
    # no bf16 step: 1 + 2^-20 survives (bf16 would make it 1)
    assert O.accumulate_main_grad(0.0, 1.0 + 2.0 ** -20) == 1.0 + 2.0 ** -20


# ----------------------------------------------------------------------------- hand-worked one-token cases
def _single_token_cases():
    """Cases of tests/golden/mlp_single_token.txt as (header, inputs, expected outputs)."""
    from conftest import read_golden
    cases, cur = [], None
    for line in read_golden("mlp_single_token.txt"):
        p = line.split()
        if p[0] == "case":
            kv = dict(zip(p[3::2], p[4::2]))
            cur = {"name": p[1], "act": p[2], "H": int(kv["H"]), "ffn": int(kv["ffn"]), "p": float(kv["p"]),
                   "in": [], "out": []}
            cases.append(cur)
        else:
            cur[p[0]].append((p[1], tuple(int(v) for v in p[2:-1]), float(p[-1])))
    return cases


def _run_single_token(case, skip_first_rounding=None):
    """The oracle's forward + backward of one case.  skip_first_rounding = "forward" / "backward"
    plants a mistake: that pass's first bf16 rounding (h, respectively da) is left out."""
    H, ffn = case["H"], case["ffn"]
    f1 = 2 * ffn if case["act"] == O.SWIGLU else ffn
    t = {"x": np.zeros((1, H)), "w1": np.zeros((1, f1, H)), "w2": np.zeros((1, H, ffn)), "dy": np.zeros((1, H))}
    for name, idx, v in case["in"]:
        t[name][idx] = v
    bits = {k: F.f64_to_bf16_bits(v) for k, v in t.items()}
    for k, v in t.items():
        assert np.array_equal(F.bf16_bits_to_f64(bits[k]), v), f"{k} must hold bf16 values"
    real = O.round_bf16

    def plant(phase):
        calls = []

        def rounding(x):
            calls.append(1)
            return np.asarray(x, np.float64) if (phase == skip_first_rounding and len(calls) == 1) else real(x)
        O.round_bf16 = rounding

    try:
        plant("forward")
        fwd = O.forward(bits["x"], [1], bits["w1"], bits["w2"], np.array([case["p"]], np.float32), case["act"],
                        O.Recipe(O.MXFP8))
        plant("backward")
        bwd = O.backward(fwd, bits["dy"])
    finally:
        O.round_bf16 = real
    got = {"y": F.round_bf16(fwd["y_f64"]), "dx": F.round_bf16(bwd["dx_f64"]), "dprob": bwd["dprob"],
           "dw1": F.round_bf16(bwd["dw1_f64"]), "dw2": F.round_bf16(bwd["dw2_f64"])}
    want = {k: np.zeros(v.shape) for k, v in got.items()}
    for name, idx, v in case["out"]:
        want[name][idx] = v
    return got, want


def _single_token_mismatches(**kw):
    bad = []
    for case in _single_token_cases():
        got, want = _run_single_token(case, **kw)
        bad += [(case["name"], k) for k in got if not np.array_equal(np.asarray(got[k], np.float64), want[k])]
    return bad


def test_single_token_hand_worked_cases():
    """Every output of the one-token cases equals the hand derivation exactly."""
    assert len(_single_token_cases()) == 3
    assert _single_token_mismatches() == []


@pytest.mark.parametrize("phase", ["forward", "backward"])
def test_single_token_cases_catch_a_missing_bf16_rounding(phase):
    """Planted mistake: h (forward) or da (backward) is used unrounded, where it feeds the activation
    or its gradient in fp64.  (a and dh reach the quantizer as bf16 bit patterns, so the oracle
    cannot skip their rounding; the GPU test of these cases pins those two on the kernels.)"""
    bad = _single_token_mismatches(skip_first_rounding=phase)
    assert bad, f"the first {phase} rounding left out, yet every hand-worked output still matches"
    assert any(name == "srelu_rounding" for name, _ in bad)


def test_single_token_cases_catch_prob_inside_the_activation(monkeypatch):
    """Planted mistake: the prob scales h before the activation instead of the activation's value."""
    real_fwd = O.act_forward

    def planted(h, activation):
        return real_fwd(h * 1.0625, activation) / 1.0625 if activation == O.SRELU else real_fwd(h, activation)

    monkeypatch.setattr(O, "act_forward", planted)
    assert _single_token_mismatches()


def test_single_token_cases_catch_swapped_gate_and_up(monkeypatch):
    """Planted mistake: SwiGLU takes the gate from the second half of h and the up from the first."""
    real_fwd, real_bwd = O.act_forward, O.act_backward

    def swap(h):
        f = h.shape[1] // 2
        return np.concatenate([h[:, f:], h[:, :f]], axis=1)

    monkeypatch.setattr(O, "act_forward", lambda h, a: real_fwd(swap(h), a) if a == O.SWIGLU else real_fwd(h, a))

    def bwd(h, da, p, a):
        if a != O.SWIGLU:
            return real_bwd(h, da, p, a)
        dh, dp = real_bwd(swap(h), da, p, a)
        return swap(dh), dp

    monkeypatch.setattr(O, "act_backward", bwd)
    assert ("swiglu_order", "dw1") in _single_token_mismatches()
