"""torch.autograd over the fused grouped MLP (GroupedMLPFunction, grouped_mlp): the gradients that
autograd delivers are bit for bit those of the direct forward + backward calls on the same
operands, a frozen input or frozen weights get no gradient, and with accumulate_main_grad the weight
gradients are added to the weights' fp32 main_grad exactly as the backward's accumulate output adds them."""
import pytest
import torch

import nvfp4_block_scaled_mxfp8_amd as g
from gpu_util import bits16, dev_bf16, dev_f32, dev_splits
from workloads import small_case

pytestmark = pytest.mark.gpu

CASES = [("mxfp8", "swiglu"), ("nvfp4", "srelu")]


def _case(kind, act):
    wl = small_case([0, 37, 300, 129, 5], 512, 384, activation=act, recipe=kind, seed=3, w_std=0.05)
    E, H, ffn, F1 = wl.config.experts, wl.config.hidden, wl.config.ffn, wl.config.f1
    d = {"x": dev_bf16(wl.x), "splits": dev_splits(wl.m_splits), "probs": dev_f32(wl.probs),
         "w1": dev_bf16(wl.w1.reshape(E * F1, H)).view(E, F1, H),
         "w2": dev_bf16(wl.w2.reshape(E * H, ffn)).view(E, H, ffn), "dy": dev_bf16(wl.dy)}
    rec = g.recipe(kind, wl.sign_mask)
    return wl, d, rec, g.weight_quantize(d["w1"], rec), g.weight_quantize(d["w2"], rec)


def _same(a, b, what):
    assert a is not None and b is not None, what
    assert a.dtype == b.dtype and a.shape == b.shape, what
    if a.dtype == torch.bfloat16:
        assert (bits16(a) == bits16(b)).all(), what
    else:
        assert torch.equal(a.detach().cpu(), b.detach().cpu()), what


@pytest.mark.parametrize("kind,act", CASES, ids=[f"{k}-{a}" for k, a in CASES])
@pytest.mark.parametrize("recompute", [False, True], ids=["saved", "recompute"])
def test_autograd_gradients_equal_the_direct_calls(kind, act, recompute):
    print(f"autograd {kind} {act} recompute={recompute}", flush=True)
    wl, d, rec, w1q, w2q = _case(kind, act)
    y_ref, ctx = g.grouped_mlp_forward(d["x"], d["splits"], w1q, w2q, d["probs"], act, rec, recompute=recompute)
    ref = g.grouped_mlp_backward(d["dy"], d["splits"], w1q, w2q, d["probs"], ctx)

    x = d["x"].clone().requires_grad_(True)
    probs = d["probs"].clone().requires_grad_(True)
    w1 = d["w1"].clone().requires_grad_(True)
    w2 = d["w2"].clone().requires_grad_(True)
    y = g.grouped_mlp(x, probs, w1, w2, d["splits"], act, rec, w1q=w1q, w2q=w2q, recompute=recompute)
    y.backward(d["dy"])
    torch.cuda.synchronize()
    _same(y, y_ref, "y")
    _same(x.grad, ref["dx"], "dx")
    _same(probs.grad, ref["dprobs"], "dprobs")
    _same(w1.grad, ref["dw1"], "dw1")
    _same(w2.grad, ref["dw2"], "dw2")


def test_autograd_quantizes_the_weights_itself_and_respects_frozen_tensors():
    wl, d, rec, w1q, w2q = _case("mxfp8", "swiglu")
    y_ref, ctx = g.grouped_mlp_forward(d["x"], d["splits"], w1q, w2q, d["probs"], "swiglu", rec)
    ref = g.grouped_mlp_backward(d["dy"], d["splits"], w1q, w2q, d["probs"], ctx)

    # weights quantized inside the call (the same weight_quantize), weights frozen
    x = d["x"].clone().requires_grad_(True)
    probs = d["probs"].clone().requires_grad_(True)
    w1, w2 = d["w1"].clone(), d["w2"].clone()
    y = g.grouped_mlp(x, probs, w1, w2, d["splits"], "swiglu", rec)
    y.backward(d["dy"])
    torch.cuda.synchronize()
    _same(y, y_ref, "y")
    _same(x.grad, ref["dx"], "dx")
    _same(probs.grad, ref["dprobs"], "dprobs")
    assert w1.grad is None and w2.grad is None

    # input frozen, weights trained
    x = d["x"].clone()
    probs = d["probs"].clone().requires_grad_(True)
    w1 = d["w1"].clone().requires_grad_(True)
    w2 = d["w2"].clone().requires_grad_(True)
    y = g.grouped_mlp(x, probs, w1, w2, d["splits"], "swiglu", rec, w1q=w1q, w2q=w2q)
    y.backward(d["dy"])
    torch.cuda.synchronize()
    assert x.grad is None
    _same(probs.grad, ref["dprobs"], "dprobs")
    _same(w1.grad, ref["dw1"], "dw1")
    _same(w2.grad, ref["dw2"], "dw2")


@pytest.mark.parametrize("kind,act", CASES, ids=[f"{k}-{a}" for k, a in CASES])
def test_autograd_accumulates_into_main_grad(kind, act):
    print(f"autograd main_grad {kind} {act}", flush=True)
    wl, d, rec, w1q, w2q = _case(kind, act)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    mg1 = torch.randn(d["w1"].shape, device="cuda", generator=gen)
    mg2 = torch.randn(d["w2"].shape, device="cuda", generator=gen)
    ref1, ref2 = mg1.clone(), mg2.clone()
    w1 = d["w1"].clone().requires_grad_(True)
    w2 = d["w2"].clone().requires_grad_(True)
    w1.main_grad, w2.main_grad = mg1, mg2
    for step in range(2):                         # two steps: the second adds to the first's sums
        _, ctx = g.grouped_mlp_forward(d["x"], d["splits"], w1q, w2q, d["probs"], act, rec)
        ref = g.grouped_mlp_backward(d["dy"], d["splits"], w1q, w2q, d["probs"], ctx,
                                     wgrad_dtype=g.OUT_FP32_ACCUMULATE, out={"dw1": ref1, "dw2": ref2})
        x = d["x"].clone().requires_grad_(True)
        y = g.grouped_mlp(x, d["probs"], w1, w2, d["splits"], act, rec, w1q=w1q, w2q=w2q,
                          accumulate_main_grad=True)
        y.backward(d["dy"])
        torch.cuda.synchronize()
        _same(x.grad, ref["dx"], f"dx step {step}")
        _same(w1.main_grad, ref1, f"w1.main_grad step {step}")
        _same(w2.main_grad, ref2, f"w2.main_grad step {step}")
        assert w1.grad is None and w2.grad is None


def test_autograd_only_the_routing_probabilities_trained():
    """x and the weights frozen, probs trained: the backward computes dprobs alone (no dgrad or
    wgrad GEMM of fc1), bit for bit the full backward's."""
    wl, d, rec, w1q, w2q = _case("nvfp4", "srelu")
    _, ctx = g.grouped_mlp_forward(d["x"], d["splits"], w1q, w2q, d["probs"], "srelu", rec)
    ref = g.grouped_mlp_backward(d["dy"], d["splits"], w1q, w2q, d["probs"], ctx)
    probs = d["probs"].clone().requires_grad_(True)
    w1, w2 = d["w1"].clone(), d["w2"].clone()
    y = g.grouped_mlp(d["x"], probs, w1, w2, d["splits"], "srelu", rec, w1q=w1q, w2q=w2q)
    y.backward(d["dy"])
    torch.cuda.synchronize()
    _same(probs.grad, ref["dprobs"], "dprobs")
    assert w1.grad is None and w2.grad is None
