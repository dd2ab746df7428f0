"""The fused forward + backward and the allocation-free group quantize captured into a HIP graph
(torch.cuda.CUDAGraph): every call is stream-ordered, allocates nothing itself and records no
memset, so a captured graph replays the same work.  Each replay, with other work and host
synchronisations in between, must give the eager call's outputs bit for bit."""
import ctypes

import pytest
import torch

import nvfp4_block_scaled_mxfp8_amd as g
from gpu_util import dev_bf16, dev_f32, dev_splits
from workloads import random_bf16, small_case

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _upload(wl):
    E, H, ffn, F1 = wl.config.experts, wl.config.hidden, wl.config.ffn, wl.config.f1
    return {"x": dev_bf16(wl.x), "splits": dev_splits(wl.m_splits), "probs": dev_f32(wl.probs), "dy": dev_bf16(wl.dy),
            "w1": dev_bf16(wl.w1.reshape(E * F1, H)).view(E, F1, H),
            "w2": dev_bf16(wl.w2.reshape(E * H, ffn)).view(E, H, ffn)}


def _step(d, w1q, w2q, act, rec, recompute):
    y, ctx = g.grouped_mlp_forward(d["x"], d["splits"], w1q, w2q, d["probs"], act, rec, recompute=recompute)
    out = g.grouped_mlp_backward(d["dy"], d["splits"], w1q, w2q, d["probs"], ctx)
    out["y"] = y
    return out


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("kind,act,recompute", [("mxfp8", "swiglu", False), ("nvfp4", "srelu", True),
                                                ("mxfp8", ("tanh_srelu", 2.0), True)],
                         ids=["mxfp8-swiglu", "nvfp4-srelu-recompute", "mxfp8-tanh_srelu-recompute"])
def test_forward_backward_graph_replays_match_eager(kind, act, recompute):
    print(f"graph {kind} {act} recompute={recompute}", flush=True)
    wl = small_case([0, 37, 300, 129, 5], 256, 256, activation=act, recipe=kind, seed=21, w_std=0.05)
    d = _upload(wl)
    rec = g.recipe(kind, wl.sign_mask)
    w1q, w2q = g.weight_quantize(d["w1"], rec), g.weight_quantize(d["w2"], rec)
    ref = _step(d, w1q, w2q, act, rec, recompute)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in ref.items() if torch.is_tensor(v)}
    # warm up on a side stream, as torch asks before capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(d, w1q, w2q, act, rec, recompute)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = _step(d, w1q, w2q, act, rec, recompute)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        for k in ref:                         # the graph must write every output itself
            out[k].fill_(7 if out[k].dtype != torch.bfloat16 else 0)
        _step(d, w1q, w2q, act, rec, not recompute)       # other work on the stream in between
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in ref.items():
            assert torch.equal(_bits(out[k]), _bits(v)), (r, k)
    del graph


def test_noalloc_group_quantize_graph_replays_match_eager():
    """gmlp_group_quantize_noalloc, the entry point for callers that cannot allocate, captured:
    the replays' outputs equal the eager call's, also after an eager call with other sizes has
    rewritten the library's fixed workspace in between."""
    rec = g.recipe("nvfp4", 0x2B71)
    splits_list = [300, 0, 517, 33, 129]
    M, K = sum(splits_list), 256
    x = dev_bf16(random_bf16((M, K), seed=5))
    splits = dev_splits(splits_list)
    q = g.alloc_grouped_q(rec, M, K, len(splits_list), True, True)
    x2 = dev_bf16(random_bf16((100, 128), seed=6))
    splits2 = dev_splits([60, 40])
    q2 = g.alloc_grouped_q(rec, 100, 128, 2, True, True)

    def call(xx, ss, qq):
        st = qq.struct()
        status = g.lib().gmlp_group_quantize_noalloc(g._p(xx), xx.shape[0], xx.shape[1], g._p(ss), ss.numel(), rec,
                                                     1, 1, ctypes.byref(st), g._stream())
        assert status == 0, g.last_error()

    for v in q.bufs.values():                 # the buffers' unwritten padding compares as zeros
        v.zero_()
    call(x, splits, q)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in q.bufs.items()}
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(x, splits, q)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        for v in q.bufs.values():
            v.zero_()
        call(x2, splits2, q2)                 # rewrites the fixed workspace with other split tables
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in ref.items():
            assert torch.equal(q.bufs[k], v), (r, k)
    del graph
