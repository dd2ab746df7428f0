"""gmlp_group_quantize_noalloc (the group quantize whose workspace is the library's fixed device
array) against gmlp_group_quantize with a caller workspace, through the C ABI: bit for bit, two
calls in a row, the second with fewer rows and fewer groups (the array keeps the first call's
contents, so the second must not depend on them)."""
import ctypes

import numpy as np
import pytest
import torch

import nvfp4_block_scaled_mxfp8_amd as g
from gpu_util import dev_bf16, dev_splits
from workloads import random_bf16

pytestmark = pytest.mark.gpu

CALLS = [([300, 0, 517, 33, 129], 256, 11), ([65, 200], 128, 12)]


def _buffers(q):
    return {k: v.detach().cpu().clone() for k, v in q.bufs.items()}


def _call(name, x, splits, rec, q, ws=None):
    M, K = x.shape
    st = q.struct()
    L = g.lib()
    if ws is None:
        status = L.gmlp_group_quantize_noalloc(g._p(x), M, K, g._p(splits), splits.numel(), rec, 1, 1,
                                               ctypes.byref(st), g._stream())
    else:
        status = L.gmlp_group_quantize(g._p(x), M, K, g._p(splits), splits.numel(), rec, 1, 1, ctypes.byref(st),
                                       g._p(ws), ws.numel(), g._stream())
    assert status == 0, (name, g.last_error())


@pytest.mark.parametrize("kind", ["mxfp8", "nvfp4"])
def test_noalloc_matches_workspace_call_twice(kind):
    rec = g.recipe(kind, 0x4C3D)
    for splits, K, seed in CALLS:
        M, G = sum(splits), len(splits)
        print(f"noalloc {kind}: splits={splits} K={K}", flush=True)
        x = dev_bf16(random_bf16((M, K), seed=seed, dist="wide" if kind == "mxfp8" else "normal"))
        sd = dev_splits(splits)
        ref = g.alloc_grouped_q(rec, M, K, G, True, True)
        got = g.alloc_grouped_q(rec, M, K, G, True, True)
        for t in list(ref.bufs.values()) + list(got.bufs.values()):
            t.fill_(0)
        ws = g.quant_workspace(G, "cuda")
        _call("with workspace", x, sd, rec, ref, ws)
        _call("noalloc", x, sd, rec, got)
        torch.cuda.synchronize()
        a, b = _buffers(ref), _buffers(got)
        assert a.keys() == b.keys()
        for k in a:
            assert torch.equal(a[k].view(torch.uint8), b[k].view(torch.uint8)), (kind, splits, k)


def test_noalloc_rejects_too_many_groups():
    """More groups than the static workspace holds: an error before anything is enqueued."""
    x = dev_bf16(np.zeros((4, 128), np.uint16))
    sd = dev_splits([1] * 4 + [0] * 1021)
    q = g.alloc_grouped_q(g.recipe("mxfp8"), 4, 128, 1025, True, True)
    st = q.struct()
    status = g.lib().gmlp_group_quantize_noalloc(g._p(x), 4, 128, g._p(sd), 1025, g.recipe("mxfp8"), 1, 1,
                                                 ctypes.byref(st), g._stream())
    assert status == 2 and "1024 groups" in g.last_error()
