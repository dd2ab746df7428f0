"""The C ABI library: it loads, exports every symbol include/gmlp.h declares, and validates
arguments before touching a device (CPU only: no compute call reaches a GPU)."""
import ctypes
import os
import re

import pytest
import torch

import nvfp4_block_scaled_mxfp8_amd as g

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "gmlp.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gmlp_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = g.lib()
    names = declared_symbols()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    # and the binding declares a signature for each of them
    assert set(names) == set(g._SIGS), set(names) ^ set(g._SIGS)


def test_support_query_reasons():
    ok, why, st = g.check_support(8, 4096, 1536, "swiglu", g.recipe("mxfp8"), arch="gfx950")
    assert ok and st == 0
    ok, why, st = g.check_support(8, 4096, 1536, "swiglu", g.recipe("mxfp8"), arch="gfx942")
    assert not ok and why.startswith("system:") and st == 2
    ok, why, st = g.check_support(8, 4096, 1500, "swiglu", g.recipe("mxfp8"), arch="gfx950")
    assert not ok and why.startswith("dims:")
    ok, why, st = g.check_support(8, 4096, 1536, "swiglu", g.Recipe(7, 0), arch="gfx950")
    assert not ok and why.startswith("recipe:")
    ok, why, st = g.check_support(8, 4096, 1536, 5, g.recipe("mxfp8"), arch="gfx950")
    assert not ok and why.startswith("activation:")
    ok, why, st = g.check_support(0, 4096, 1536, "swiglu", g.recipe("nvfp4", 0x1234), arch="gfx950")
    assert not ok and st == 1


def test_query_sizes_grow_with_recompute_off():
    on = g.query_sizes(32768, 8, 4096, 1536, "swiglu", g.recipe("mxfp8"), recompute=True)
    off = g.query_sizes(32768, 8, 4096, 1536, "swiglu", g.recipe("mxfp8"), recompute=False)
    # without recompute the forward also keeps the column-wise fc2 input
    assert off["ctx_bytes"] - on["ctx_bytes"] >= 1536 * 32768
    assert on["ws_bytes"] > 0 and on["quant_ws_bytes"] > 0


def test_validation_happens_before_any_launch():
    """Bad arguments return an error status and a reason with null device pointers."""
    L = g.lib()
    q = g.GroupedQ()
    st = L.gmlp_group_quantize(None, 64, 100, None, 1, g.recipe("mxfp8"), 1, 1, ctypes.byref(q), None, 0, None)
    assert st == 2 and "multiple of 32" in g.last_error()
    st = L.gmlp_group_quantize(None, 64, 128, None, 1, g.recipe("mxfp8"), 1, 1, ctypes.byref(q), None, 0, None)
    assert st == 1 and "null" in g.last_error()
    st = L.gmlp_group_quantize_with_amax(None, 64, 128, None, 1, g.recipe("mxfp8"), 1, 1, ctypes.byref(q), None, 0,
                                         None)
    assert st == 2 and g.last_error().startswith("recipe:")
    st = L.gmlp_grouped_gemm(0, g.recipe("mxfp8"), ctypes.byref(q), ctypes.byref(q), ctypes.c_void_p(16), 1, 64,
                             128, 96, ctypes.c_void_p(16), 0, None, 0, None)
    assert st == 2 and "multiple of 128" in g.last_error()
    args = g.FwdArgs()
    args.E, args.M, args.H, args.ffn = 2, 64, 128, 100
    args.recipe = g.recipe("mxfp8")
    assert L.gmlp_grouped_mlp_forward(ctypes.byref(args), None) == 2
    assert "ffn" in g.last_error()


def test_grouped_gemm_workspace_query():
    """MXFP8 GEMMs need only the split tables; NVFP4 ones also hold both operands expanded to bf16."""
    mx = g.grouped_gemm_ws_bytes(g.GEMM_FPROP, g.recipe("mxfp8"), 8, 32768, 4096, 3072)
    assert 0 < mx < 1 << 20
    nv = g.grouped_gemm_ws_bytes(g.GEMM_FPROP, g.recipe("nvfp4", 1), 8, 32768, 4096, 3072)
    assert nv >= 2 * (32768 * 3072 + 8 * 4096 * 3072)
    wg = g.grouped_gemm_ws_bytes(g.GEMM_WGRAD, g.recipe("nvfp4", 1), 8, 32768, 4096, 1536)
    assert wg >= 2 * (4096 + 1536) * (32768 + 127 * 8)
    with pytest.raises(g.GmlpError):
        g.grouped_gemm_ws_bytes(5, g.recipe("mxfp8"), 8, 32768, 4096, 3072)


def test_nvfp4_sizes_hold_bf16_operand_panels():
    """Inside the fused MLP the NVFP4 casts are kept as bf16 GEMM panels (2 bytes per element)."""
    M, E, H, ffn = 24576, 8, 5120, 2048
    nv = g.query_sizes(M, E, H, ffn, "srelu", g.recipe("nvfp4", 3), recompute=False)
    assert nv["ctx_bytes"] >= 2 * H * M + 2 * ffn * M           # column-wise x and fc2 input panels
    assert nv["ws_bytes"] >= 2 * M * H                          # row-wise dy (or x) panels


def test_nvfp4_gemm_operand_validation():
    L = g.lib()
    q = g.GroupedQ()                                            # no data, scales or amax
    st = L.gmlp_grouped_gemm(0, g.recipe("nvfp4", 1), ctypes.byref(q), ctypes.byref(q), ctypes.c_void_p(16), 1, 64,
                             128, 128, ctypes.c_void_p(16), 0, None, 0, None)
    assert st == 1 and "amax" in g.last_error()


def test_launch_range_limits_are_reported():
    """Inputs too large for one launch's grid are rejected on the host with a dims reason."""
    L = g.lib()
    q = g.GroupedQ()
    # 2 x (M / 128 + G) half tiles must fit the grid's y dimension
    st = L.gmlp_group_quantize(None, 128 * 33000, 128, None, 1, g.recipe("mxfp8"), 1, 1, ctypes.byref(q), None, 0,
                               None)
    assert st == 2 and "tile range" in g.last_error()
    args = g.FwdArgs()
    args.E, args.M, args.H, args.ffn = 8, 600000, 128, 128
    args.recipe = g.recipe("nvfp4", 1)
    assert L.gmlp_grouped_mlp_forward(ctypes.byref(args), None) == 2
    assert "row range" in g.last_error()


def test_output_dtype_validation():
    """Unknown output dtypes are rejected, and accumulation is for weight gradients only."""
    L = g.lib()
    q = g.GroupedQ()
    dummy = ctypes.c_void_p(16)
    st = L.gmlp_grouped_gemm(1, g.recipe("mxfp8"), ctypes.byref(q), ctypes.byref(q), dummy, 1, 64, 128, 128, dummy,
                             7, None, 0, None)
    assert st == 1 and "output dtype" in g.last_error()
    st = L.gmlp_grouped_gemm(0, g.recipe("mxfp8"), ctypes.byref(q), ctypes.byref(q), dummy, 1, 64, 128, 128, dummy,
                             g.OUT_FP32_ACCUMULATE, None, 0, None)
    assert st == 2 and "WGRAD" in g.last_error()
    args = g.BwdArgs()
    args.E, args.M, args.H, args.ffn = 2, 64, 128, 128
    args.recipe = g.recipe("mxfp8")
    args.m_splits = args.dy = args.probs = args.dprobs = args.dw1 = args.dw2 = 16
    args.weight_requires_grad, args.wgrad_dtype = 1, 9
    assert L.gmlp_grouped_mlp_backward(ctypes.byref(args), None) == 1
    assert "wgrad dtype" in g.last_error()


def test_deferred_wgrad_validation():
    """The deferred weight-gradient call checks its arguments like the backward, before any launch."""
    L = g.lib()
    args = g.BwdArgs()
    args.E, args.M, args.H, args.ffn = 2, 64, 128, 128
    args.recipe = g.recipe("mxfp8")
    args.m_splits = args.dw1 = args.dw2 = 16
    assert L.gmlp_grouped_mlp_wgrad(ctypes.byref(args), None) == 1
    assert "weight_requires_grad" in g.last_error()
    args.weight_requires_grad = 1
    assert L.gmlp_grouped_mlp_wgrad(ctypes.byref(args), None) == 3          # no ctx / workspace
    assert "ctx too small" in g.last_error()
    args.wgrad_dtype = 4
    assert L.gmlp_grouped_mlp_wgrad(ctypes.byref(args), None) == 1
    assert "wgrad dtype" in g.last_error()


def test_accumulating_gradients_need_the_callers_main_grads():
    """The binding refuses OUT_FP32_ACCUMULATE without existing fp32 main_grads of the right shape
    (host check, before any launch), in the backward and in the deferred weight-gradient call."""
    import torch
    E, M, H, ffn = 2, 64, 128, 128
    rec = g.recipe("mxfp8")
    ctx = g.MlpContext(torch.empty(0, dtype=torch.uint8), M, E, H, ffn, g.SWIGLU, rec, False, True, True)
    dy = torch.zeros(M, H, dtype=torch.bfloat16)
    splits = torch.tensor([M // 2, M // 2], dtype=torch.int32)
    probs = torch.zeros(M)
    with pytest.raises(ValueError, match="main_grad"):
        g.grouped_mlp_backward(dy, splits, None, None, probs, ctx, wgrad_dtype=g.OUT_FP32_ACCUMULATE)
    bad = {"dw1": torch.zeros(E, 2 * ffn, H, dtype=torch.bfloat16), "dw2": torch.zeros(E, H, ffn)}
    with pytest.raises(ValueError, match="dw1 main_grad"):
        g.grouped_mlp_backward(dy, splits, None, None, probs, ctx, wgrad_dtype=g.OUT_FP32_ACCUMULATE, out=bad)
    deferred = g.DeferredWgrad(splits, ctx, torch.empty(0, dtype=torch.uint8))
    with pytest.raises(ValueError, match="main_grad"):
        g.grouped_mlp_wgrad(deferred, wgrad_dtype=g.OUT_FP32_ACCUMULATE)


def test_binding_refuses_host_tensors():
    """The Python binding hands the library device addresses only: a host tensor among the
    arguments is refused (ValueError naming it) before any library call that launches work."""
    rec = g.recipe("mxfp8")
    x = torch.zeros((64, 128), dtype=torch.bfloat16)
    splits = torch.tensor([64], dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU tensor"):
        g.group_quantize(x, splits, rec)
    with pytest.raises(ValueError, match="GPU tensor"):
        g.group_hadamard_amax(x, splits, 0x5A5A)
    with pytest.raises(ValueError, match="GPU tensor"):
        g.weight_quantize(torch.zeros((2, 128, 128), dtype=torch.bfloat16), rec)
    with pytest.raises(ValueError, match=r"w\[0\]"):
        g.weight_quantize([torch.zeros((128, 128), dtype=torch.bfloat16)] * 2, rec)
    q = g.alloc_grouped_q(rec, 64, 128, 1, device="cpu")
    with pytest.raises(ValueError, match="GPU tensor"):
        g.grouped_gemm(g.GEMM_FPROP, rec, q, q, splits, 64, 64, 128)
    with pytest.raises(ValueError, match="GPU tensor"):
        g.read_device_flags(torch.zeros(16, dtype=torch.uint8))


def test_binding_checks_the_dtypes_and_sizes_the_kernels_read():
    """probs is read as M fp32 values and m_splits as G int32 values: other dtypes or sizes would be
    read past their ends or misread, so the binding refuses them (host check, before any launch);
    caller-given outputs must have the shapes and dtypes the kernels write."""
    E, M, H, ffn = 2, 64, 128, 128
    rec = g.recipe("mxfp8")
    ctx = g.MlpContext(torch.empty(0, dtype=torch.uint8), M, E, H, ffn, g.SWIGLU, rec, False, True, True)
    dy = torch.zeros(M, H, dtype=torch.bfloat16)
    splits = torch.tensor([M // 2, M // 2], dtype=torch.int32)
    probs = torch.zeros(M)
    with pytest.raises(TypeError, match="probs"):
        g.grouped_mlp_backward(dy, splits, None, None, probs.to(torch.bfloat16), ctx)
    with pytest.raises(TypeError, match="probs"):
        g.grouped_mlp_backward(dy, splits, None, None, probs[:-1], ctx)
    with pytest.raises(TypeError, match="m_splits"):
        g.grouped_mlp_backward(dy, splits.long(), None, None, probs, ctx)
    with pytest.raises(ValueError, match="m_splits"):
        g.grouped_mlp_backward(dy, splits[:1], None, None, probs, ctx)
    with pytest.raises(ValueError, match="dprobs"):
        g.grouped_mlp_backward(dy, splits, None, None, probs, ctx, out={"dprobs": torch.zeros(M - 1)})
    with pytest.raises(ValueError, match="dx"):
        g.grouped_mlp_backward(dy, splits, None, None, probs, ctx, out={"dx": torch.zeros(M, H)})
    with pytest.raises(TypeError, match="m_splits"):
        g.group_quantize(dy, splits.long(), rec)
    with pytest.raises(TypeError, match="probs"):
        g.grouped_mlp_forward(dy, splits, None, None, probs.double(), "swiglu", rec)


def test_binding_checks_quantized_buffer_sizes():
    """A caller-given quantized tensor smaller than the call's sizes need is refused (host check,
    before any launch): the kernels address it from the sizes, not from the buffers."""
    rec = g.recipe("mxfp8")
    x = torch.zeros((64, 128), dtype=torch.bfloat16)
    splits = torch.tensor([64], dtype=torch.int32)
    small = g.alloc_grouped_q(rec, 32, 128, 1, device="cpu")
    with pytest.raises(ValueError, match="row_data"):
        g.group_quantize(x, splits, rec, out=small)
    wsmall = g.alloc_weight_q(rec, 2, 128, 64, device="cpu")
    with pytest.raises(ValueError, match="out.row_data"):
        g.weight_quantize(torch.zeros((2, 128, 128), dtype=torch.bfloat16), rec, out=wsmall)
    w1q = g.alloc_weight_q(rec, 2, 256, 128, device="cpu")       # SwiGLU F1 = 2 ffn with ffn 128
    w2q = g.alloc_weight_q(rec, 2, 128, 128, device="cpu")
    probs = torch.zeros(64)
    splits2 = torch.tensor([32, 32], dtype=torch.int32)
    w1_small = g.alloc_weight_q(rec, 2, 128, 128, device="cpu")  # F1 = ffn: too small for SwiGLU
    with pytest.raises(ValueError, match="w1q"):
        g.grouped_mlp_forward(x, splits2, w1_small, w2q, probs, "swiglu", rec)
    # the right sizes pass the size check and stop at the host-tensor check
    with pytest.raises(ValueError, match="GPU tensor"):
        g.grouped_mlp_forward(x, splits2, w1q, w2q, probs, "swiglu", rec)


@pytest.mark.parametrize("kind", ["mxfp8", "nvfp4"])
def test_allocators_satisfy_the_size_checks(kind):
    """What alloc_grouped_q and alloc_weight_q allocate passes the binding's size checks for the
    same sizes (the checks take the least the kernels address; the allocators the most)."""
    rec = g.recipe(kind, 1)
    for M, K, G in ((1, 128, 1), (192, 256, 2), (1000, 384, 7), (0, 128, 3)):
        g._check_q_sizes(g.alloc_grouped_q(rec, M, K, G, device="meta"), g._grouped_need(rec, M, K, G), "q")
    for E, N, K in ((1, 128, 128), (3, 256, 384)):
        g._check_q_sizes(g.alloc_weight_q(rec, E, N, K, device="meta"), g._weight_need(rec, E, N, K), "w")
    # and one buffer a row short is refused
    q = g.alloc_grouped_q(rec, 192, 256, 2, device="meta")
    q.bufs["row_data"] = q.bufs["row_data"][:-1]
    with pytest.raises(ValueError, match="row_data"):
        g._check_q_sizes(q, g._grouped_need(rec, 192, 256, 2), "q")
