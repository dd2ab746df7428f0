"""Fused MoE grouped MLP with MXFP8 / NVFP4 group quantization on MI355X (gfx950).

Python binding of libgmlp.so (include/gmlp.h): argument marshalling only.  Every
step of the path runs in the library's HIP kernels; torch only allocates device
memory and supplies the stream.  The library must be built (python -m
nvfp4_block_scaled_mxfp8_amd.build); nothing here falls back to another
implementation when it is missing.

Names follow the C ABI: group_quantize (and group_quantize_noalloc), group_hadamard_amax,
group_quantize_with_amax, weight_quantize, grouped_gemm, grouped_mlp_forward,
grouped_mlp_backward.  grouped_mlp (GroupedMLPFunction) puts the fused forward and backward
under torch.autograd.
"""
import ctypes
import os
from dataclasses import dataclass, field

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgmlp.so")

MXFP8, NVFP4_RHT = 0, 1
SWIGLU, SRELU, TANH_SRELU, QGEGLU = 0, 1, 2, 3
OUT_BF16, OUT_FP32, OUT_FP32_ACCUMULATE = 0, 1, 2
GEMM_FPROP, GEMM_WGRAD, GEMM_DGRAD = 0, 1, 2
STATUS = {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "WORKSPACE", 4: "HIP_ERROR"}
COL_PAD = 128
LAUNCH_KINDS = ("scan", "mxfp8_quantize", "hadamard_amax", "nvfp4_quantize", "gemm", "dprob_reduce", "fill")


class GmlpError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"gmlp {STATUS.get(status, status)}: {msg}")
        self.status = status


# ----------------------------------------------------------------------------- C structs
class Recipe(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("rht_sign_mask", ctypes.c_uint32)]


_Q_FIELDS = ("row_data", "row_scale", "row_scale_mfma", "col_data", "col_scale", "col_scale_mfma",
             "amax_pre", "amax_post", "row_bf16", "col_bf16")


class GroupedQ(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _Q_FIELDS]


class Sizes(ctypes.Structure):
    _fields_ = [("ctx_bytes", ctypes.c_size_t), ("ws_bytes", ctypes.c_size_t),
                ("quant_ws_bytes", ctypes.c_size_t)]


class FwdArgs(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("m_splits", ctypes.c_void_p), ("M", ctypes.c_int64),
                ("E", ctypes.c_int32), ("H", ctypes.c_int64), ("ffn", ctypes.c_int64),
                ("w1", ctypes.POINTER(GroupedQ)), ("w2", ctypes.POINTER(GroupedQ)),
                ("probs", ctypes.c_void_p), ("activation", ctypes.c_int32), ("recipe", Recipe),
                ("recompute", ctypes.c_int32), ("input_requires_grad", ctypes.c_int32),
                ("weight_requires_grad", ctypes.c_int32), ("y", ctypes.c_void_p),
                ("ctx", ctypes.c_void_p), ("ctx_bytes", ctypes.c_size_t),
                ("ws", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t), ("fc2_amax_in_fc1", ctypes.c_int32),
                ("tanh_clamp_scale", ctypes.c_float)]


class BwdArgs(ctypes.Structure):
    _fields_ = [("dy", ctypes.c_void_p), ("m_splits", ctypes.c_void_p), ("M", ctypes.c_int64),
                ("E", ctypes.c_int32), ("H", ctypes.c_int64), ("ffn", ctypes.c_int64),
                ("w1", ctypes.POINTER(GroupedQ)), ("w2", ctypes.POINTER(GroupedQ)),
                ("probs", ctypes.c_void_p), ("activation", ctypes.c_int32), ("recipe", Recipe),
                ("recompute", ctypes.c_int32), ("input_requires_grad", ctypes.c_int32),
                ("weight_requires_grad", ctypes.c_int32), ("dx", ctypes.c_void_p),
                ("dprobs", ctypes.c_void_p), ("dw1", ctypes.c_void_p), ("dw2", ctypes.c_void_p),
                ("wgrad_dtype", ctypes.c_int32), ("ctx", ctypes.c_void_p),
                ("ctx_bytes", ctypes.c_size_t), ("ws", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t),
                ("defer_wgrad", ctypes.c_int32), ("tanh_clamp_scale", ctypes.c_float)]


_SIGS = {
    "gmlp_last_error": (ctypes.c_char_p, []),
    "gmlp_check_support": (ctypes.c_int, [ctypes.c_char_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_int32, Recipe]),
    "gmlp_query_sizes": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_int32, Recipe, ctypes.c_int32, ctypes.POINTER(Sizes)]),
    "gmlp_read_device_flags": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_uint32), ctypes.c_void_p]),
    "gmlp_group_quantize": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                           ctypes.c_int32, Recipe, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.POINTER(GroupedQ), ctypes.c_void_p, ctypes.c_size_t,
                                           ctypes.c_void_p]),
    "gmlp_group_quantize_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                                   ctypes.c_void_p, ctypes.c_int32, Recipe, ctypes.c_int32,
                                                   ctypes.c_int32, ctypes.POINTER(GroupedQ), ctypes.c_void_p]),
    "gmlp_group_hadamard_amax": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                                ctypes.c_int32, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p,
                                                ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "gmlp_group_quantize_with_amax": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                                     ctypes.c_void_p, ctypes.c_int32, Recipe, ctypes.c_int32,
                                                     ctypes.c_int32, ctypes.POINTER(GroupedQ), ctypes.c_void_p,
                                                     ctypes.c_size_t, ctypes.c_void_p]),
    "gmlp_weight_quantize": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                            ctypes.c_int64, Recipe, ctypes.POINTER(GroupedQ), ctypes.c_void_p,
                                            ctypes.c_size_t, ctypes.c_void_p]),
    "gmlp_grouped_gemm": (ctypes.c_int, [ctypes.c_int32, Recipe, ctypes.POINTER(GroupedQ),
                                         ctypes.POINTER(GroupedQ), ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                         ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32,
                                         ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "gmlp_grouped_mlp_forward": (ctypes.c_int, [ctypes.POINTER(FwdArgs), ctypes.c_void_p]),
    "gmlp_grouped_mlp_backward": (ctypes.c_int, [ctypes.POINTER(BwdArgs), ctypes.c_void_p]),
    "gmlp_forward_saved": (ctypes.c_int, [ctypes.POINTER(FwdArgs), ctypes.POINTER(ctypes.c_void_p),
                                          ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_void_p)]),
    "gmlp_grouped_mlp_wgrad": (ctypes.c_int, [ctypes.POINTER(BwdArgs), ctypes.c_void_p]),
    "gmlp_last_launch_counts": (ctypes.c_int, [ctypes.POINTER(ctypes.c_int32), ctypes.c_int32]),
    "gmlp_grouped_gemm_ws_bytes": (ctypes.c_int, [ctypes.c_int32, Recipe, ctypes.c_int32, ctypes.c_int64,
                                                  ctypes.c_int64, ctypes.c_int64, ctypes.POINTER(ctypes.c_size_t)]),
}

_lib = None


def lib():
    """The loaded libgmlp.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m nvfp4_block_scaled_mxfp8_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status):
    if status != 0:
        raise GmlpError(status, lib().gmlp_last_error().decode())


def _dev_ptr(t, name="tensor"):
    """The device address of a GPU tensor (None for None).  Every pointer the library receives
    goes through here: a host tensor would reach a kernel as a host address, so it is refused."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        where = t.device if isinstance(t, torch.Tensor) else type(t).__name__
        raise ValueError(f"{name}: a GPU tensor is required, got {where}")
    return t.data_ptr()


def _p(t, name="tensor"):
    return ctypes.c_void_p(_dev_ptr(t, name) or 0)


def _stream(device=None):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def recipe(kind="mxfp8", sign_mask=0):
    k = {"mxfp8": MXFP8, "nvfp4": NVFP4_RHT, MXFP8: MXFP8, NVFP4_RHT: NVFP4_RHT}[kind]
    return Recipe(k, int(sign_mask) & 0xFFFF)


_ACT_NAMES = {"swiglu": SWIGLU, "srelu": SRELU, "tanh_srelu": TANH_SRELU, "qgeglu": QGEGLU}


def activation_spec(act):
    """An activation as (C enum, tanh clamp scale): 'swiglu', 'srelu', 'qgeglu', or
    ('tanh_srelu', c); integers (or (int, c)) pass through (the library validates them)."""
    if isinstance(act, tuple):
        name, c = act
        return (name if isinstance(name, int) else _ACT_NAMES[name]), float(c)
    return (act if isinstance(act, int) else _ACT_NAMES[act]), 0.0


def activation_id(act):
    return activation_spec(act)[0]


def is_glu(act):
    """Gated activations read h = [gate | up] (F1 = 2 ffn)."""
    return activation_id(act) in (SWIGLU, QGEGLU)


def last_error():
    return lib().gmlp_last_error().decode()


def last_launch_counts():
    c = (ctypes.c_int32 * 8)()
    _check(lib().gmlp_last_launch_counts(c, 8))
    return dict(zip(LAUNCH_KINDS, list(c)[:7]))


def check_support(experts, hidden, ffn, activation="swiglu", rec=None, arch=None):
    """(ok, reason) -- host-only support query; arch=None asks device 0."""
    rec = rec if rec is not None else recipe()
    st = lib().gmlp_check_support(arch.encode() if arch else None, experts, hidden, ffn,
                                  activation_id(activation), rec)
    return st == 0, ("" if st == 0 else last_error()), st


def query_sizes(M, experts, hidden, ffn, activation="swiglu", rec=None, recompute=False):
    rec = rec if rec is not None else recipe()
    s = Sizes()
    _check(lib().gmlp_query_sizes(M, experts, hidden, ffn, activation_id(activation), rec, int(recompute),
                                  ctypes.byref(s)))
    return {"ctx_bytes": s.ctx_bytes, "ws_bytes": s.ws_bytes, "quant_ws_bytes": s.quant_ws_bytes}


def quant_workspace(G, device):
    n = query_sizes(0, G, 128, 128)["quant_ws_bytes"]
    return torch.empty(n, dtype=torch.uint8, device=device)


def read_device_flags(ws):
    v = ctypes.c_uint32(0)
    _check(lib().gmlp_read_device_flags(_p(ws), ctypes.byref(v), _stream(ws.device)))
    return v.value


# ----------------------------------------------------------------------------- quantized tensors
@dataclass
class QTensor:
    """Device buffers of a group-quantized tensor (layouts as in include/gmlp.h)."""
    kind: int
    bufs: dict = field(default_factory=dict)

    def struct(self):
        return GroupedQ(*[_dev_ptr(self.bufs.get(n), n) for n in _Q_FIELDS])


def col_rows_bound(M, G):
    return M + (COL_PAD - 1) * G


def alloc_grouped_q(rec, M, K, G, row=True, col=True, device="cuda"):
    """Buffers for group_quantize of [M, K] into G groups (column-wise sized for the worst padding)."""
    u8 = dict(dtype=torch.uint8, device=device)
    PR = col_rows_bound(M, G)
    b = {}
    if rec.kind == MXFP8:
        if row:
            b["row_data"] = torch.empty(M * K, **u8)
            b["row_scale"] = torch.empty(M * K // 32, **u8)
            b["row_scale_mfma"] = torch.empty(((K + 127) // 128) * M, dtype=torch.int32, device=device)
        if col:
            b["col_data"] = torch.empty(K * PR, **u8)
            b["col_scale"] = torch.empty(K * PR // 32, **u8)
            b["col_scale_mfma"] = torch.empty(K * ((M + 127) // 128 + G), dtype=torch.int32, device=device)
    else:
        if row:
            b["row_data"] = torch.empty(M * K // 2, **u8)
            b["row_scale"] = torch.empty(M * K // 16, **u8)
        if col:
            b["col_data"] = torch.empty(K * PR // 2, **u8)
            b["col_scale"] = torch.empty(K * PR // 16, **u8)
        b["amax_pre"] = torch.empty(G, dtype=torch.float32, device=device)
        b["amax_post"] = torch.empty(G, dtype=torch.float32, device=device)
    return QTensor(rec.kind, b)


def _bits(x):
    """bf16 tensor (or int16 bit view) -> contiguous tensor whose storage is the bf16 bits."""
    if x.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"expected bf16 data, got {x.dtype}")
    return x.contiguous()


def _splits(m_splits, G=None):
    """m_splits as the library reads it: int32 [G] on the device, contiguous."""
    if not isinstance(m_splits, torch.Tensor) or m_splits.dtype != torch.int32 or m_splits.dim() != 1:
        raise TypeError("m_splits: a 1-D int32 tensor is required")
    if G is not None and m_splits.numel() != G:
        raise ValueError(f"m_splits: {G} groups expected, got {m_splits.numel()}")
    return m_splits.contiguous()


def _probs(probs, M):
    """probs as the library reads it: fp32 [M] (read as M consecutive floats)."""
    if M == 0:
        return probs
    if not isinstance(probs, torch.Tensor) or probs.dtype != torch.float32 or probs.numel() != M:
        raise TypeError(f"probs: an fp32 tensor of {M} elements is required")
    return probs.contiguous()


def group_quantize(x, m_splits, rec, want_row=True, want_col=True, out=None, ws=None):
    x = _bits(x)
    m_splits = _splits(m_splits)
    M, K = x.shape
    G = m_splits.numel()
    if out is not None:
        _check_q_sizes(out, _grouped_need(rec, M, K, G, want_row, want_col), "out")
    out = out or alloc_grouped_q(rec, M, K, G, want_row, want_col, x.device)
    ws = ws if ws is not None else quant_workspace(G, x.device)
    q = out.struct()
    _check(lib().gmlp_group_quantize(_p(x), M, K, _p(m_splits), G, rec, int(want_row), int(want_col),
                                     ctypes.byref(q), _p(ws), ws.numel(), _stream(x.device)))
    return out


def group_quantize_noalloc(x, m_splits, rec, want_row=True, want_col=True, out=None):
    """group_quantize with the library's fixed device workspace (no workspace argument; at most
    1024 groups).  out must be given by callers that cannot allocate."""
    x = _bits(x)
    m_splits = _splits(m_splits)
    M, K = x.shape
    G = m_splits.numel()
    if out is not None:
        _check_q_sizes(out, _grouped_need(rec, M, K, G, want_row, want_col), "out")
    out = out or alloc_grouped_q(rec, M, K, G, want_row, want_col, x.device)
    q = out.struct()
    _check(lib().gmlp_group_quantize_noalloc(_p(x), M, K, _p(m_splits), G, rec, int(want_row), int(want_col),
                                             ctypes.byref(q), _stream(x.device)))
    return out


def group_hadamard_amax(x, m_splits, sign_mask, ws=None):
    x = _bits(x)
    m_splits = _splits(m_splits)
    M, K = x.shape
    G = m_splits.numel()
    pre = torch.empty(G, dtype=torch.float32, device=x.device)
    post = torch.empty(G, dtype=torch.float32, device=x.device)
    ws = ws if ws is not None else quant_workspace(G, x.device)
    _check(lib().gmlp_group_hadamard_amax(_p(x), M, K, _p(m_splits), G, int(sign_mask) & 0xFFFF, _p(pre),
                                          _p(post), _p(ws), ws.numel(), _stream(x.device)))
    return pre, post


def group_quantize_with_amax(x, m_splits, rec, amax_pre, amax_post, want_row=True, want_col=True, out=None,
                             ws=None):
    x = _bits(x)
    m_splits = _splits(m_splits)
    M, K = x.shape
    G = m_splits.numel()
    if out is not None:
        _check_q_sizes(out, _grouped_need(rec, M, K, G, want_row, want_col), "out")
    out = out or alloc_grouped_q(rec, M, K, G, want_row, want_col, x.device)
    out.bufs["amax_pre"] = amax_pre
    out.bufs["amax_post"] = amax_post
    ws = ws if ws is not None else quant_workspace(G, x.device)
    q = out.struct()
    _check(lib().gmlp_group_quantize_with_amax(_p(x), M, K, _p(m_splits), G, rec, int(want_row), int(want_col),
                                               ctypes.byref(q), _p(ws), ws.numel(), _stream(x.device)))
    return out


def alloc_weight_q(rec, E, N, K, device="cuda", bf16_panels=True):
    u8 = dict(dtype=torch.uint8, device=device)
    b = {}
    if rec.kind == MXFP8:
        b["row_data"] = torch.empty(E * N * K, **u8)
        b["row_scale"] = torch.empty(E * N * K // 32, **u8)
        b["row_scale_mfma"] = torch.empty(E * ((K + 127) // 128) * N, dtype=torch.int32, device=device)
        b["col_data"] = torch.empty(E * K * N, **u8)
        b["col_scale"] = torch.empty(E * K * N // 32, **u8)
        b["col_scale_mfma"] = torch.empty(E * ((N + 127) // 128) * K, dtype=torch.int32, device=device)
    else:
        b["row_data"] = torch.empty(E * N * K // 2, **u8)
        b["row_scale"] = torch.empty(E * N * K // 16, **u8)
        b["col_data"] = torch.empty(E * K * N // 2, **u8)
        b["col_scale"] = torch.empty(E * K * N // 16, **u8)
        b["amax_pre"] = torch.empty(E, dtype=torch.float32, device=device)
        if bf16_panels:               # the operands the GEMMs read, expanded once here
            b["row_bf16"] = torch.empty(2 * E * N * K, **u8)
            b["col_bf16"] = torch.empty(2 * E * K * N, **u8)
    return QTensor(rec.kind, b)


def _grouped_need(rec, M, K, G, row=True, col=True):
    """Bytes the kernels address in each buffer of a group-quantized [M, K] tensor (layouts of
    include/gmlp.h).  Column-wise buffers hold K x sum P_g elements, P_g = m_g rounded up to 128,
    which depends on the splits on the device: the bound here is the least any splits of M rows
    need (P = M rounded up to 128); alloc_grouped_q sizes them for the most (M + 127 G)."""
    P = (M + COL_PAD - 1) // COL_PAD * COL_PAD
    need = {}
    if rec.kind == MXFP8:
        if row:
            need.update(row_data=M * K, row_scale=M * K // 32, row_scale_mfma=4 * ((K + 127) // 128) * M)
        if col:
            need.update(col_data=K * P, col_scale=K * P // 32, col_scale_mfma=4 * K * P // 128)
    else:
        if row:
            need.update(row_data=M * K // 2, row_scale=M * K // 16, row_bf16=2 * M * K)
        if col:
            need.update(col_data=K * P // 2, col_scale=K * P // 16, col_bf16=2 * K * P)
        need.update(amax_pre=4 * G, amax_post=4 * G)
    return need


def _weight_need(rec, E, N, K):
    """Bytes the kernels address in each buffer of a quantized weight [E, N, K] (alloc_weight_q's
    layout)."""
    return {k: t.numel() * t.element_size() for k, t in alloc_weight_q(rec, E, N, K, "meta").bufs.items()}


def _check_q_sizes(q, need, name):
    """Every buffer q holds must be a contiguous buffer of at least need[buffer] bytes: the kernels
    address the buffers from the call's sizes, not from the buffers.  A buffer q lacks is left to
    the library's null check."""
    if not isinstance(q, QTensor):
        raise TypeError(f"{name}: a QTensor is required")
    for k, n in need.items():
        b = q.bufs.get(k)
        if b is None:
            continue
        have = b.numel() * b.element_size()
        if have < n or not b.is_contiguous():
            raise ValueError(f"{name}.{k}: a contiguous buffer of at least {n} bytes is required, got {have}")


def weight_quantize(w, rec, out=None):
    """w: stacked bf16 [E, N, K] tensor, or a list of E [N, K] tensors (discrete weights)."""
    if isinstance(w, (list, tuple)):
        ws_list = [_bits(t) for t in w]
        E = len(ws_list)
        N, K = ws_list[0].shape
        if any(tuple(t.shape) != (N, K) for t in ws_list):
            raise ValueError(f"w: every expert's weight must have the shape {(N, K)}")
        dev = ws_list[0].device
    else:
        w = _bits(w)
        E, N, K = w.shape
        dev = w.device
    if out is not None:
        _check_q_sizes(out, _weight_need(rec, E, N, K), "out")
    if isinstance(w, (list, tuple)):
        ptrs = (ctypes.c_void_p * E)(*[_dev_ptr(t, f"w[{i}]") for i, t in enumerate(ws_list)])
        base = ctypes.c_void_p(0)
    else:
        ptrs = None
        base = _p(w, "w")
    out = out or alloc_weight_q(rec, E, N, K, dev)
    ws = quant_workspace(1, dev)
    q = out.struct()
    _check(lib().gmlp_weight_quantize(base, ptrs, E, N, K, rec, ctypes.byref(q), _p(ws), ws.numel(),
                                      _stream(dev)))
    return out


def grouped_gemm_ws_bytes(layout, rec, G, M, n, k):
    v = ctypes.c_size_t(0)
    _check(lib().gmlp_grouped_gemm_ws_bytes(layout, rec, G, M, n, k, ctypes.byref(v)))
    return v.value


def _check_out(t, shape, dtype, name):
    if t is None or tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name}: an existing contiguous {dtype} tensor of shape {tuple(shape)} is required")


def grouped_gemm(layout, rec, a, b, m_splits, M, n, k, out_dtype=OUT_BF16, ws=None, out=None):
    """out: the output tensor (required for OUT_FP32_ACCUMULATE, whose product is added to it)."""
    m_splits = _splits(m_splits)
    G = m_splits.numel()
    dev = m_splits.device
    dt = torch.bfloat16 if out_dtype == OUT_BF16 else torch.float32
    shape = (G, n, k) if layout == GEMM_WGRAD else (M, n)
    if out is not None or out_dtype == OUT_FP32_ACCUMULATE:
        _check_out(out, shape, dt, "grouped_gemm out")
        c = out
    else:
        c = torch.empty(shape, dtype=dt, device=dev)
    if layout == GEMM_WGRAD:
        _check_q_sizes(a, _grouped_need(rec, M, n, G, row=False), "a")
        _check_q_sizes(b, _grouped_need(rec, M, k, G, row=False), "b")
    else:
        _check_q_sizes(a, _grouped_need(rec, M, k, G, col=False), "a")
        wn, wk = (n, k) if layout == GEMM_FPROP else (k, n)      # the weight's [N, K]
        _check_q_sizes(b, _weight_need(rec, G, wn, wk), "b")
    if ws is None:
        ws = torch.empty(grouped_gemm_ws_bytes(layout, rec, G, M, n, k), dtype=torch.uint8, device=dev)
    qa, qb = a.struct(), b.struct()
    _check(lib().gmlp_grouped_gemm(layout, rec, ctypes.byref(qa), ctypes.byref(qb), _p(m_splits), G, M, n, k,
                                   _p(c), out_dtype, _p(ws), ws.numel(), _stream(dev)))
    return c


# ----------------------------------------------------------------------------- fused MLP
@dataclass
class MlpContext:
    """What the forward leaves for the backward (opaque buffer + the call's settings)."""
    buf: torch.Tensor
    M: int
    E: int
    H: int
    ffn: int
    activation: int
    rec: Recipe
    recompute: bool
    input_requires_grad: bool
    weight_requires_grad: bool
    clamp: float = 0.0             # tanh clamp scale (tanh-clamped squared ReLU)


def grouped_mlp_forward(x, m_splits, w1q, w2q, probs, activation, rec, recompute=False,
                        input_requires_grad=True, weight_requires_grad=True, ws=None, y=None, ctx=None,
                        fc2_amax_in_fc1=False):
    """activation: as activation_spec.  fc2_amax_in_fc1 (NVFP4, squared-ReLU activations): take the
    fc2 input's amax in the fc1 GEMM's epilogue instead of a pass over h (the same values)."""
    x = _bits(x)
    M, H = x.shape
    m_splits = _splits(m_splits)
    probs = _probs(probs, M)
    E = m_splits.numel()
    act, clamp = activation_spec(activation)
    ffn = ffn_from_w2(w2q, rec, E, H)
    F1 = 2 * ffn if is_glu(act) else ffn
    _check_q_sizes(w1q, _weight_need(rec, E, F1, H), "w1q")
    _check_q_sizes(w2q, _weight_need(rec, E, H, ffn), "w2q")
    sizes = query_sizes(M, E, H, ffn, act, rec, recompute)
    dev = x.device
    ws = ws if ws is not None else torch.empty(sizes["ws_bytes"], dtype=torch.uint8, device=dev)
    cbuf = ctx.buf if ctx is not None else torch.empty(sizes["ctx_bytes"], dtype=torch.uint8, device=dev)
    if y is not None:
        _check_out(y, (M, H), torch.bfloat16, "y")
    else:
        y = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    s1, s2 = w1q.struct(), w2q.struct()
    a = FwdArgs(_dev_ptr(x, "x"), _dev_ptr(m_splits, "m_splits"), M, E, H, ffn, ctypes.pointer(s1),
                ctypes.pointer(s2), _dev_ptr(probs, "probs") if M else None, act, rec, int(recompute), int(input_requires_grad),
                int(weight_requires_grad), _dev_ptr(y, "y") if M else None, _dev_ptr(cbuf, "ctx"), cbuf.numel(),
                _dev_ptr(ws, "ws"), ws.numel(), int(bool(fc2_amax_in_fc1)), clamp)
    _check(lib().gmlp_grouped_mlp_forward(ctypes.byref(a), _stream(dev)))
    c = MlpContext(cbuf, M, E, H, ffn, act, rec, bool(recompute), bool(input_requires_grad),
                   bool(weight_requires_grad), clamp)
    return y, c


def forward_saved(ctx):
    """Views into a forward's context: h [M, F1] bf16 and (NVFP4) the fc2 input's per-group pre- and
    post-RHT amax (fp32 [E]; None for MXFP8)."""
    a = FwdArgs()
    a.M, a.E, a.H, a.ffn, a.activation, a.recipe = ctx.M, ctx.E, ctx.H, ctx.ffn, ctx.activation, ctx.rec
    a.recompute, a.ctx, a.ctx_bytes = int(ctx.recompute), _dev_ptr(ctx.buf, "ctx"), ctx.buf.numel()
    h, pre, post = ctypes.c_void_p(), ctypes.c_void_p(), ctypes.c_void_p()
    _check(lib().gmlp_forward_saved(ctypes.byref(a), ctypes.byref(h), ctypes.byref(pre), ctypes.byref(post)))
    base = ctx.buf.data_ptr()
    F1 = 2 * ctx.ffn if is_glu(ctx.activation) else ctx.ffn

    def view(ptr, n, dtype):
        if not ptr.value:
            return None
        off = ptr.value - base
        nbytes = n * torch.tensor([], dtype=dtype).element_size()
        return ctx.buf[off:off + nbytes].view(dtype)

    hv = view(h, ctx.M * F1, torch.bfloat16)
    return (hv.view(ctx.M, F1) if hv is not None else None, view(pre, ctx.E, torch.float32),
            view(post, ctx.E, torch.float32))


def grouped_mlp_backward(dy, m_splits, w1q, w2q, probs, ctx, wgrad_dtype=OUT_BF16, ws=None, out=None,
                         defer_wgrad=False):
    """out: optional {"dx", "dprobs", "dw1", "dw2"} tensors to write; with wgrad_dtype
    OUT_FP32_ACCUMULATE, "dw1" and "dw2" are required: the fp32 main_grads the weight
    gradients are added to.  defer_wgrad: dw1 and dw2 are left to grouped_mlp_wgrad, which
    takes the returned "deferred" handle (it holds the workspace with the cast operands)."""
    dy = _bits(dy)
    M, H = dy.shape
    E, ffn, act = ctx.E, ctx.ffn, ctx.activation
    m_splits = _splits(m_splits, E)
    probs = _probs(probs, M)
    F1 = 2 * ffn if is_glu(act) else ffn
    dev = dy.device
    sizes = query_sizes(M, E, H, ffn, act, ctx.rec, ctx.recompute)
    ws = ws if ws is not None else torch.empty(sizes["ws_bytes"], dtype=torch.uint8, device=dev)
    wdt = torch.bfloat16 if wgrad_dtype == OUT_BF16 else torch.float32
    o = out or {}

    def given_or_new(name, shape, dtype):
        t = o.get(name)
        if t is None:
            return torch.empty(shape, dtype=dtype, device=dev)
        _check_out(t, shape, dtype, name)
        return t

    dx = given_or_new("dx", (M, H), torch.bfloat16) if ctx.input_requires_grad else None
    dprobs = given_or_new("dprobs", (M,), torch.float32)
    dw1 = dw2 = None
    if ctx.weight_requires_grad and not defer_wgrad:
        if wgrad_dtype == OUT_FP32_ACCUMULATE:
            dw1, dw2 = o.get("dw1"), o.get("dw2")
            _check_out(dw1, (E, F1, H), wdt, "dw1 main_grad")
            _check_out(dw2, (E, H, ffn), wdt, "dw2 main_grad")
        else:
            dw1 = given_or_new("dw1", (E, F1, H), wdt)
            dw2 = given_or_new("dw2", (E, H, ffn), wdt)
    _check_q_sizes(w1q, _weight_need(ctx.rec, E, F1, H), "w1q")
    _check_q_sizes(w2q, _weight_need(ctx.rec, E, H, ffn), "w2q")
    s1, s2 = w1q.struct(), w2q.struct()
    a = BwdArgs(_dev_ptr(dy, "dy"), _dev_ptr(m_splits, "m_splits"), M, E, H, ffn, ctypes.pointer(s1),
                ctypes.pointer(s2), _dev_ptr(probs, "probs") if M else None, act, ctx.rec, int(ctx.recompute), int(ctx.input_requires_grad),
                int(ctx.weight_requires_grad), _dev_ptr(dx, "dx") if M else None,
                _dev_ptr(dprobs, "dprobs") if M else None, _dev_ptr(dw1, "dw1"), _dev_ptr(dw2, "dw2"),
                wgrad_dtype, _dev_ptr(ctx.buf, "ctx"), ctx.buf.numel(), _dev_ptr(ws, "ws"), ws.numel(), int(bool(defer_wgrad)), ctx.clamp)
    _check(lib().gmlp_grouped_mlp_backward(ctypes.byref(a), _stream(dev)))
    res = {"dx": dx, "dprobs": dprobs, "dw1": dw1, "dw2": dw2}
    if defer_wgrad and ctx.weight_requires_grad:
        res["deferred"] = DeferredWgrad(m_splits, ctx, ws)
    return res


@dataclass
class DeferredWgrad:
    """What a deferring backward leaves for grouped_mlp_wgrad: the splits, the forward's context
    and the workspace holding the cast weight-gradient operands (keep both untouched)."""
    m_splits: torch.Tensor
    ctx: MlpContext
    ws: torch.Tensor


def grouped_mlp_wgrad(deferred, wgrad_dtype=OUT_BF16, out=None):
    """The weight gradients of a backward called with defer_wgrad; out as in grouped_mlp_backward
    ("dw1", "dw2")."""
    ctx, ws = deferred.ctx, deferred.ws
    E, H, ffn, act = ctx.E, ctx.H, ctx.ffn, ctx.activation
    F1 = 2 * ffn if is_glu(act) else ffn
    dev = ws.device
    wdt = torch.bfloat16 if wgrad_dtype == OUT_BF16 else torch.float32
    o = out or {}
    if wgrad_dtype == OUT_FP32_ACCUMULATE:
        dw1, dw2 = o.get("dw1"), o.get("dw2")
        _check_out(dw1, (E, F1, H), wdt, "dw1 main_grad")
        _check_out(dw2, (E, H, ffn), wdt, "dw2 main_grad")
    else:
        dw1, dw2 = o.get("dw1"), o.get("dw2")
        if dw1 is not None:
            _check_out(dw1, (E, F1, H), wdt, "dw1")
        else:
            dw1 = torch.empty((E, F1, H), dtype=wdt, device=dev)
        if dw2 is not None:
            _check_out(dw2, (E, H, ffn), wdt, "dw2")
        else:
            dw2 = torch.empty((E, H, ffn), dtype=wdt, device=dev)
    a = BwdArgs()
    a.m_splits, a.M, a.E, a.H, a.ffn = _dev_ptr(deferred.m_splits, "m_splits"), ctx.M, E, H, ffn
    a.activation, a.recipe, a.recompute, a.tanh_clamp_scale = act, ctx.rec, int(ctx.recompute), ctx.clamp
    a.input_requires_grad, a.weight_requires_grad = int(ctx.input_requires_grad), 1
    a.dw1, a.dw2, a.wgrad_dtype = _dev_ptr(dw1, "dw1"), _dev_ptr(dw2, "dw2"), wgrad_dtype
    a.ctx, a.ctx_bytes, a.ws, a.ws_bytes = _dev_ptr(ctx.buf, "ctx"), ctx.buf.numel(), _dev_ptr(ws, "ws"), ws.numel()
    _check(lib().gmlp_grouped_mlp_wgrad(ctypes.byref(a), _stream(dev)))
    return {"dw1": dw1, "dw2": dw2}


def ffn_from_w2(w2q, rec, E, H):
    n = w2q.bufs["row_data"].numel()
    return (n // (E * H)) if rec.kind == MXFP8 else (2 * n // (E * H))


# ----------------------------------------------------------------------------- torch autograd
class GroupedMLPFunction(torch.autograd.Function):
    """torch.autograd over grouped_mlp_forward / grouped_mlp_backward, so that the fused MLP sits
    in a training step like the pages' fused op ("GEMM + Swiglu fused Grouped MLP for MXFP8",
    sequence diagram: one forward call that saves its context, one backward call).

    Inputs: x [M, H] bf16, probs [M] fp32, w1 [E, F1, H] and w2 [E, H, ffn] bf16 (the parameters
    the weight gradients flow to), m_splits [E] int32 on the device, w1q / w2q the weights'
    quantized forms (weight_quantize of w1 and w2, made by the caller once per weight update),
    then activation, recipe and recompute as in grouped_mlp_forward.  The backward computes dx
    only when x requires grad and dw1, dw2 (bf16) only when w1 or w2 does; dprobs always.
    accumulate_main_grad: the weight gradients are added in fp32 to w1.main_grad and w2.main_grad
    (fp32 tensors of the weights' shapes, as in the pages' main_grad accumulation: review comments
    on overwrite_main_grad) and autograd receives no gradient for w1 and w2."""

    @staticmethod
    def forward(fctx, x, probs, w1, w2, m_splits, w1q, w2q, activation, rec, recompute=False,
                accumulate_main_grad=False):
        need = fctx.needs_input_grad
        fctx.main_grads = (w1.main_grad, w2.main_grad) if accumulate_main_grad else None
        y, c = grouped_mlp_forward(x, m_splits, w1q, w2q, probs.contiguous(), activation, rec,
                                   recompute=recompute, input_requires_grad=need[0],
                                   weight_requires_grad=need[2] or need[3])
        fctx.mlp = (c, w1q, w2q)
        fctx.save_for_backward(probs, m_splits)
        return y

    @staticmethod
    def backward(fctx, dy):
        probs, m_splits = fctx.saved_tensors
        c, w1q, w2q = fctx.mlp
        need = fctx.needs_input_grad
        acc = fctx.main_grads is not None and c.weight_requires_grad
        kw = {"wgrad_dtype": OUT_FP32_ACCUMULATE,
              "out": {"dw1": fctx.main_grads[0], "dw2": fctx.main_grads[1]}} if acc else {}
        r = grouped_mlp_backward(dy.to(torch.bfloat16).contiguous(), m_splits, w1q, w2q, probs.contiguous(), c,
                                 **kw)
        return (r["dx"] if need[0] else None, r["dprobs"] if need[1] else None,
                r["dw1"] if need[2] and not acc else None, r["dw2"] if need[3] and not acc else None,
                None, None, None, None, None, None, None)


def grouped_mlp(x, probs, w1, w2, m_splits, activation, rec, w1q=None, w2q=None, recompute=False,
                accumulate_main_grad=False):
    """y = the fused grouped MLP of x, differentiable in x, probs, w1 and w2 (GroupedMLPFunction).
    w1q / w2q default to weight_quantize(w1 / w2, rec) made in this call."""
    if accumulate_main_grad:
        for w, name in ((w1, "w1"), (w2, "w2")):
            mg = getattr(w, "main_grad", None)
            _check_out(mg, tuple(w.shape), torch.float32, f"{name}.main_grad")
    w1q = w1q if w1q is not None else weight_quantize(w1.detach(), rec)
    w2q = w2q if w2q is not None else weight_quantize(w2.detach(), rec)
    return GroupedMLPFunction.apply(x, probs, w1, w2, m_splits, w1q, w2q, activation, rec, recompute,
                                    accumulate_main_grad)
