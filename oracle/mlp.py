"""Grouped GEMMs and the unfused forward / backward of the grouped MLP.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
* "GEMM + Swiglu fused Grouped MLP for MXFP8" -- sequence diagram: forward
  FC1 GLU kernel (x and fc1 weight in MXFP8, prob, bf16 pre-activation
  ``c_tensor``, MXFP8 activation row + column) then the fc2 GEMM; backward
  FC2 dGLU kernel (dy in MXFP8, saved pre-activation, fc2 weight column-wise ->
  fc1 grad in MXFP8 and ``dprob``), FC1 dgrad, and both wgrads as grouped GEMMs.
* "Reduce NVFP4 quantization work for the fused GroupedMLP fc2 input ..." --
  Description and commits: the SReLU path, the accumulator rounded through the
  C dtype (bf16) before the activation, the fc2 input re-built in backward.
* The MLP statement: GroupedLinear (fc1) + SwiGLU or squared ReLU scaled by the
  router probability + GroupedLinear (fc2) over per-expert token splits.

The fused path reaches exactly the result of this unfused per-expert sequence:
quantize -> GEMM -> bf16 -> activation * prob -> bf16 -> quantize -> GEMM.
Activation recompute regenerates the same bf16 activation, so it has no
separate definition here.

Readings (the pages are silent on these):
* Linear weights are stored [out, in]: W1 [E, F1, H], W2 [E, H, ffn].
* SwiGLU: h = [gate | up] along F1 = 2 * ffn; a = silu(gate) * up * p.
  SReLU: F1 = ffn; a = max(h, 0)^2 * p.  p multiplies after the activation,
  before the bf16 rounding.
* The tanh-clamped SReLU ("Reduce NVFP4 quantization work ...", Changes and
  commits: ScaledTanhSReLU, its soft clamp and tanh_clamp_scale; no formula on
  the pages): F1 = ffn; a = c * tanh(max(h, 0)^2 / c) * p with c the clamp
  scale, i.e. the squared ReLU softly clamped to (0, c).  Written
  ("tanh_srelu", c).
* QGeGLU ("Add NVTE_CUTEDSL_FUSED_GROUPED_MLP_WARN_FALLBACK ...", review: named
  only): the GLU with the quick-GELU gate, h = [gate | up], a = gate *
  sigmoid(1.702 gate) * up * p (the sigmoid approximation of GELU, Hendrycks and
  Gimpel, "Gaussian Error Linear Units", section 2).
* h, a, y, da, dh, dx and the weight gradients are bf16 (round to nearest
  even); dprob is fp32.  Activations are evaluated in fp64 from bf16 h.
* Backward operands: dy row-wise (blocks along H) times W2 quantized along H
  (da); dh row-wise (blocks along F1) times W1 quantized along F1 (dx); the
  wgrads contract over tokens with both operands column-wise.  For NVFP4 the
  column-wise (wgrad) operands carry the RHT with one recipe-wide mask (the
  same orthogonal transform on both, so it cancels in the product); weights
  never get the RHT.
* NVFP4 global scales: per group from the pre-RHT amax for row-wise casts and
  the post-RHT amax for column-wise casts; per expert (amax of the whole
  weight matrix) for weights.
* Empty experts contribute no rows and a zero weight gradient.
* A weight gradient accumulated into an fp32 main_grad is the exact gradient
  added to the stored fp32 value, rounded once to fp32 (no bf16 step).
"""
import numpy as np

from .formats import bf16_bits_to_f64, f32, f64_to_bf16_bits, round_bf16
from .formats import pack_fp4
from .quant import (mxfp8_dequant_rows, mxfp8_group_quantize, mxfp8_quantize_rows,
                    nvfp4_dequant_packed, nvfp4_dequant_rows, nvfp4_group_quantize_with_amax,
                    nvfp4_quantize_rows, padded)
from .rht import group_hadamard_amax

SWIGLU = "swiglu"
SRELU = "srelu"
TANH_SRELU = "tanh_srelu"
QGEGLU = "qgeglu"
QUICK_GELU_K = 1.702
MXFP8 = "mxfp8"
NVFP4 = "nvfp4"


def act_kind(activation):
    """(name, clamp scale or None): an activation is a name or ("tanh_srelu", c)."""
    if isinstance(activation, tuple):
        name, c = activation
        return name, float(c)
    return activation, None


def is_glu(activation):
    """The gated activations read h = [gate | up]."""
    return act_kind(activation)[0] in (SWIGLU, QGEGLU)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _gate(g, kind):
    """The gate's value g s(k g) and its derivative s (1 + k g (1 - s)) (k = 1 for SwiGLU)."""
    k = QUICK_GELU_K if kind == QGEGLU else 1.0
    s = _sigmoid(k * g)
    return g * s, s * (1.0 + k * g * (1.0 - s))


def act_forward(h, activation):
    """Activation value without the prob, from bf16 h (fp64)."""
    kind, c = act_kind(activation)
    if kind in (SWIGLU, QGEGLU):
        f = h.shape[1] // 2
        g, u = h[:, :f], h[:, f:]
        return _gate(g, kind)[0] * u
    r = np.maximum(h, 0.0)
    if kind == TANH_SRELU:
        return c * np.tanh(r * r / c)
    assert kind == SRELU, kind
    return r * r


def act_backward(h, da, p, activation):
    """(dh, dprob) for a = act(h) * p given da = dL/da; dh unrounded fp64, dprob fp64."""
    kind, c = act_kind(activation)
    if kind in (SWIGLU, QGEGLU):
        f = h.shape[1] // 2
        g, u = h[:, :f], h[:, f:]
        gs, dgs = _gate(g, kind)
        dgate = da * p[:, None] * u * dgs
        dup = da * p[:, None] * gs
        dprob = np.sum(da * gs * u, axis=1)
        return np.concatenate([dgate, dup], axis=1), dprob
    r = np.maximum(h, 0.0)
    if kind == TANH_SRELU:
        t = np.tanh(r * r / c)
        dh = da * p[:, None] * (1.0 - t * t) * 2.0 * r
        dprob = np.sum(da * c * t, axis=1)
        return dh, dprob
    dh = da * p[:, None] * 2.0 * r
    dprob = np.sum(da * r * r, axis=1)
    return dh, dprob


# ----------------------------------------------------------------------------- GEMM
def grouped_gemm_nt(a_groups, b_groups):
    """C_g = A_g @ B_g^T in fp64 for every group (A_g [m, K], B_g [n, K])."""
    return [a @ b.T for a, b in zip(a_groups, b_groups)]


def _split_rows(t, m_splits):
    out, off = [], 0
    for m in m_splits:
        out.append(t[off:off + m])
        off += m
    return out


# ----------------------------------------------------------------------------- operands
class Recipe:
    def __init__(self, kind, sign_mask=0):
        assert kind in (MXFP8, NVFP4)
        self.kind = kind
        self.sign_mask = int(sign_mask) & 0xFFFF


def quantize_activation(x_bits, m_splits, recipe, row=True, col=True, amax=None):
    """Group-quantize an activation-like tensor; returns (quantized dict, dequantized views).

    Dequantized views: ``row`` [M, K] fp64 and ``col`` = per-group [K, P_g] fp64.
    For NVFP4 the per-group (pre, post) amax is computed here unless given.
    """
    deq = {}
    if recipe.kind == MXFP8:
        q = mxfp8_group_quantize(x_bits, m_splits, row=row, col=col)
        if row:
            deq["row"] = mxfp8_dequant_rows(q["row_data"], q["row_scale"])
        if col:
            deq["col"] = [mxfp8_dequant_rows(d, s) for d, s in q["col_groups"]]
        return q, deq
    if amax is None:
        amax = group_hadamard_amax(x_bits, m_splits, recipe.sign_mask)
    pre, post = amax
    q = nvfp4_group_quantize_with_amax(x_bits, m_splits, pre, post, recipe.sign_mask,
                                       row=row, col=col, rht=True)
    q["amax_pre"], q["amax_post"] = pre, post
    if row:
        rows = []
        for g, xg in enumerate(_split_rows(np.arange(x_bits.shape[0]), m_splits)):
            if len(xg):
                rows.append(nvfp4_dequant_packed(q["row_data"][xg], q["row_scale"][xg], pre[g]))
        deq["row"] = np.concatenate(rows) if rows else np.zeros((0, x_bits.shape[1]))
    if col:
        deq["col"] = [nvfp4_dequant_packed(d, s, post[g]) for g, (d, s) in enumerate(q["col_groups"])]
    return q, deq


def quantize_weight(w_bits, recipe):
    """Quantize stacked weights [E, N, K] for fprop (blocks along K) and dgrad (blocks along N).

    The dgrad operand is each expert's W_e^T [K, N] cast row-wise, i.e. with blocks along N.
    Returns (quantized dict, dequantized dict) with ``row`` = [E, N, K] and ``colT`` = [E, K, N].
    """
    e, n, k = w_bits.shape
    w = bf16_bits_to_f64(w_bits.reshape(e * n, k)).reshape(e, n, k)
    q = {"row": [], "colT": []}
    row, colT = [], []
    if recipe.kind == MXFP8:
        for i in range(e):
            qr, sr = mxfp8_quantize_rows(w[i])
            qc, sc = mxfp8_quantize_rows(np.ascontiguousarray(w[i].T))
            q["row"].append((qr, sr))
            q["colT"].append((qc, sc))
            row.append(mxfp8_dequant_rows(qr, sr))
            colT.append(mxfp8_dequant_rows(qc, sc))
    else:
        q["amax"] = np.array([np.max(np.abs(w[i])) if w[i].size else 0.0 for i in range(e)], dtype=np.float32)
        for i in range(e):
            cr, sr = nvfp4_quantize_rows(w[i], q["amax"][i])
            cc, sc = nvfp4_quantize_rows(np.ascontiguousarray(w[i].T), q["amax"][i])
            q["row"].append((pack_fp4(cr), sr))
            q["colT"].append((pack_fp4(cc), sc))
            row.append(nvfp4_dequant_rows(cr, sr, q["amax"][i]))
            colT.append(nvfp4_dequant_rows(cc, sc, q["amax"][i]))
    stack = lambda a, shape: np.stack(a) if a else np.zeros(shape)
    return q, {"row": stack(row, (0, n, k)), "colT": stack(colT, (0, k, n))}


# ----------------------------------------------------------------------------- forward
def forward(x_bits, m_splits, w1_bits, w2_bits, probs, activation, recipe, wq1=None, wq2=None):
    """Unfused grouped MLP forward.  Returns a dict of every intermediate.

    y = bf16( Q(a) . Q(W2)^T ),  a = bf16( act(h) * p ),  h = bf16( Q(x) . Q(W1)^T ).
    """
    m_splits = [int(m) for m in m_splits]
    p = np.asarray(probs, dtype=np.float32).astype(np.float64)
    if wq1 is None:
        wq1 = quantize_weight(w1_bits, recipe)
    if wq2 is None:
        wq2 = quantize_weight(w2_bits, recipe)
    xq, xd = quantize_activation(x_bits, m_splits, recipe, row=True, col=True)
    h_groups = grouped_gemm_nt(_split_rows(xd["row"], m_splits), list(wq1[1]["row"]))
    h = round_bf16(np.concatenate(h_groups)) if h_groups else np.zeros((0, w1_bits.shape[1]))
    a = round_bf16(act_forward(h, activation) * p[:, None])
    a_bits = f64_to_bf16_bits(a)
    aq, ad = quantize_activation(a_bits, m_splits, recipe, row=True, col=True)
    y_groups = grouped_gemm_nt(_split_rows(ad["row"], m_splits), list(wq2[1]["row"]))
    y = np.concatenate(y_groups) if y_groups else np.zeros((0, w2_bits.shape[1]))
    return {
        "m_splits": m_splits, "activation": activation, "recipe": recipe, "probs": p,
        "xq": xq, "xd": xd, "wq1": wq1, "wq2": wq2,
        "h_f64": np.concatenate(h_groups) if h_groups else h, "h": h, "h_bits": f64_to_bf16_bits(h),
        "a": a, "a_bits": a_bits, "aq": aq, "ad": ad,
        "y_f64": y, "y_bits": f64_to_bf16_bits(y),
    }


# ----------------------------------------------------------------------------- backward
def backward(fwd, dy_bits):
    """Unfused grouped MLP backward from the forward's intermediates.

    da = bf16( Q_row(dy) . Q(W2 along H) ),  (dh, dprob) = act'(h, da, p) with dh -> bf16,
    dx = bf16( Q_row(dh) . Q(W1 along F1) ),
    dW2_g = bf16( Q_col(dy_g)^T . Q_col(a_g) ),  dW1_g = bf16( Q_col(dh_g)^T . Q_col(x_g) ).
    """
    m_splits, recipe, act = fwd["m_splits"], fwd["recipe"], fwd["activation"]
    p = fwd["probs"]
    e = len(m_splits)
    dyq, dyd = quantize_activation(dy_bits, m_splits, recipe, row=True, col=True)
    da_groups = grouped_gemm_nt(_split_rows(dyd["row"], m_splits), list(fwd["wq2"][1]["colT"]))
    da = round_bf16(np.concatenate(da_groups))
    dh_raw, dprob = act_backward(fwd["h"], da, p, act)
    dh = round_bf16(dh_raw)
    dh_bits = f64_to_bf16_bits(dh)
    dhq, dhd = quantize_activation(dh_bits, m_splits, recipe, row=True, col=True)
    dx_groups = grouped_gemm_nt(_split_rows(dhd["row"], m_splits), list(fwd["wq1"][1]["colT"]))
    dx = np.concatenate(dx_groups)
    n_h, n_f = dy_bits.shape[1], fwd["a"].shape[1]
    n_f1 = dh.shape[1]
    dw2 = np.zeros((e, n_h, n_f))
    dw1 = np.zeros((e, n_f1, n_h))
    for g in range(e):
        if m_splits[g] == 0:
            continue
        dw2[g] = dyd["col"][g] @ fwd["ad"]["col"][g].T
        dw1[g] = dhd["col"][g] @ fwd["xd"]["col"][g].T
    return {
        "dyq": dyq, "dyd": dyd, "da_f64": np.concatenate(da_groups), "da": da,
        "dh": dh, "dh_bits": dh_bits, "dhq": dhq, "dhd": dhd,
        "dprob": dprob.astype(np.float32),
        "dx_f64": dx, "dx_bits": f64_to_bf16_bits(dx),
        "dw1_f64": dw1, "dw1_bits": f64_to_bf16_bits(dw1),
        "dw2_f64": dw2, "dw2_bits": f64_to_bf16_bits(dw2),
    }


def accumulate_main_grad(main_grad, dw):
    """fp32 main_grad after the weight gradient is added to it: fp32(main_grad + dW).

    "GEMM + Swiglu fused Grouped MLP for MXFP8", review comments on overwrite_main_grad: the
    grouped wgrad either overwrites the parameter's fp32 main_grad or accumulates into it.
    main_grad holds fp32 values; dw is the fp64 gradient (``dw1_f64`` / ``dw2_f64``).  The sum
    is formed in fp64 and rounded once to fp32; for an fp32-representable dw that is exactly
    IEEE fp32 addition (53 >= 2 * 24 + 2).  An empty expert's zero gradient leaves it as it is.
    """
    return f32(np.asarray(main_grad, dtype=np.float64) + np.asarray(dw, dtype=np.float64))


# ----------------------------------------------------------------------------- sampled evaluation (MXFP8)
# For MXFP8 every forward step and the dgrad chain are row-local: the row-wise cast blocks run
# along a row, the GEMMs produce a row from that row, the activation and its derivative act
# elementwise.  Rows of the full computation can therefore be evaluated on their own, which
# lets full-size runs be checked on sampled rows.  A weight-gradient entry contracts one
# feature column of each operand over the group's tokens (column-wise blocks of 32 tokens,
# zero padded to P_g), so it needs those two columns over all of the group's rows.

def _mx_rows(v):
    q, s = mxfp8_quantize_rows(v)
    return mxfp8_dequant_rows(q, s)


def mxfp8_rows(x_bits, dy_bits, p, wd1, wd2, activation):
    """Rows of one expert's MXFP8 forward + backward, exactly as ``forward`` / ``backward``
    compute them.  ``wd1`` / ``wd2`` are that expert's dequantized weights
    {"row": [N, K], "colT": [K, N]} (from ``quantize_weight``).  Returns h, a, y (fp64, before
    its bf16 rounding), da, dh, dprob, dx (fp64, before its bf16 rounding)."""
    p = np.asarray(p, dtype=np.float32).astype(np.float64)
    xd = _mx_rows(bf16_bits_to_f64(x_bits))
    h = round_bf16(xd @ wd1["row"].T)
    a = round_bf16(act_forward(h, activation) * p[:, None])
    y = _mx_rows(a) @ wd2["row"].T
    da = round_bf16(_mx_rows(bf16_bits_to_f64(dy_bits)) @ wd2["colT"].T)
    dh_raw, dprob = act_backward(h, da, p, activation)
    dh = round_bf16(dh_raw)
    dx = _mx_rows(dh) @ wd1["colT"].T
    return {"h": h, "a": a, "y_f64": y, "da": da, "dh": dh, "dprob": dprob, "dx_f64": dx}


def _mx_col(v):
    """Column-wise MXFP8 cast of one feature over a group's tokens, dequantized (length m)."""
    m = v.shape[0]
    t = np.zeros((1, padded(m)))
    t[0, :m] = v
    return _mx_rows(t)[0, :m]


def mxfp8_wgrad_entries(x_bits, dy_bits, p, wd1, wd2, activation, dw1_idx, dw2_idx):
    """Entries (f1, k) of dW1_g = Q_col(dh_g)^T Q_col(x_g) and (n, f) of dW2_g = Q_col(dy_g)^T
    Q_col(a_g) for one expert whose rows are ``x_bits`` / ``dy_bits`` (all of the group's
    rows), fp64 before the bf16 rounding."""
    p = np.asarray(p, dtype=np.float32).astype(np.float64)
    x = bf16_bits_to_f64(x_bits)
    dy = bf16_bits_to_f64(dy_bits)
    xd, dyd = _mx_rows(x), _mx_rows(dy)
    ffn = wd2["row"].shape[1]
    glu = is_glu(activation)

    def h_cols(j):
        cols = [j, ffn + j] if glu else [j]
        return round_bf16(xd @ wd1["row"][cols].T)                       # [m, 1 or 2]

    def a_col(f):
        return round_bf16(act_forward(h_cols(f), activation)[:, 0] * p)

    def dh_col(f1):
        j = f1 % ffn if glu else f1
        da = round_bf16(dyd @ wd2["colT"][j])
        dh, _ = act_backward(h_cols(j), da[:, None], p, activation)
        return round_bf16(dh[:, 1 if (glu and f1 >= ffn) else 0])

    dw1 = np.array([_mx_col(dh_col(f1)) @ _mx_col(x[:, k]) for f1, k in dw1_idx])
    dw2 = np.array([_mx_col(dy[:, n]) @ _mx_col(a_col(f)) for n, f in dw2_idx])
    return dw1, dw2


def reference_mlp_f64(x, m_splits, w1, w2, probs, activation):
    """Unquantized fp64 grouped MLP forward (no rounding anywhere), for format-error sanity checks."""
    out, off = [], 0
    for g, m in enumerate(m_splits):
        xg = x[off:off + m]
        h = xg @ w1[g].T
        a = act_forward(h, activation) * probs[off:off + m, None]
        out.append(a @ w2[g].T)
        off += m
    return np.concatenate(out)


def rel_fro(a, b):
    """Relative Frobenius error ||a - b|| / ||b||."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb else float(np.linalg.norm(a - b))


__all__ = ["forward", "backward", "grouped_gemm_nt", "quantize_activation", "quantize_weight",
           "mxfp8_rows", "mxfp8_wgrad_entries",
           "act_forward", "act_backward", "Recipe", "reference_mlp_f64", "rel_fro",
           "SWIGLU", "SRELU", "TANH_SRELU", "QGEGLU", "MXFP8", "NVFP4", "padded", "mxfp8_quantize_rows",
           "act_kind", "is_glu"]
