"""Seeded synthetic inputs for the fused MoE grouped MLP.

This module only draws random numbers and shapes them; it holds none of the
method's arithmetic.  Both the HIP library's tests and the CPU oracle take their
inputs from here (and only from here).

Every tensor is drawn in numpy from child streams of ``SeedSequence(seed)``,
spawned in the fixed order [splits, x, w1, w2, probs, dy, sign_mask]; weights
take one further child stream per expert, so one expert's weights can be drawn
alone.  Values are drawn in fp32 and converted to bf16 by torch's
round-to-nearest-even cast; the same bf16 bit patterns (numpy uint16) go to
both sides.
"""
from dataclasses import dataclass, field

import numpy as np
import torch

SWIGLU = "swiglu"
SRELU = "srelu"
TANH_SRELU = "tanh_srelu"
QGEGLU = "qgeglu"
MXFP8 = "mxfp8"
NVFP4 = "nvfp4"

STREAMS = ("splits", "x", "w1", "w2", "probs", "dy", "sign_mask")


def to_bf16_bits(a):
    """fp32 numpy array -> bf16 bit patterns (uint16), torch's RNE cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


@dataclass
class Config:
    name: str
    experts: int
    hidden: int
    ffn: int
    activation: object               # a name, or ("tanh_srelu", clamp scale)
    recipe: str
    rows: int
    splits: str                      # "fixed" | "uniform" | "equal" | "zipf" | "dirichlet"
    fixed_splits: tuple = ()
    tokens: int = 0
    topk: int = 0
    x_std: float = 1.0
    w1_std: float = 0.02
    w2_std: float = 0.02
    probs: str = "uniform"           # "uniform" | "softmax_topk" | "normalized_topk"
    backward: bool = True
    stacked: bool = False
    zipf_s: float = 1.2
    zipf_zero: int = 0
    dirichlet_alpha: float = 0.5
    description: str = ""

    @property
    def f1(self):
        # gated activations (SwiGLU, QGeGLU) read [gate | up]; an activation is a name or
        # ("tanh_srelu", clamp scale)
        name = self.activation[0] if isinstance(self.activation, tuple) else self.activation
        return 2 * self.ffn if name in (SWIGLU, QGEGLU) else self.ffn


CONFIGS = {
    "tiny": Config(
        "tiny", 2, 128, 128, SWIGLU, MXFP8, 192, "fixed", fixed_splits=(64, 128),
        w1_std=1 / np.sqrt(128), w2_std=1 / np.sqrt(128), probs="uniform", backward=False,
        description="2 experts, hidden 128, ffn 128, m_splits [64, 128], MXFP8 SwiGLU, forward only"),
    "mid": Config(
        "mid", 8, 4096, 1536, SWIGLU, MXFP8, 32768, "uniform", tokens=16384, topk=2,
        probs="softmax_topk",
        description="8 experts, hidden 4096, ffn 1536, 16384 tokens top-2 = 32768 rows, "
                    "uniform multinomial splits, MXFP8 SwiGLU, fwd+bwd"),
    "nvfp4": Config(
        "nvfp4", 8, 5120, 2048, SRELU, NVFP4, 24576, "equal", probs="uniform",
        description="8 experts, hidden 5120, ffn 2048, 24576 rows split equally, "
                    "NVFP4 + 16x16 RHT, prob-scaled SReLU, fwd+bwd with recompute on and off"),
    "zipf": Config(
        "zipf", 64, 2048, 1408, SWIGLU, MXFP8, 49152, "zipf", tokens=8192, topk=6,
        probs="normalized_topk", zipf_zero=4,
        description="64 experts, hidden 2048, ffn 1408, 8192 tokens top-6 = 49152 rows, "
                    "Zipf(1.2) counts with 4 empty experts, MXFP8 SwiGLU, fwd+bwd"),
    "large": Config(
        "large", 128, 7168, 2048, SWIGLU, MXFP8, 65536, "dirichlet", tokens=8192, topk=8,
        w1_std=0.01, w2_std=0.01, probs="normalized_topk", stacked=True,
        description="128 experts, hidden 7168, ffn 2048, 8192 tokens top-8 = 65536 rows, "
                    "Dirichlet(0.5) counts, stacked weights, MXFP8 SwiGLU, fwd+bwd"),
}


@dataclass
class Workload:
    config: Config
    m_splits: np.ndarray             # int32 [E]
    x: np.ndarray                    # uint16 bf16 bits [M, H]
    w1: np.ndarray                   # uint16 bf16 bits [E, F1, H]
    w2: np.ndarray                   # uint16 bf16 bits [E, H, ffn]
    probs: np.ndarray                # float32 [M]
    dy: np.ndarray                   # uint16 bf16 bits [M, H] (None when forward only)
    sign_mask: int
    seed: int = 0
    extra: dict = field(default_factory=dict)


def _streams(seed):
    return dict(zip(STREAMS, np.random.SeedSequence(seed).spawn(len(STREAMS))))


def draw_splits(cfg, ss):
    rng = np.random.default_rng(ss)
    e, m = cfg.experts, cfg.rows
    if cfg.splits == "fixed":
        s = np.array(cfg.fixed_splits, dtype=np.int64)
    elif cfg.splits == "equal":
        s = np.full(e, m // e, dtype=np.int64)
        s[: m - s.sum()] += 1
    elif cfg.splits == "uniform":
        s = rng.multinomial(m, np.full(e, 1.0 / e))
    elif cfg.splits == "zipf":
        ranks = rng.permutation(e) + 1
        p = ranks.astype(np.float64) ** (-cfg.zipf_s)
        p /= p.sum()
        s = rng.multinomial(m, p)
        if cfg.zipf_zero:
            order = np.argsort(p)                      # smallest probability first
            moved = s[order[: cfg.zipf_zero]].sum()
            s[order[: cfg.zipf_zero]] = 0
            s[order[-1]] += moved
    elif cfg.splits == "dirichlet":
        p = rng.dirichlet(np.full(e, cfg.dirichlet_alpha))
        s = rng.multinomial(m, p)
    else:
        raise ValueError(cfg.splits)
    assert s.sum() == m
    return s.astype(np.int32)


def draw_normal_bf16(ss, shape, std):
    rng = np.random.default_rng(ss)
    return to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))


def draw_weights(ss, experts, shape, std, only=None):
    """Per-expert child streams: expert e's [N, K] matrix comes from child e alone."""
    kids = ss.spawn(experts)
    idx = range(experts) if only is None else only
    return np.stack([draw_normal_bf16(kids[e], shape, std) for e in idx]) if len(idx) else \
        np.zeros((0,) + tuple(shape), np.uint16)


def draw_probs(cfg, ss, rows):
    rng = np.random.default_rng(ss)
    if cfg.probs == "uniform":
        return rng.random(rows, dtype=np.float32)
    logits = rng.standard_normal((cfg.tokens, cfg.experts))
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    sm = z / z.sum(axis=1, keepdims=True)
    top = -np.sort(-sm, axis=1)[:, : cfg.topk]
    if cfg.probs == "normalized_topk":
        top = top / top.sum(axis=1, keepdims=True)
    flat = top.reshape(-1).astype(np.float32)
    assert flat.size == rows
    return flat


def make_workload(cfg, seed=0, with_weights=True):
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    st = _streams(seed)
    splits = draw_splits(cfg, st["splits"])
    m = int(splits.sum())
    x = draw_normal_bf16(st["x"], (m, cfg.hidden), cfg.x_std)
    w1 = draw_weights(st["w1"], cfg.experts, (cfg.f1, cfg.hidden), cfg.w1_std) if with_weights else None
    w2 = draw_weights(st["w2"], cfg.experts, (cfg.hidden, cfg.ffn), cfg.w2_std) if with_weights else None
    probs = draw_probs(cfg, st["probs"], m)
    dy = draw_normal_bf16(st["dy"], (m, cfg.hidden), 1.0) if cfg.backward else None
    mask = int(np.random.default_rng(st["sign_mask"]).integers(0, 1 << 16))
    return Workload(cfg, splits, x, w1, w2, probs, dy, mask, seed)


def expert_weights(cfg, seed, experts):
    """Draw only the listed experts' (W1, W2) -- identical to the full draw's slices."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    st = _streams(seed)
    w1 = draw_weights(st["w1"], cfg.experts, (cfg.f1, cfg.hidden), cfg.w1_std, only=list(experts))
    w2 = draw_weights(st["w2"], cfg.experts, (cfg.hidden, cfg.ffn), cfg.w2_std, only=list(experts))
    return w1, w2


def iter_expert_weights(cfg, seed=0, chunk=16, threads=8):
    """Yield (experts, W1 bits [n, F1, H], W2 bits [n, H, ffn]) for consecutive chunks of experts,
    each expert drawn on a worker thread from its own child stream (identical to the full draw);
    keeps host memory to one chunk for the largest workloads."""
    from concurrent.futures import ThreadPoolExecutor
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    with ThreadPoolExecutor(threads) as ex:
        for e0 in range(0, cfg.experts, chunk):
            idx = list(range(e0, min(cfg.experts, e0 + chunk)))
            parts = list(ex.map(lambda e: expert_weights(cfg, seed, [e]), idx))
            yield idx, np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def small_case(m_splits, hidden, ffn, activation=SWIGLU, recipe=MXFP8, seed=0,
               x_std=1.0, w_std=None, backward=True, probs="uniform"):
    """A small ad-hoc case for parity tests (same stream layout as the configs)."""
    e = len(m_splits)
    if w_std is None:
        w_std = 1.0 / np.sqrt(hidden)
    cfg = Config(f"small{tuple(m_splits)}", e, hidden, ffn, activation, recipe, int(sum(m_splits)),
                 "fixed", fixed_splits=tuple(int(v) for v in m_splits), x_std=x_std,
                 w1_std=w_std, w2_std=1.0 / np.sqrt(ffn), probs=probs, backward=backward)
    return make_workload(cfg, seed)


def random_bf16(shape, seed, std=1.0, dist="normal"):
    """Plain seeded bf16 tensor (bit patterns) for kernel-level tests."""
    rng = np.random.default_rng(seed)
    if dist == "normal":
        a = rng.standard_normal(shape, dtype=np.float32) * np.float32(std)
    elif dist == "srelu":                       # prob-scaled squared-ReLU-shaped activations
        h = rng.standard_normal(shape, dtype=np.float32)
        a = np.maximum(h, 0) ** 2 * rng.random(shape[:1], dtype=np.float32)[:, None]
    elif dist == "wide":                        # magnitudes spread over many binades
        a = rng.standard_normal(shape, dtype=np.float32) * np.exp2(
            rng.integers(-40, 40, size=shape)).astype(np.float32)
    else:
        raise ValueError(dist)
    return to_bf16_bits(a)


def all_bf16_finite():
    """Every finite bf16 bit pattern (65536 minus the NaN/Inf ones)."""
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    exp = (b >> 7) & 0xFF
    return b[exp != 0xFF]
