"""Helpers shared by the GPU parity tests (host <-> device marshalling of test data only)."""
import numpy as np
import torch


def dev_bf16(bits):
    """numpy uint16 bf16 bit patterns -> bf16 tensor on cuda:0."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)


def dev_splits(splits):
    return torch.tensor(np.asarray(splits, dtype=np.int32), device="cuda")


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")


def u8(t):
    return t.detach().cpu().contiguous().view(torch.uint8).numpy()


def u32(t):
    return t.detach().cpu().contiguous().view(torch.int32).numpy().view(np.uint32)


def bits16(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def f32bits(t):
    return t.detach().cpu().contiguous().float().numpy().view(np.uint32)


def col_total(splits, pad=128):
    return int(sum(-(-int(m) // pad) * pad for m in splits))


def assert_bytes_equal(got, want, what):
    got = np.asarray(got).reshape(-1)
    want = np.asarray(want).reshape(-1)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{what}: {bad.size} of {want.size} differ; first at {bad[:5]}: got {got[bad[:5]]}, want {want[bad[:5]]}"


def unpanel(buf, R, K):
    """MXFP8 data in 64-byte K panels -> [R, K] row-major.  Panel p holds columns
    [64 p, 64 p + w), w = min(64, K - 64 p), as R rows of w bytes starting at byte 64 p R."""
    buf = np.asarray(buf).reshape(-1)
    out = np.empty((R, K), np.uint8)
    for p0 in range(0, K, 64):
        w = min(64, K - p0)
        out[:, p0:p0 + w] = buf[p0 * R:p0 * R + R * w].reshape(R, w)
    return out


def unpanel_groups(buf, K, splits, pad=128):
    """Column-wise MXFP8 data of groups [K, P_g] (each in 64-byte token panels) -> the
    concatenation of the groups' [K, P_g] row-major blocks."""
    buf = np.asarray(buf).reshape(-1)
    parts, off = [], 0
    for m in splits:
        P = -(-int(m) // pad) * pad
        parts.append(unpanel(buf[off:off + K * P], K, P).reshape(-1))
        off += K * P
    return np.concatenate(parts) if parts else np.zeros(0, np.uint8)
