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
