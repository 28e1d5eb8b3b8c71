"""Transfers between NumPy arrays (bf16 as uint16 bits) and CUDA tensors, and tolerance checks."""

import numpy as np
import torch


def dev():
    return torch.device("cuda:0")


def to_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev())


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def bf16_bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def host(t):
    return t.detach().cpu().numpy()


def assert_close(got, ref, rel_l2=1e-2, max_abs=2e-2, scale_abs=False, what=""):
    """rel-L2 <= rel_l2 and max |got - ref| <= max_abs (times max(1, rms(ref)) if scale_abs)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = got - ref
    den = np.linalg.norm(ref)
    rl2 = np.linalg.norm(err) / den if den > 0 else np.linalg.norm(err)
    mab = np.max(np.abs(err)) if err.size else 0.0
    lim = max_abs * (max(1.0, float(np.sqrt(np.mean(ref ** 2)))) if scale_abs else 1.0)
    assert rl2 <= rel_l2 and mab <= lim, f"{what}: rel-L2 {rl2:.3e} (<= {rel_l2}), max-abs {mab:.3e} (<= {lim:.3e})"
    return rl2, mab
