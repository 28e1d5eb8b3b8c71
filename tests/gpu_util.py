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


def bf16_half_ulp(v):
    """Half a bf16 unit in the last place at |v| (8 significant bits): the largest error
    of storing v in bf16 with round-to-nearest."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - 8), 0.0)


def assert_close(got, ref, rel_l2=1e-2, max_abs=2e-2, scale_abs=False, bf16_out=False, what=""):
    """rel-L2 <= rel_l2 and |got - ref| <= max_abs elementwise (times max(1, rms(ref)) if
    scale_abs). For an output stored in bf16 (bf16_out) each element may in addition be off
    by the storage rounding, half a bf16 ulp of the reference value."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = got - ref
    den = np.linalg.norm(ref)
    rl2 = np.linalg.norm(err) / den if den > 0 else np.linalg.norm(err)
    mab = np.max(np.abs(err)) if err.size else 0.0
    lim = max_abs * (max(1.0, float(np.sqrt(np.mean(ref ** 2)))) if scale_abs else 1.0)
    bound = lim + (bf16_half_ulp(ref) if bf16_out else 0.0)
    excess = np.max(np.abs(err) - bound) if err.size else 0.0
    if bf16_out:
        # the margin without the storage allowance, so the allowance's need stays on record
        bare = np.max(np.abs(err) - lim) if err.size else 0.0
        print(f"MARGIN {what}: rel-L2 {rl2:.3e}, max-abs {mab:.3e}, limit {lim:.3e}, "
              f"excess without the half-ulp allowance {bare:.3e}, with it {excess:.3e}", flush=True)
    assert rl2 <= rel_l2 and excess <= 0, (
        f"{what}: rel-L2 {rl2:.3e} (<= {rel_l2}), max-abs {mab:.3e} (<= {lim:.3e}"
        f"{' + half bf16 ulp' if bf16_out else ''}; worst excess {excess:.3e})")
    return rl2, mab
