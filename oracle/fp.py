"""Oracle-side float format helpers (bf16 is carried as uint16 bit patterns).

TEST INFRASTRUCTURE ONLY (see the package header).
"""

import numpy as np


def bf16_to_f32(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32: the bf16 bits are the top half."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_to_f64(bits) -> np.ndarray:
    return bf16_to_f32(bits).astype(np.float64)


def f32_to_bf16(x) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); NaN maps to a quiet NaN."""
    x32 = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x32.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(x32)
    if nan.any():
        r = np.where(nan, np.uint16(0x7FC0), r)
    return r
