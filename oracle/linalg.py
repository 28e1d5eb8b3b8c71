"""fp64 matrix products of the substitute linear layers.

TEST INFRASTRUCTURE ONLY (see the package header).

The substitute layer runs the quantized weight against bf16 activations over all
draft-tree tokens at once ([Summary] "Approach"; [Abstract]): Y = X · deq(W)^T,
with deq(W) = (q - z) · s taken exactly.
"""

import numpy as np

from .fp import bf16_to_f64
from .quant import dequant_exact64


def matmul64(x64: np.ndarray, w64: np.ndarray) -> np.ndarray:
    """Y[m, n] = sum_k X[m, k] W[n, k] in fp64."""
    return np.asarray(x64, dtype=np.float64) @ np.asarray(w64, dtype=np.float64).T


def w4a16_matmul64(x_bf16_bits, q, s16, z16, group: int = 64) -> np.ndarray:
    """W4A16 substitute linear layer in fp64: bf16 X [T][K] times the exact dequantized W [N][K]."""
    return matmul64(bf16_to_f64(x_bf16_bits), dequant_exact64(q, s16, z16, group))
