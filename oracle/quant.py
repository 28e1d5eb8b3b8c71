"""Substitute construction: int4 group quantization, packing and dequantization.

TEST INFRASTRUCTURE ONLY (see the package header).

[Review] §6.2 and [Summary] "Approach" say the substitute layers are data-free,
training-free 4-bit copies of the target's own layers (named HQQ); [Abstract]
describes them as low-bit quantized stand-ins for the offloaded layers. No page gives
the quantizer's steps,
group size or zero format, so this oracle takes the plainest reading of a data-free
4-bit quantizer: asymmetric min-max round-to-nearest per group of 64 consecutive
input features, with fp16 scale and fp16 (real-valued) zero.

Bit-exact rules, each a single IEEE operation rounded to nearest-even, in fp32
unless stated:
  lo, hi   = min and max of the group (exact: bf16 widens exactly to fp32)
  scale    = (hi - lo) / 15
  s        = fp16(scale); +inf saturates to 65504; s == 0 becomes 1
  z        = fp16((0 - lo) / s)
  if z overflows fp16, the group range is widened to include 0 (lo = min(lo, 0),
    hi = max(hi, 0)) and s, z are recomputed; then 0 <= z <= 15 cannot overflow
  q        = clamp(rint_even(w / s + z), 0, 15)      (two fp32 ops, no FMA)
  dequant  = fp16((q - z) * s)                        (two fp32 ops, no FMA)
"""

import numpy as np

from .fp import bf16_to_f32

F32 = np.float32
F16 = np.float16


def _scale_zero(lo: np.ndarray, hi: np.ndarray):
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        scale = (hi - lo) / F32(15)
        s16 = scale.astype(F16)
        s16 = np.where(np.isinf(s16), F16(65504), s16)
        s16 = np.where(s16 == F16(0), F16(1), s16)
        z32 = (F32(0) - lo) / s16.astype(F32)
        z16 = z32.astype(F16)
    return s16, z16


def quantize(w_bf16_bits: np.ndarray, group: int = 64):
    """Quantize a bf16 weight [N][K] (uint16 bits) to int4 codes, fp16 scales and zeros.

    Returns (q uint8 [N][K] with values 0..15, s float16 [N][K/group], z float16 [N][K/group]).
    """
    w = np.asarray(w_bf16_bits)
    N, K = w.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    G = K // group
    w32 = bf16_to_f32(w).reshape(N, G, group)
    lo = w32.min(axis=2)
    hi = w32.max(axis=2)
    s16, z16 = _scale_zero(lo, hi)
    wide = np.isinf(z16)
    if wide.any():
        s2, z2 = _scale_zero(np.minimum(lo, F32(0)), np.maximum(hi, F32(0)))
        s16 = np.where(wide, s2, s16)
        z16 = np.where(wide, z2, z16)
    s32 = s16.astype(F32)[:, :, None]
    z32 = z16.astype(F32)[:, :, None]
    with np.errstate(over="ignore", invalid="ignore"):
        v = (w32 / s32) + z32
    q = np.clip(np.rint(v), 0, 15).astype(np.uint8).reshape(N, K)
    return q, s16, z16


def pack_int4(q: np.ndarray) -> np.ndarray:
    """Pack codes [N][K] into bytes [N][K/2]: even k in the low nibble, odd k in the high nibble."""
    q = np.asarray(q, dtype=np.uint8)
    N, K = q.shape
    lo = q[:, 0::2] & 0xF
    hi = q[:, 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8).reshape(N, K // 2)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    N, KH = p.shape
    q = np.empty((N, KH * 2), dtype=np.uint8)
    q[:, 0::2] = p & 0xF
    q[:, 1::2] = p >> 4
    return q


def dequantize_f16(q: np.ndarray, s16: np.ndarray, z16: np.ndarray, group: int = 64) -> np.ndarray:
    """fp16 export of the substitute weight: fp16((q - z) * s), each step fp32, no FMA."""
    N, K = q.shape
    G = K // group
    q32 = q.reshape(N, G, group).astype(F32)
    d = (q32 - z16.astype(F32)[:, :, None]) * s16.astype(F32)[:, :, None]
    return d.astype(F16).reshape(N, K)


def dequant_exact64(q: np.ndarray, s16: np.ndarray, z16: np.ndarray, group: int = 64) -> np.ndarray:
    """The substitute weight as a real number, (q - z) * s, evaluated in fp64 (exact)."""
    N, K = q.shape
    G = K // group
    d = (q.reshape(N, G, group).astype(np.float64) - z16.astype(np.float64)[:, :, None]) \
        * s16.astype(np.float64)[:, :, None]
    return d.reshape(N, K)
