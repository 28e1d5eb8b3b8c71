"""Pins of the oracle's float-format helpers and fp64 matrix products.

bf16 rounding and widening are checked against IEEE-754 rounding on exact rationals
(tests/ieee_exact.py) and an independent sign / exponent / mantissa decode; the fp64
products against explicit triple loops over the packed int4 codes, and against the
special case that identity rows of X return the dequantized weight rows.
"""

import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests.ieee_exact import bf16 as bf16_exact


def decode_bf16(bits: int):
    """Value of a bf16 bit pattern from its fields: 1 sign, 8 exponent, 7 mantissa bits."""
    s = -1 if (bits >> 15) & 1 else 1
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    if e == 0xFF:
        return math.nan if m else s * math.inf
    if e == 0:
        return s * Fraction(m, 128) * Fraction(2) ** -126
    return s * (1 + Fraction(m, 128)) * Fraction(2) ** (e - 127)


def f32_of_bits(u: int) -> np.float32:
    return np.array([u], dtype=np.uint32).view(np.float32)[0]


def _sweep_f32_patterns():
    """fp32 bit patterns at, just below and just above every bf16 rounding tie of a
    sweep of exponents (normal, subnormal, near overflow), plus zeros, infinities,
    the largest finite values and random patterns."""
    pats = set()
    rng = np.random.default_rng(1234)
    exps = list(range(0, 6)) + list(range(100, 140)) + list(range(249, 255))
    for e in exps:
        for sign in (0, 1):
            for m_hi in rng.integers(0, 128, 6).tolist() + [0, 1, 126, 127]:
                base = (sign << 31) | (e << 23) | (m_hi << 16)
                for low in (0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF):
                    pats.add(base | low)
    pats.update([0x00000000, 0x80000000, 0x7F800000, 0xFF800000, 0x7F7FFFFF, 0xFF7FFFFF,
                 0x7F7F7FFF, 0x7F7F8000, 0x7F7F8001, 0x00000001, 0x807FFFFF, 0x00008000,
                 0x00018000])
    pats.update(rng.integers(0, 2 ** 32, 4000, dtype=np.uint64).astype(np.uint32).tolist())
    return sorted(pats)


def test_f32_to_bf16_is_ieee_round_to_nearest_even():
    pats = _sweep_f32_patterns()
    x = np.array(pats, dtype=np.uint32).view(np.float32)
    got = oracle.f32_to_bf16(x)
    for u, g in zip(pats, got.tolist()):
        f = f32_of_bits(u)
        if np.isnan(f):
            # any NaN input gives a NaN pattern (exponent all ones, mantissa non-zero)
            assert (g >> 7) & 0xFF == 0xFF and (g & 0x7F) != 0, hex(u)
            continue
        want = bf16_exact(Fraction(float(f))) if np.isfinite(f) else (math.inf if f > 0 else -math.inf)
        have = decode_bf16(g)
        if want == 0:
            assert have == 0, hex(u)
            # the sign of zero is kept
            assert (g >> 15) == (u >> 31), hex(u)
        else:
            assert have == want, (hex(u), hex(g), want)


def test_f32_to_bf16_ties_go_to_even():
    # 1 + 2^-8 lies halfway between bf16 1.0 and 1 + 2^-7: even mantissa (1.0) wins;
    # 1 + 3 * 2^-8 lies between 1 + 2^-7 and 1 + 2^-6: even (1 + 2^-6) wins
    vals = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8)], dtype=np.float32)
    assert oracle.f32_to_bf16(vals).tolist() == [0x3F80, 0x3F82, 0xBF80]


def test_f32_to_bf16_nan_and_overflow():
    vals = np.array([np.nan, np.inf, -np.inf, np.finfo(np.float32).max], dtype=np.float32)
    r = oracle.f32_to_bf16(vals).tolist()
    assert (r[0] >> 7) & 0xFF == 0xFF and r[0] & 0x7F
    assert r[1] == 0x7F80 and r[2] == 0xFF80
    assert r[3] == 0x7F80   # fp32 max rounds past the largest bf16 to +inf


@pytest.mark.filterwarnings("ignore:invalid value encountered in cast")
def test_bf16_widening_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    w32 = oracle.bf16_to_f32(bits)
    w64 = oracle.bf16_to_f64(bits)
    assert w32.dtype == np.float32 and w64.dtype == np.float64
    for b in range(65536):
        want = decode_bf16(b)
        if isinstance(want, float) and math.isnan(want):
            assert np.isnan(w32[b]) and np.isnan(w64[b])
            continue
        assert Fraction(float(w32[b])) == want if not isinstance(want, float) else w32[b] == want, hex(b)
        assert Fraction(float(w64[b])) == want if not isinstance(want, float) else w64[b] == want, hex(b)
        if want == 0:
            assert math.copysign(1.0, float(w64[b])) == (-1.0 if b >> 15 else 1.0)


def test_widen_then_round_is_identity():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    fin = np.isfinite(oracle.bf16_to_f32(bits))
    back = oracle.f32_to_bf16(oracle.bf16_to_f32(bits))
    assert np.array_equal(back[fin], bits[fin])


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (4, 2, 9), (6, 3, 1)])
def test_matmul64_is_the_triple_loop(M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    x = rng.standard_normal((M, K))
    w = rng.standard_normal((N, K))
    y = oracle.matmul64(x, w)
    assert y.shape == (M, N)
    for m in range(M):
        for n in range(N):
            ref = 0.0
            for k in range(K):
                ref += x[m, k] * w[n, k]
            assert abs(y[m, n] - ref) <= 1e-12 * (1 + sum(abs(x[m, k] * w[n, k]) for k in range(K)))


def _tiny_w4():
    rng = np.random.default_rng(7)
    N, K = 3, 128
    w = oracle.f32_to_bf16((rng.standard_normal((N, K)) * 0.05).astype(np.float32))
    q, s, z = oracle.quantize(w)
    return N, K, q, s, z


def test_w4a16_matmul64_is_the_triple_loop_over_packed_codes():
    N, K, q, s, z = _tiny_w4()
    packed = oracle.pack_int4(q)
    rng = np.random.default_rng(8)
    M = 2
    x = oracle.f32_to_bf16(rng.standard_normal((M, K)).astype(np.float32))
    y = oracle.w4a16_matmul64(x, q, s, z)
    assert y.shape == (M, N)
    for m in range(M):
        for n in range(N):
            ref = Fraction(0)
            for k in range(K):
                byte = int(packed[n, k // 2])
                code = (byte >> 4) if (k % 2) else (byte & 0xF)
                sc = Fraction(float(s[n, k // 64]))
                ze = Fraction(float(z[n, k // 64]))
                ref += decode_bf16(int(x[m, k])) * (code - ze) * sc
            assert abs(Fraction(float(y[m, n])) - ref) <= Fraction(1, 10 ** 12) * (1 + abs(ref)), (m, n)


def test_w4a16_identity_rows_return_dequantized_rows():
    N, K, q, s, z = _tiny_w4()
    eye = oracle.f32_to_bf16(np.eye(K, dtype=np.float32))
    y = oracle.w4a16_matmul64(eye, q, s, z)       # [K][N]: row k is column k of deq(W)
    d = oracle.dequant_exact64(q, s, z)           # [N][K]
    assert np.array_equal(y, d.T)
    # and each dequantized value is (q - z) s of its own group
    for n in range(N):
        for k in range(0, K, 37):
            assert d[n, k] == (float(q[n, k]) - float(z[n, k // 64])) * float(s[n, k // 64])
