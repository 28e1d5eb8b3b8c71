"""Pins of the oracle's quantize / pack / dequantize against definitions independent of it.

- exact re-derivation of every IEEE step with rational arithmetic (tests/ieee_exact.py);
- brute force: each code is the nearest of the 16 levels (ties to even) unless clamped;
- the half-step error bound per group, on stored fp16 scale and zero;
- special cases: min -> 0, max -> 15, constant groups round-trip, zero groups;
- an exhaustive pack / unpack round trip and a hand-built packing example.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from synth import gen
from tests.ieee_exact import INF, f16, f32, round_even_int

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _groups_mix(seed=0):
    """A [rows][256] bf16 matrix whose 64-groups cover the interesting regimes."""
    rng = np.random.default_rng(seed)
    rows = []
    rows.append(rng.standard_normal(256) * 0.02)                  # the configs' distribution
    rows.append(rng.uniform(-3, 3, 256))
    rows.append(rng.standard_t(2, 256))                            # heavy tails
    rows.append(np.r_[np.full(64, 0.375), np.full(64, -1.5), np.zeros(64), np.full(64, 7.0)])
    # constant groups beyond fp16 range (z overflows: range widened to include 0), a group
    # whose scale saturates fp16, and a near-constant group far from 0
    rows.append(np.r_[np.full(64, 1.0e5), np.full(64, -2.5e5), np.linspace(-6e5, 6e5, 64),
                      200 + 4 * rng.standard_normal(64)])
    rows.append(np.r_[rng.uniform(0, 1, 128), -rng.uniform(0, 1, 128)])   # one-signed groups
    rows.append(1e-30 * rng.standard_normal(256))                  # scale underflows to 0
    rows.append(np.r_[np.full(64, -0.0), rng.standard_normal(192) * 1e3])
    return gen.bf16_bits(np.array(rows))


def _spec_group(wvals):
    """Quantize one group with rational arithmetic and explicit IEEE roundings."""
    lo, hi = min(wvals), max(wvals)

    def sz(lo, hi):
        scale = f32(f32(hi - lo) / 15)
        s = f16(scale)
        if s == INF:
            s = Fraction(65504)
        if s == 0:
            s = Fraction(1)
        z = f16(f32((0 - lo) / s))
        return s, z

    s, z = sz(lo, hi)
    if abs(z) == INF:
        s, z = sz(min(lo, Fraction(0)), max(hi, Fraction(0)))
    q = [min(15, max(0, round_even_int(f32(f32(w / s) + z)))) for w in wvals]
    return s, z, q


def test_quantize_matches_exact_ieee_derivation():
    w = _groups_mix()
    q, s, z = oracle.quantize(w)
    wf = oracle.bf16_to_f32(w)
    N, K = w.shape
    for n in range(N):
        for g in range(K // 64):
            vals = [Fraction(float(x)) for x in wf[n, 64 * g:64 * (g + 1)]]
            ss, zz, qq = _spec_group(vals)
            assert Fraction(float(s[n, g])) == ss, (n, g)
            assert Fraction(float(z[n, g])) == zz, (n, g)
            assert list(q[n, 64 * g:64 * (g + 1)]) == qq, (n, g)


def test_zero_is_positive_zero():
    # 0 - lo is +0 for lo = +-0, so zero groups and groups whose minimum is zero store +0.
    w = gen.bf16_bits(np.r_[np.full(64, -0.0), np.zeros(64), np.linspace(0, 1, 64)][None, :])
    _, _, z = oracle.quantize(w)
    assert np.all(z.view(np.uint16) == 0)


def test_codes_are_nearest_level_brute_force():
    rng = np.random.default_rng(3)
    w = gen.bf16_bits(rng.standard_normal((16, 512)) * 0.02)
    q, s, z = oracle.quantize(w)
    wf = oracle.bf16_to_f32(w)
    checked = 0
    for n in range(16):
        for k in range(512):
            g = k // 64
            u = Fraction(float(wf[n, k])) / Fraction(float(s[n, g])) + Fraction(float(z[n, g]))
            errs = sorted((abs(u - c), c) for c in range(16))
            (e0, c0), (e1, _) = errs[0], errs[1]
            if e1 - e0 < Fraction(1, 1 << 18):      # near tie: fp32 rounding may pick either
                continue
            assert q[n, k] == c0, (n, k, float(u))
            checked += 1
    assert checked > 8000


def test_half_step_error_bound():
    rng = np.random.default_rng(5)
    rows = np.concatenate([rng.standard_normal((64, 512)) * 0.02,
                           rng.uniform(-2, 5, (32, 512)),
                           rng.standard_t(3, (32, 512)),
                           300 + rng.standard_normal((8, 512)) * 0.05])
    w = gen.bf16_bits(rows)
    q, s, z = oracle.quantize(w)
    wf = oracle.bf16_to_f32(w).astype(np.float64)
    s64 = np.repeat(s.astype(np.float64), 64, axis=1)
    z64 = np.repeat(z.astype(np.float64), 64, axis=1)
    recon = (q.astype(np.float64) - z64) * s64
    bound = 0.5 * s64 + 2.0 ** -24 * (np.abs(wf) + 16 * s64)
    assert np.all(np.abs(wf - recon) <= bound)
    deq = oracle.dequantize_f16(q, s, z).astype(np.float64)
    ulp16 = np.spacing(np.abs(deq).astype(np.float16)).astype(np.float64)
    bound16 = 0.5 * s64 + 0.5 * ulp16 + 2.0 ** -21 * (np.abs(wf) + 16 * s64)
    assert np.all(np.abs(wf - deq) <= bound16)


def test_group_extremes_map_to_end_codes():
    rng = np.random.default_rng(7)
    w = gen.bf16_bits(rng.standard_normal((32, 256)))
    q, _, _ = oracle.quantize(w)
    wf = oracle.bf16_to_f32(w).reshape(32, 4, 64)
    qg = q.reshape(32, 4, 64)
    lo_idx = wf.argmin(axis=2)
    hi_idx = wf.argmax(axis=2)
    assert np.all(np.take_along_axis(qg, lo_idx[..., None], 2) == 0)
    assert np.all(np.take_along_axis(qg, hi_idx[..., None], 2) == 15)


def test_constant_groups_round_trip_exactly():
    vals = np.array([0.0, 1.0, -2.5, 0.0625, 1024.0, -3.140625, 6.0e4])
    w = gen.bf16_bits(np.repeat(vals, 64)[None, :])
    q, s, z = oracle.quantize(w)
    assert np.all(q == 0) and np.all(s == np.float16(1))
    deq = oracle.dequantize_f16(q, s, z)
    assert np.array_equal(deq.astype(np.float32), oracle.bf16_to_f32(w))


def test_dequantize_f16_exact_derivation():
    rng = np.random.default_rng(11)
    w = gen.bf16_bits(rng.standard_normal((4, 256)) * 0.05)
    q, s, z = oracle.quantize(w)
    deq = oracle.dequantize_f16(q, s, z)
    for n in range(4):
        for k in range(0, 256, 3):
            g = k // 64
            d = f16(f32(f32(int(q[n, k]) - Fraction(float(z[n, g]))) * Fraction(float(s[n, g]))))
            assert Fraction(float(deq[n, k])) == d


def test_exact_dequant_is_the_rational_value():
    rng = np.random.default_rng(13)
    w = gen.bf16_bits(rng.standard_normal((3, 128)))
    q, s, z = oracle.quantize(w)
    d = oracle.dequant_exact64(q, s, z)
    for n in range(3):
        for k in range(128):
            g = k // 64
            exact = (int(q[n, k]) - Fraction(float(z[n, g]))) * Fraction(float(s[n, g]))
            assert Fraction(float(d[n, k])) == exact


def test_pack_unpack_exhaustive():
    a, b = np.meshgrid(np.arange(16, dtype=np.uint8), np.arange(16, dtype=np.uint8))
    q = np.stack([a.ravel(), b.ravel()], axis=1).reshape(1, 512)
    p = oracle.pack_int4(q)
    assert p.shape == (1, 256)
    assert sorted(p.ravel().tolist()) == list(range(256))
    assert np.array_equal(oracle.unpack_int4(p), q)
    rng = np.random.default_rng(17)
    q2 = rng.integers(0, 16, (64, 4096)).astype(np.uint8)
    assert np.array_equal(oracle.unpack_int4(oracle.pack_int4(q2)), q2)


def test_golden_pack_example():
    gold = json.load(open(os.path.join(GOLD, "pack_example.json")))
    q = np.array(gold["codes"], dtype=np.uint8)[None, :]
    assert oracle.pack_int4(q).ravel().tolist() == gold["bytes"]
    words = oracle.pack_int4(q).view(np.uint32).ravel().tolist()
    assert words == gold["le_u32_words"]


def test_golden_ramp_group():
    gold = json.load(open(os.path.join(GOLD, "quant_ramp.json")))
    w = gen.bf16_bits(np.array([[(k - 16) / 32 for k in range(64)]]))
    q, s, z = oracle.quantize(w)
    assert float(s[0, 0]) == gold["scale"]
    assert float(z[0, 0]) == gold["zero"]
    for k, code in gold["codes"].items():
        assert int(q[0, int(k)]) == code
    deq = oracle.dequantize_f16(q, s, z)
    for k, val in gold["dequant"].items():
        assert float(deq[0, int(k)]) == val


def test_rejects_ragged_k():
    with pytest.raises(ValueError):
        oracle.quantize(np.zeros((2, 96), dtype=np.uint16))
