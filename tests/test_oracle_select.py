"""Pins of the oracle's row argmax and sharpened draft selection.

- brute force with plain Python loops (ties included) for argmax and top-k;
- exact re-derivation of y = fp32(fp32(l * inv_t) + g) with rational arithmetic;
- special case: g = 0 is plain top-k of the logits for any positive inverse temperature;
- statistics: with Gumbel noise the top-1 frequency over many draws follows
  softmax(l / t) (the Gumbel-max property), within 4 standard errors.
"""

from fractions import Fraction

import numpy as np

import oracle
from synth import gen
from tests.ieee_exact import f32


def test_argmax_brute_force_with_ties():
    rng = np.random.default_rng(0)
    lg = rng.integers(-3, 4, (50, 37)).astype(np.float32)      # many ties
    got = oracle.row_argmax(lg)
    for r in range(50):
        best = 0
        for j in range(37):
            if lg[r, j] > lg[r, best]:
                best = j
        assert got[r] == best


def _topk_brute(y, k):
    return [j for _, j in sorted(((-float(v), j) for j, v in enumerate(y)))[:k]]


def test_greedy_select_is_topk_of_logits():
    rng = np.random.default_rng(1)
    lg = np.round(rng.standard_normal((20, 300)) * 4).astype(np.float32)   # ties
    for inv_t in (1.0, 5.0, 1.0 / 0.6):
        got = oracle.draft_select(lg, None, np.float32(inv_t), 6)
        for r in range(20):
            assert got[r].tolist() == _topk_brute(lg[r] * np.float32(inv_t), 6)
            # scaling by a positive factor only changes ties created by rounding
            assert set(got[r].tolist()) <= set(_topk_brute(lg[r], 12))


def test_select_exact_rounding_derivation():
    rng = np.random.default_rng(2)
    lg = rng.standard_normal((4, 200)).astype(np.float32) * 3
    g = gen.gumbel_f32(4, 200, seed=2)
    inv_t = np.float32(1.0) / np.float32(0.2)
    got = oracle.draft_select(lg, g, inv_t, 6)
    for r in range(4):
        y = [f32(f32(Fraction(float(lg[r, j])) * Fraction(float(inv_t))) + Fraction(float(g[r, j])))
             for j in range(200)]
        ref = [j for _, j in sorted((-v, j) for j, v in enumerate(y))[:6]]
        assert got[r].tolist() == ref


def test_gumbel_top1_follows_tempered_softmax():
    V, draws, t = 5, 20000, 0.6
    lg = np.array([[0.0, 0.3, -0.5, 0.9, 0.1]], dtype=np.float32)
    g = gen.gumbel_f32(draws, V, seed=3)
    tops = oracle.draft_select(np.repeat(lg, draws, axis=0), g, np.float32(1 / t), 1)[:, 0]
    p = np.exp(lg[0] / t) / np.exp(lg[0] / t).sum()
    freq = np.bincount(tops, minlength=V) / draws
    se = np.sqrt(p * (1 - p) / draws)
    assert np.all(np.abs(freq - p) < 4 * se)


def test_topk_are_distinct_and_ordered():
    rng = np.random.default_rng(4)
    lg = rng.standard_normal((8, 1000)).astype(np.float32)
    g = gen.gumbel_f32(8, 1000, seed=4)
    out = oracle.draft_select(lg, g, np.float32(5.0), 6)
    y = lg * np.float32(5.0) + g
    for r in range(8):
        assert len(set(out[r].tolist())) == 6
        vals = y[r, out[r]]
        assert np.all(vals[:-1] >= vals[1:])
        assert np.all(y[r] <= vals[0])
