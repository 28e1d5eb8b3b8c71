"""Pins of the draft-tree expansion oracle (oracle/expand.py) against facts that do not
come from it: the schedule's arithmetic, log-probabilities from scipy's logsumexp, a
closed-form chain, brute-force ranking of every child on small trees, and the tree
invariants of the finished template."""
import itertools

import numpy as np
import pytest
from scipy.special import log_softmax

import oracle
from oracle import expand as ex


@pytest.mark.parametrize("T,D", [(64, 48), (48, 48 - 1), (16, 5), (9, 8), (256, 48), (7, 6)])
def test_schedule_fills_the_template(T, D):
    b = ex.schedule(T, D)
    assert len(b) == D and sum(b) == T - 1 and min(b) >= 1
    assert max(b) == -(-(T - 1) // D)
    assert all(x >= y for x, y in zip(b, b[1:]))          # front-loaded, never growing


def test_schedule_of_the_7b_template():
    # 63 nodes over 48 levels: 15 levels of two, then 33 of one (depth 48)
    assert ex.schedule(64, 48) == [2] * 15 + [1] * 33


def test_child_scores_are_scipy_log_softmax():
    rng = np.random.default_rng(1)
    l = rng.normal(0, 3, 1000).astype(np.float32)
    inv_t = np.float32(1.0) / np.float32(0.2)
    y = ex.sharpened(l, inv_t)
    ids, lp = ex.children(y, 6)
    ref = log_softmax(y.astype(np.float64))
    assert np.allclose(lp, ref[ids], rtol=0, atol=1e-12)
    # the top 6 by value, lower index on ties
    assert list(ids) == sorted(range(1000), key=lambda i: (-float(y[i]), i))[:6]


def test_ties_prefer_the_lower_token_id():
    y = np.array([1.0, 3.0, 3.0, 2.0, 3.0], dtype=np.float32)
    ids, _ = ex.children(y, 4)
    assert list(ids) == [1, 2, 4, 3]


def test_dominant_token_gives_the_greedy_chain():
    # one token per row far above the rest: with one node per level the tree is the chain
    # of those tokens, each score ~0 (probability ~1)
    T, D, V = 9, 8, 50

    def logits_of(step, parents, tokens, frontier):
        rows = np.zeros((len(frontier), V), np.float32)
        for r, f in enumerate(frontier):
            rows[r, (tokens[f] * 7 + 3) % V] = 40.0
        return rows

    par, tok, cum = ex.expand_tree(11, T, D, logits_of, 1.0 / 0.2, 6)
    assert list(par) == [-1] + list(range(T - 1))
    want = [11]
    for _ in range(T - 1):
        want.append((want[-1] * 7 + 3) % V)
    assert list(tok) == want
    assert np.all(cum <= 0) and np.all(cum > -1e-6)


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_ranking_on_small_trees(seed):
    # every child of every frontier node is scored from scipy's log_softmax; the appended
    # nodes must be the B best of the k best children per node, in score order
    rng = np.random.default_rng(seed)
    T, D, V, k, inv_t = 12, 5, 9, 3, 1.0 / 0.6
    table = rng.normal(0, 2, (T * 4, V)).astype(np.float32)

    def logits_of(step, parents, tokens, frontier):
        return np.stack([table[(tokens[f] * 5 + f + step) % len(table)] for f in frontier])

    par, tok, cum = ex.expand_tree(0, T, D, logits_of, inv_t, k)
    # replay the steps independently
    n, frontier = 1, [0]
    cum_ref = {0: 0.0}
    toks = {0: 0}
    for s, b in enumerate(ex.schedule(T, D)):
        cands = []
        for r, f in enumerate(frontier):
            y = (table[(toks[f] * 5 + f + s) % len(table)] * np.float32(inv_t)).astype(np.float32)
            lp = log_softmax(y.astype(np.float64))
            top = sorted(range(V), key=lambda i: (-float(y[i]), i))[:k]
            for rank, c in enumerate(top):
                cands.append((cum_ref[f] + lp[c], r, rank, f, c))
        best = sorted(cands, key=lambda c: (-c[0], c[1], c[2]))[:b]
        # no unchosen candidate beats a chosen one
        chosen = set((c[3], c[4]) for c in best)
        worst = min(c[0] for c in best)
        assert all(c[0] <= worst + 1e-12 for c in cands if (c[3], c[4]) not in chosen)
        new = []
        for i, c in enumerate(best):
            slot = n + i
            assert par[slot] == c[3] and tok[slot] == c[4] and abs(cum[slot] - c[0]) < 1e-9
            cum_ref[slot], toks[slot] = c[0], c[4]
            new.append(slot)
        n += b
        frontier = new


def test_finished_template_invariants():
    rng = np.random.default_rng(3)
    T, D, V = 64, 48, 300
    table = rng.normal(0, 1.5, (97, V)).astype(np.float32)
    par, tok, cum = ex.expand_tree(5, T, D, lambda s, p, t, fr: np.stack([table[(t[f] + s) % 97] for f in fr]),
                                   1.0 / 0.2, 6)
    assert oracle.validate_tree(par)
    depth = oracle.tree_depth(par)
    assert depth.max() == D
    # slots are appended level by level: depth never decreases with the slot index
    assert np.all(np.diff(depth[1:]) >= 0)
    # a child's score is its parent's plus a log-probability (<= 0)
    assert all(cum[i] <= cum[par[i]] + 1e-12 for i in range(1, T))
    assert len(set(zip(par[1:], tok[1:]))) == T - 1        # no duplicate (parent, token) pair
