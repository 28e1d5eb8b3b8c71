"""Pins of the oracle's tree mask and greedy acceptance walk.

- brute force: the mask equals explicit parent-chasing on every tree of up to 7 nodes;
- closed forms: a chain gives the lower-triangular mask and depth i;
- brute force: the walk equals the longest fully-matching root path on all small trees;
- invariants: draft == target accepts the whole chain; total mismatch accepts nothing;
  the seeded logits' planted acceptance is recovered exactly;
- a hand-built example (tests/golden/tree_example.json).
"""

import itertools
import json
import os

import numpy as np
import pytest

import oracle
from synth import gen

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def all_trees(T):
    for rest in itertools.product(*[range(i) for i in range(1, T)]):
        yield np.array((-1,) + rest, dtype=np.int32)


def chase(parents, i):
    out = set()
    while i >= 0:
        out.add(i)
        i = int(parents[i])
    return out


def mask_bit(m, i, j):
    return (int(m[i, j // 64]) >> (j % 64)) & 1


@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 6, 7])
def test_mask_equals_parent_chasing_all_trees(T):
    for par in all_trees(T):
        m = oracle.tree_mask(par)
        d = oracle.tree_depth(par)
        for i in range(T):
            anc = chase(par, i)
            assert {j for j in range(T) if mask_bit(m, i, j)} == anc
            assert d[i] == len(anc) - 1


@pytest.mark.parametrize("T", [1, 63, 64, 65, 130, 256])
def test_chain_mask_is_lower_triangle(T):
    par = gen.tree_parents(T, "chain")
    m = oracle.tree_mask(par)
    assert m.shape == (T, (T + 63) // 64)
    for i in range(T):
        for j in range(T):
            assert mask_bit(m, i, j) == (1 if j <= i else 0)
    assert np.array_equal(oracle.tree_depth(par), np.arange(T))


@pytest.mark.parametrize("kind,T", [("R", 200), ("CB", 64), ("RB", 256)])
def test_mask_large_random_trees(kind, T):
    par = gen.tree_parents(T, kind, seed=1)
    m = oracle.tree_mask(par)
    for i in range(0, T, 7):
        anc = chase(par, i)
        assert {j for j in range(T) if mask_bit(m, i, j)} == anc


def test_validate_rejects_bad_trees():
    assert oracle.validate_tree([-1, 0, 1])
    assert not oracle.validate_tree([])
    assert not oracle.validate_tree([0, 0])          # root must have parent -1
    assert not oracle.validate_tree([-1, 1])         # self-loop
    assert not oracle.validate_tree([-1, 2, 0])      # forward reference
    assert not oracle.validate_tree([-1, -1])        # second root
    with pytest.raises(ValueError):
        oracle.tree_mask([-1, 2, 0])


def brute_accept(parents, tokens, tgt):
    """Longest root path whose every node's token is the target's choice at its parent."""
    T = len(parents)
    best = []
    for leaf in range(T):
        path = []
        j = leaf
        while j > 0:
            path.append(j)
            j = int(parents[j])
        path = path[::-1]
        ok = all(int(tokens[n]) == int(tgt[int(parents[n])]) for n in path)
        if ok and len(path) > len(best):
            best = path
    return best


def test_accept_equals_brute_force_small_trees():
    rng = np.random.default_rng(0)
    n = 0
    for T in range(1, 8):
        for par in all_trees(T):
            for _ in range(4):
                # distinct sibling tokens from a 3-token alphabet where possible
                tok = np.zeros(T, dtype=np.int32)
                for p in set(par.tolist()):
                    kids = [i for i in range(T) if par[i] == p]
                    tok[kids] = rng.permutation(max(3, len(kids)))[:len(kids)]
                tgt = rng.integers(0, 3, T).astype(np.int32)
                path, L, bonus = oracle.accept(par, tok, tgt)
                best = brute_accept(par, tok, tgt)
                assert path == best and L == len(best)
                assert bonus == int(tgt[best[-1] if best else 0])
                n += 1
    assert n > 1000


@pytest.mark.parametrize("kind,T", [("CB", 48), ("CB", 64), ("RB", 256), ("R", 16)])
def test_draft_equals_target_accepts_whole_chain(kind, T):
    par = gen.tree_parents(T, kind, seed=2)
    tok = gen.tree_tokens(par, 1000, seed=2)
    chain = gen.chain_path(par)
    tgt = np.full(T, 999999, dtype=np.int32)
    for a, b in zip(chain[:-1], chain[1:]):
        tgt[a] = tok[b]
    path, L, bonus = oracle.accept(par, tok, tgt)
    assert path == chain[1:]
    assert L == int(oracle.tree_depth(par)[chain[-1]])
    assert bonus == 999999


def test_total_mismatch_accepts_nothing():
    par = gen.tree_parents(64, "CB", seed=3)
    tok = gen.tree_tokens(par, 1000, seed=3)
    tgt = np.full(64, 5000, dtype=np.int32)
    assert oracle.accept(par, tok, tgt) == ([], 0, 5000)


@pytest.mark.parametrize("L_star", [0, 1, 27, 48])
def test_planted_logits_recover_L_star(L_star):
    T, V = 64, 2000
    par = gen.tree_parents(T, "CB", seed=4)
    tok = gen.tree_tokens(par, V, seed=4)
    lg = gen.target_logits(par, tok, V, L_star, seed=4)
    tgt = np.argmax(lg, axis=1)
    path, L, _ = oracle.accept(par, tok, tgt)
    assert L == L_star
    assert path == gen.chain_path(par)[1:L_star + 1]


def test_golden_tree_example():
    gold = json.load(open(os.path.join(GOLD, "tree_example.json")))
    par = np.array(gold["parents"], dtype=np.int32)
    m = oracle.tree_mask(par)
    assert m[:, 0].tolist() == gold["mask_words"]
    assert oracle.tree_depth(par).tolist() == gold["depth"]
    for case in gold["accept_cases"]:
        path, L, bonus = oracle.accept(par, gold["tokens"], case["target_argmax"])
        assert path == case["path"] and L == case["accept_len"] and bonus == case["bonus"]
