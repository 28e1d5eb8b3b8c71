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


# ------------------------------------------------------------------ KV commit

def _kv_case(T, C, c_stride, nkv=2, hd=64, seed=0, kind="CB"):
    par = gen.tree_parents(T, kind, seed=seed)
    tok = gen.tree_tokens(par, 1000, seed=seed)
    rng = np.random.default_rng(seed)
    kc = rng.integers(0, 1 << 16, (nkv, c_stride, hd), dtype=np.uint16)
    vc = rng.integers(0, 1 << 16, (nkv, c_stride, hd), dtype=np.uint16)
    kt = rng.integers(0, 1 << 16, (nkv, T, hd), dtype=np.uint16)
    vt = rng.integers(0, 1 << 16, (nkv, T, hd), dtype=np.uint16)
    return par, tok, kc, vc, kt, vt


def test_kv_commit_writes_only_the_committed_rows():
    T, C, cs = 40, 100, 160
    par, tok, kc, vc, kt, vt = _kv_case(T, C, cs, seed=3)
    tgt = gen.target_logits(par, tok, 1000, 9, seed=3).argmax(axis=1)
    path, L, _ = oracle.accept(par, tok, tgt)
    assert L == len(path) > 0
    k2, v2 = oracle.kv_commit(kc, vc, kt, vt, path, C)
    rows = C + L + 1
    assert np.array_equal(k2[:, :C], kc[:, :C]) and np.array_equal(k2[:, rows:], kc[:, rows:])
    assert np.array_equal(v2[:, :C], vc[:, :C]) and np.array_equal(v2[:, rows:], vc[:, rows:])
    assert np.array_equal(k2[:, C], kt[:, 0]) and np.array_equal(v2[:, C], vt[:, 0])   # the root first
    for i, node in enumerate(path):
        assert np.array_equal(k2[:, C + 1 + i], kt[:, node])
        assert np.array_equal(v2[:, C + 1 + i], vt[:, node])
    # nothing accepted: only the root is committed
    k0, _ = oracle.kv_commit(kc, vc, kt, vt, [], C)
    assert np.array_equal(k0[:, C], kt[:, 0]) and np.array_equal(k0[:, C + 1:], kc[:, C + 1:])


def test_kv_commit_matches_attention_over_the_accepted_path():
    # The accepted path is the ancestor chain of its last node, so that node's tree
    # attention must equal plain attention (every key visible) over the committed cache:
    # checked against torch's scaled-dot-product attention, not against the oracle.
    torch = pytest.importorskip("torch")
    T, C, nkv, grp, hd = 48, 64, 2, 3, 64
    par, tok, _, _, _, _ = _kv_case(T, C, C + T, nkv=nkv, hd=hd, seed=5)
    tgt = gen.target_logits(par, tok, 1000, 20, seed=5).argmax(axis=1)
    path, L, _ = oracle.accept(par, tok, tgt)
    assert L >= 10
    rng = np.random.default_rng(5)
    bf = lambda a: oracle.f32_to_bf16(a.astype(np.float32))
    q = bf(rng.standard_normal((T, nkv * grp, hd)))
    kc = bf(rng.standard_normal((nkv, C + T, hd)))
    vc = bf(rng.standard_normal((nkv, C + T, hd)))
    kt = bf(rng.standard_normal((nkv, T, hd)))
    vt = bf(rng.standard_normal((nkv, T, hd)))
    f = oracle.bf16_to_f64
    tree_out = oracle.tree_attention64(f(q), f(kc), f(vc), f(kt), f(vt), par, C)
    last = path[-1]
    k2, v2 = oracle.kv_commit(kc, vc, kt, vt, path, C)
    n = C + L + 1
    for h in range(nkv * grp):
        kvh = h // grp
        qh = torch.from_numpy(f(q[last, h])).view(1, 1, 1, hd)
        kh = torch.from_numpy(f(k2[kvh, :n])).view(1, 1, n, hd)
        vh = torch.from_numpy(f(v2[kvh, :n])).view(1, 1, n, hd)
        ref = torch.nn.functional.scaled_dot_product_attention(qh, kh, vh).view(hd).numpy()
        np.testing.assert_allclose(tree_out[last, h], ref, rtol=1e-10, atol=1e-12)
