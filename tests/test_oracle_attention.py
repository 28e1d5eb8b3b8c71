"""Pins of the oracle's tree attention.

- library routine: torch's scaled_dot_product_attention (CPU, fp64) with a boolean mask
  built here by parent-chasing, with GQA expanded by repeat_interleave;
- closed form: a chain tree with no prefix is exactly causal attention (is_causal=True);
- special cases: the root with no prefix sees only itself, so its output is its own v;
  q = 0 gives the mean of the visible values;
- the dense masked form equals the per-query loop form;
- relabelling the tree nodes in another topological order permutes the outputs.
"""

import numpy as np
import pytest
import torch

import oracle
from synth import gen


def _inputs(T, C, nq, nkv, hd, seed=0, kind="R"):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, nq, hd))
    kc = rng.standard_normal((nkv, C + 3, hd))
    vc = rng.standard_normal((nkv, C + 3, hd))
    kt = rng.standard_normal((nkv, T, hd))
    vt = rng.standard_normal((nkv, T, hd))
    par = gen.tree_parents(T, kind, seed=seed)
    return q, kc, vc, kt, vt, par


def _chase_mask(par, C):
    T = len(par)
    m = np.zeros((T, C + T), dtype=bool)
    m[:, :C] = True
    for i in range(T):
        j = i
        while j >= 0:
            m[i, C + j] = True
            j = int(par[j])
    return m


def _sdpa(q, kc, vc, kt, vt, mask_bool, C, nq, nkv, is_causal=False):
    K = np.concatenate([kc[:, :C], kt], axis=1)
    V = np.concatenate([vc[:, :C], vt], axis=1)
    grp = nq // nkv
    Kt = torch.from_numpy(K).repeat_interleave(grp, dim=0)          # [nq][C+T][hd]
    Vt = torch.from_numpy(V).repeat_interleave(grp, dim=0)
    Q = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))  # [nq][T][hd]
    if is_causal:
        out = torch.nn.functional.scaled_dot_product_attention(Q, Kt, Vt, is_causal=True)
    else:
        out = torch.nn.functional.scaled_dot_product_attention(
            Q, Kt, Vt, attn_mask=torch.from_numpy(mask_bool))
    return out.numpy().transpose(1, 0, 2)


@pytest.mark.parametrize("T,C,nq,nkv,hd,kind", [
    (16, 128, 1, 1, 64, "R"), (48, 40, 7, 1, 32, "CB"), (33, 0, 4, 2, 16, "RB"),
    (70, 5, 8, 4, 16, "R"), (1, 9, 2, 1, 8, "R")])
def test_matches_sdpa_with_chased_mask(T, C, nq, nkv, hd, kind):
    q, kc, vc, kt, vt, par = _inputs(T, C, nq, nkv, hd, seed=T + C, kind=kind)
    got = oracle.tree_attention64(q, kc, vc, kt, vt, par, C)
    ref = _sdpa(q, kc, vc, kt, vt, _chase_mask(par, C), C, nq, nkv)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_chain_without_prefix_is_causal_attention():
    T, nq, nkv, hd = 40, 4, 2, 16
    q, kc, vc, kt, vt, _ = _inputs(T, 0, nq, nkv, hd, seed=5)
    par = gen.tree_parents(T, "chain")
    got = oracle.tree_attention64(q, kc, vc, kt, vt, par, 0)
    ref = _sdpa(q, kc, vc, kt, vt, None, 0, nq, nkv, is_causal=True)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    # the chain mask itself is the causal mask, bit for bit
    m = oracle.tree_mask(par)
    causal = np.tril(np.ones((T, T), dtype=bool))
    bits = np.array([[(int(m[i, j // 64]) >> (j % 64)) & 1 for j in range(T)] for i in range(T)])
    assert np.array_equal(bits.astype(bool), causal)


def test_root_without_prefix_returns_its_value():
    T, nq, nkv, hd = 8, 4, 2, 16
    q, kc, vc, kt, vt, par = _inputs(T, 0, nq, nkv, hd, seed=6)
    out = oracle.tree_attention64(q, kc, vc, kt, vt, par, 0)
    for h in range(nq):
        np.testing.assert_array_equal(out[0, h], vt[h // 2, 0])


def test_zero_query_gives_mean_of_visible_values():
    T, C, nq, nkv, hd = 12, 7, 2, 2, 8
    _, kc, vc, kt, vt, par = _inputs(T, C, nq, nkv, hd, seed=7)
    q = np.zeros((T, nq, hd))
    out = oracle.tree_attention64(q, kc, vc, kt, vt, par, C)
    for i in range(T):
        chain = []
        j = i
        while j >= 0:
            chain.append(j)
            j = int(par[j])
        for h in range(nq):
            vis = np.concatenate([vc[h, :C], vt[h, chain]], axis=0)
            np.testing.assert_allclose(out[i, h], vis.mean(axis=0), rtol=1e-13, atol=1e-14)


def test_dense_equals_loop_form():
    q, kc, vc, kt, vt, par = _inputs(20, 6, 4, 2, 8, seed=8, kind="RB")
    a = oracle.tree_attention64(q, kc, vc, kt, vt, par, 6)
    b = oracle.tree_attention_loop64(q, kc, vc, kt, vt, par, 6)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


def test_relabelling_permutes_outputs():
    T, C = 10, 4
    q, kc, vc, kt, vt, par = _inputs(T, C, 2, 1, 8, seed=9)
    # new order: a different topological order (children of the root visited in reverse)
    order = [0]
    def visit(n):
        for c in sorted([i for i in range(T) if par[i] == n], reverse=True):
            order.append(c)
            visit(c)
    visit(0)
    new_of = {old: new for new, old in enumerate(order)}
    par2 = np.array([-1] + [new_of[int(par[old])] for old in order[1:]], dtype=np.int32)
    out1 = oracle.tree_attention64(q, kc, vc, kt, vt, par, C)
    out2 = oracle.tree_attention64(q[order], kc, vc, kt[:, order], vt[:, order], par2, C)
    np.testing.assert_allclose(out2, out1[order], rtol=1e-13, atol=1e-14)
