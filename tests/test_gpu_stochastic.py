"""Stochastic tree verification on the device (ss_tree_accept_stochastic) against the
oracle's walk (oracle/stochastic.py) on seeded logits and uniforms. Accept / reject
decisions and the bonus draw are integers decided by floats: both sides decide in the same
precision (fp32 exponentials, fp64 after), so results must match exactly wherever the
decision is not closer to its boundary than summation-order rounding; every case checks
its margins first."""
import numpy as np
import pytest
import torch

from oracle import stochastic as st
from synth import gen
from tests.gpu_util import host, to_dev

pytestmark = pytest.mark.gpu

bq = pytest.importorskip("bit_quantized_draft_amd")


def _margins(parents, tokens, dl, tl, inv_td, inv_tt, u, ub):
    """Smallest relative distance of any decision of the oracle's walk from its boundary."""
    T = len(parents)
    kids = [[] for _ in range(T)]
    for i in range(1, T):
        kids[int(parents[i])].append(i)
    worst, cur = np.inf, 0
    while True:
        P = st.probs(tl[cur], inv_tt)
        Q = st.probs(dl[cur], inv_td)
        P0, nxt = P, None
        for c in kids[cur]:
            x = int(tokens[c])
            a, b = u[c] * Q[x], P[x]
            if max(a, b) > 0:
                worst = min(worst, abs(a - b) / max(a, b))
            if a < b:
                nxt = c
                break
            R = np.maximum(P - Q, 0.0)
            P = R / R.sum() if R.sum() > 0 else P0
        if nxt is None:
            c = np.cumsum(P)
            thr = ub[cur] * c[-1]
            worst = min(worst, np.min(np.abs(c - thr)) / c[-1])
            return worst
        cur = nxt


def _case(T, kind, V, seed, equal=False, sharp=0.2, temp=0.6):
    rng = np.random.default_rng(seed)
    par = gen.tree_parents(T, kind, seed=seed)
    tok = gen.tree_tokens(par, V, seed=seed)
    tl = rng.normal(0, 2.0, (T, V)).astype(np.float32)
    dl = tl.copy() if equal else (tl + rng.normal(0, 0.7, (T, V))).astype(np.float32)
    # make some children likely under both models so the walk goes deep
    for i in range(1, T):
        if rng.random() < 0.7:
            tl[par[i], tok[i]] += 6.0
            dl[par[i], tok[i]] += 6.0
    u = rng.random(T)
    ub = rng.random(T)
    inv_td = float(np.float32(1.0) / np.float32(sharp))
    inv_tt = float(np.float32(1.0) / np.float32(temp))
    return par, tok, dl, tl, inv_td, inv_tt, u, ub


@pytest.mark.parametrize("T,kind,V,seed,equal", [(64, "CB", 2000, 1, False), (17, "R", 50, 2, False),
                                                 (256, "RB", 3000, 3, False), (48, "CB", 500, 4, True),
                                                 (1, "R", 100, 5, False)])
def test_stochastic_walk_matches_oracle(T, kind, V, seed, equal):
    print(f"stochastic accept T={T} tree={kind} V={V} draft==target={equal}", flush=True)
    par, tok, dl, tl, inv_td, inv_tt, u, ub = _case(T, kind, V, seed, equal)
    assert _margins(par, tok, dl, tl, inv_td, inv_tt, u, ub) > 1e-9, "a decision sits on its boundary"
    path_o, L_o, bonus_o = st.accept_stochastic(par, tok, dl, tl, inv_td, inv_tt, u, ub)
    path, ln, bonus = bq.tree_accept_stochastic(to_dev(par), to_dev(tok), to_dev(dl), to_dev(tl), inv_td, inv_tt,
                                                torch.from_numpy(u).cuda(), torch.from_numpy(ub).cuda())
    torch.cuda.synchronize()
    assert int(host(ln)[0]) == L_o
    got = host(path)
    assert list(got[:L_o]) == path_o[1:] and np.all(got[L_o:] == -1)
    assert int(host(bonus)[0]) == bonus_o
    if equal:
        assert L_o >= 1


def test_out_of_range_token_is_rejected_without_reading():
    par, tok, dl, tl, inv_td, inv_tt, u, ub = _case(8, "chain", 64, 6)
    tok = tok.copy()
    tok[1] = 64           # the root's only child carries an id outside [0, V)
    path, ln, bonus = bq.tree_accept_stochastic(to_dev(par), to_dev(tok), to_dev(dl), to_dev(tl), inv_td, inv_tt,
                                                torch.from_numpy(np.zeros(8)).cuda(), torch.from_numpy(ub).cuda())
    torch.cuda.synchronize()
    assert int(host(ln)[0]) == 0 and 0 <= int(host(bonus)[0]) < 64
