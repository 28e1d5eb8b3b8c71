"""Draft-tree expansion on the device (ss_tree_expand_init / ss_draft_select / ss_tree_expand)
against the oracle's expansion (oracle/expand.py) on seeded logits. Each step's frontier
logits come from a seeded table indexed by the frontier node's token, so both sides see the
same rows; the host reads the device's frontier between steps only to build those rows.
The parent and token arrays must match exactly where the oracle's choice is unique (every
step's margin between the last appended and the first rejected candidate is checked to be
far above fp32 rounding, so the order is unique); the path scores match to fp32 precision."""
import numpy as np
import pytest
import torch

from oracle import expand as ex
from tests.gpu_util import host, to_dev

pytestmark = pytest.mark.gpu

bq = pytest.importorskip("bit_quantized_draft_amd")


def _table(V, rows, seed):
    return np.random.default_rng(seed).normal(0, 2.0, (rows, V)).astype(np.float32)


def _margins(T, D, logits_of, inv_t, k):
    """Smallest gap, over the steps, between the last chosen and the first rejected child."""
    par = np.zeros(T, np.int32); par[0] = -1
    tok = np.zeros(T, np.int32)
    cum = np.zeros(T)
    frontier, n, worst = [0], 1, np.inf
    for s, b in enumerate(ex.schedule(T, D)):
        rows = logits_of(s, par.copy(), tok.copy(), frontier)
        sc = []
        for r, f in enumerate(frontier):
            _, lp = ex.children(ex.sharpened(rows[r], inv_t), k)
            sc += [cum[f] + v for v in lp]
        sc = sorted(sc, reverse=True)
        if len(sc) > b:
            worst = min(worst, sc[b - 1] - sc[b])
        frontier = ex.expand_step(par, tok, cum, n, frontier, rows, inv_t, k, b)
        n += b
    return worst


@pytest.mark.parametrize("T,D,R,k,V,temp,seed", [(64, 48, 2, 6, 3000, 0.2, 1),   # the 7B template
                                                 (12, 5, 3, 3, 50, 0.6, 2),
                                                 (20, 19, 1, 6, 4096, 0.2, 3)])  # a chain of single nodes
def test_expansion_matches_oracle(T, D, R, k, V, temp, seed):
    print(f"expand T={T} D={D} R={R} k={k} V={V} t={temp}", flush=True)
    table = _table(V, 97, seed)
    inv_t = float(np.float32(1.0) / np.float32(temp))

    def logits_of(step, parents, tokens, frontier):
        return np.stack([table[(int(tokens[f]) * 31 + step) % len(table)] for f in frontier])

    assert _margins(T, D, logits_of, inv_t, k) > 1e-3, "seeded case has a near tie: pick another seed"
    root = 7
    ref_par, ref_tok, ref_cum = ex.expand_tree(root, T, D, logits_of, inv_t, k)

    dev = torch.device("cuda:0")
    st = bq.TreeState(T, D, R, k, dev)
    bq.tree_expand_init(st, root)
    children = torch.empty((R, k), dtype=torch.int32, device=dev)
    for s in range(D + 2):   # two calls past the last step must change nothing
        torch.cuda.synchronize()
        meta = host(st.meta)
        fr = list(host(st.frontier)[:max(1, meta[1])])
        rows = logits_of(s, host(st.parents), host(st.tokens), fr)
        rows = np.concatenate([rows, np.repeat(rows[:1], R - len(fr), 0)]) if len(fr) < R else rows
        lg = to_dev(np.ascontiguousarray(rows, dtype=np.float32))
        bq.draft_select(lg, None, inv_t, k, out=children)
        bq.tree_expand(st, lg, children, inv_t)
    torch.cuda.synchronize()
    meta = host(st.meta)
    assert list(meta[:3]) == [T, ex.schedule(T, D)[-1], D]
    assert np.array_equal(host(st.parents), ref_par)
    assert np.array_equal(host(st.tokens), ref_tok)
    assert np.allclose(host(st.cum).astype(np.float64), ref_cum, rtol=1e-5, atol=1e-4)
