"""Tree-masked grouped-query attention over the KV cache shared with the target.

TEST INFRASTRUCTURE ONLY (see the package header).

[Review] §4.1 and [Summary] "Approach": the draft shares the target's KV cache, so
draft and target attend over the same committed context; [Review] §6.3: each tree
node sees its own root path. Query i of head h attends to every committed prefix
key 0..C-1 and to the tree keys of i's ancestors and itself, with scaled
dot-product softmax (scale 1/sqrt(hd) unless given). Query head h reads KV head
h // (nq / nkv). Reading: the prefix is never masked.
"""

import numpy as np

from .tree import tree_mask


def _ancestor_bool(parents) -> np.ndarray:
    m = tree_mask(parents)
    T = len(parents)
    out = np.zeros((T, T), dtype=bool)
    for i in range(T):
        for j in range(T):
            out[i, j] = bool((int(m[i, j // 64]) >> (j % 64)) & 1)
    return out


def tree_attention64(q, k_cache, v_cache, k_tree, v_tree, parents, C, sm_scale=None):
    """Dense masked form.

    q [T][nq][hd]; k_cache, v_cache [nkv][>=C][hd] (first C rows used);
    k_tree, v_tree [nkv][T][hd]; all fp64 (or exactly convertible). Returns fp64 [T][nq][hd].
    """
    q = np.asarray(q, dtype=np.float64)
    T, nq, hd = q.shape
    nkv = k_tree.shape[0]
    grp = nq // nkv
    scale = (1.0 / np.sqrt(hd)) if sm_scale is None else float(sm_scale)
    vis = _ancestor_bool(parents)                          # [T][T]
    out = np.zeros((T, nq, hd), dtype=np.float64)
    for kv in range(nkv):
        K = np.concatenate([np.asarray(k_cache[kv, :C], np.float64),
                            np.asarray(k_tree[kv], np.float64)], axis=0)
        V = np.concatenate([np.asarray(v_cache[kv, :C], np.float64),
                            np.asarray(v_tree[kv], np.float64)], axis=0)
        allowed = np.concatenate([np.ones((T, C), dtype=bool), vis], axis=1)
        for h in range(kv * grp, (kv + 1) * grp):
            S = (q[:, h, :] @ K.T) * scale                  # [T][C+T]
            S = np.where(allowed, S, -np.inf)
            S = S - S.max(axis=1, keepdims=True)
            P = np.exp(S)
            P /= P.sum(axis=1, keepdims=True)
            out[:, h, :] = P @ V
    return out


def tree_attention_loop64(q, k_cache, v_cache, k_tree, v_tree, parents, C, sm_scale=None):
    """Per-query form: walk each node's ancestor chain explicitly, then a plain softmax loop."""
    q = np.asarray(q, dtype=np.float64)
    T, nq, hd = q.shape
    nkv = k_tree.shape[0]
    grp = nq // nkv
    scale = (1.0 / np.sqrt(hd)) if sm_scale is None else float(sm_scale)
    out = np.zeros((T, nq, hd), dtype=np.float64)
    for i in range(T):
        chain = []
        j = i
        while j >= 0:
            chain.append(j)
            j = int(parents[j])
        for h in range(nq):
            kv = h // grp
            keys = [np.asarray(k_cache[kv, c], np.float64) for c in range(C)] + \
                   [np.asarray(k_tree[kv, j], np.float64) for j in chain]
            vals = [np.asarray(v_cache[kv, c], np.float64) for c in range(C)] + \
                   [np.asarray(v_tree[kv, j], np.float64) for j in chain]
            s = [float(np.dot(q[i, h], kk)) * scale for kk in keys]
            m = max(s)
            e = [np.exp(x - m) for x in s]
            tot = sum(e)
            acc = np.zeros(hd)
            for w, vv in zip(e, vals):
                acc += (w / tot) * vv
            out[i, h] = acc
    return out
