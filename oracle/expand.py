"""Draft-tree expansion: the static deep-narrow template filled one level per draft step.

TEST INFRASTRUCTURE ONLY (see the package header).

[Review] §6.3-§6.4: SubSpec drafts a static token tree (k = 6 children per expanded
node, depth 48, [Review] §3.7) rather than EAGLE-2's dynamic one; [Summary]
"Approach": the draft's probabilities are sharpened at temperature 0.2 before the tree
is built. The pages do not spell out which nodes get expanded; the reading taken here
(the plain one the rest supports: a static node budget, EAGLE-style ranking by the
path's cumulative sharpened log-probability):

* The tree has T slots and is built in D steps (D = the depth). Before step 0 only the
  root (slot 0, cumulative score 0) exists; the frontier is {root}.
* Step s expands the frontier, the nodes added by step s - 1. A frontier node f with
  logits l gets its k children: the k largest entries of y = fp32(fp32(l) * fp32(1/t))
  (ties: lower token id), each child c scored cum[f] + (y[c] - logsumexp(y)), the
  path's sharpened log-probability.
* Of all children of the frontier, the B_s = ceil((T - n) / (D - s)) best (n = nodes so
  far; ties: lower frontier position, then lower child rank) are appended, in that
  order, at slots n, n + 1, ...: parent f, token c, score as above. They are the next
  frontier. After D steps all T slots are filled and the depth is D.

Every score here is fp64 (from the fp32 y); the device path keeps fp32 scores, so a
comparison takes the selection as valid where the two orders only differ on scores
closer than the fp32 rounding of the sums.
"""

import math

import numpy as np


def schedule(T, D):
    """Nodes appended by each of the D steps: B_s = ceil((T - n_s) / (D - s))."""
    if D < 1 or T - 1 < D:
        raise ValueError("need 1 <= D <= T - 1")
    out, n = [], 1
    for s in range(D):
        b = -(-(T - n) // (D - s))
        out.append(b)
        n += b
    return out


def sharpened(logits_row, inv_temp):
    """y = fp32(l * fp32(1/t)) (one fp32 rounding per element, no fused operation)."""
    return np.asarray(logits_row, dtype=np.float32) * np.float32(inv_temp)


def children(y, k):
    """The k largest entries of y, ties to the lower index: (token ids, log-probabilities)."""
    y64 = y.astype(np.float64)
    m = float(np.max(y64))
    lse = m + math.log(float(np.sum(np.exp(y64 - m))))
    order = np.lexsort((np.arange(len(y)), -y64))[:k]
    return order.astype(np.int32), y64[order] - lse


def expand_step(parents, tokens, cum, n, frontier, frontier_logits, inv_temp, k, B):
    """One expansion step; returns the new frontier (slot indices). parents / tokens /
    cum (length T, fp64 scores) are updated in place; n = nodes so far."""
    cands = []
    for r, f in enumerate(frontier):
        ids, lp = children(sharpened(frontier_logits[r], inv_temp), k)
        for rank in range(k):
            cands.append((-(cum[f] + lp[rank]), r, rank, f, int(ids[rank]), cum[f] + lp[rank]))
    cands.sort(key=lambda c: (c[0], c[1], c[2]))
    new = []
    for i, c in enumerate(cands[:B]):
        slot = n + i
        parents[slot] = c[3]
        tokens[slot] = c[4]
        cum[slot] = c[5]
        new.append(slot)
    return new


def expand_tree(root_token, T, D, logits_of, inv_temp, k, placeholder_parent=0):
    """The whole template: logits_of(step, parents, tokens, frontier) returns the
    frontier's logits rows. Unfilled slots hold (parent 0, the root's token)."""
    parents = np.full(T, placeholder_parent, dtype=np.int32)
    parents[0] = -1
    tokens = np.full(T, root_token, dtype=np.int32)
    cum = np.zeros(T, dtype=np.float64)
    frontier, n = [0], 1
    for s, b in enumerate(schedule(T, D)):
        lg = logits_of(s, parents.copy(), tokens.copy(), list(frontier))
        frontier = expand_step(parents, tokens, cum, n, frontier, lg, inv_temp, k, b)
        n += b
    return parents, tokens, cum
