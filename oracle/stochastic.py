"""Stochastic tree verification: multi-round speculative sampling over the draft tree.

TEST INFRASTRUCTURE ONLY (see the package header).

[Review] §3.6 and §6.2: with target sampling (temperature 0.6) SubSpec keeps the target's
output distribution exact by speculative sampling with correction (Leviathan et al.);
[Review] §6.3: the tree's candidates are verified in one target pass. Reading (the pages
do not spell the tree rule out; this is the plain multi-round form of the same test):

* P_u = softmax(y_t) with y_t = fp32(target_logits[u] * fp32(1 / t_target)), and
  Q_u = softmax(y_d) with y_d = fp32(draft_logits[u] * fp32(1 / t_draft)): the target's
  and the draft's distributions at node u. Precision (the decisions below are taken in
  it on both sides): e(v) = fp32 exp of fp32(y(v) - max y), widened to fp64; the
  normalizer and every later quantity in fp64.
* From the root, at node u the children c (in index order) are tried: child c with
  token x is accepted iff uniforms[c] * Q_u(x) < P(x) (u < P / Q; strict, so a token the
  target cannot emit is never accepted), P the current residual (P_u at first); then the
  walk moves to c. A rejection replaces P by max(P - Q_u, 0)
  renormalized and tries the next child.
* When no child is accepted (or u has none), the bonus token is drawn from the current
  P by inverse CDF with bonus_uniforms[u]: the lowest x whose cumulative P exceeds
  bonus_uniforms[u] (sums in index order). If P has no mass left it is P_u.
* Outputs as the greedy walk: path (root first), L = accepted draft nodes, bonus.

The random numbers are inputs (uniform on [0, 1)), so the result is a function of them.
"""

import numpy as np


def probs(logits_row, inv_temp):
    y = np.asarray(logits_row, dtype=np.float32) * np.float32(inv_temp)
    d = (y - y.max()).astype(np.float32)
    e = np.exp(d).astype(np.float64)
    return e / e.sum()


def sample_inverse_cdf(p, u):
    """Lowest index x with sum(p[0..x]) > u * sum(p) (sums in index order)."""
    c = np.cumsum(p)
    x = int(np.searchsorted(c, u * c[-1], side="right"))
    return min(x, len(p) - 1)


def accept_stochastic(parents, tokens, draft_logits, target_logits, inv_t_draft, inv_t_target, uniforms,
                      bonus_uniforms):
    parents = np.asarray(parents)
    T = len(parents)
    kids = [[] for _ in range(T)]
    for i in range(1, T):
        kids[int(parents[i])].append(i)
    path, cur = [0], 0
    while True:
        P = probs(target_logits[cur], inv_t_target)
        Q = probs(draft_logits[cur], inv_t_draft)
        P0, nxt = P, None
        for c in kids[cur]:
            x = int(tokens[c])
            if uniforms[c] * Q[x] < P[x]:
                nxt = c
                break
            R = np.maximum(P - Q, 0.0)
            s = R.sum()
            P = R / s if s > 0 else P0
        if nxt is None:
            return path, len(path) - 1, sample_inverse_cdf(P, bonus_uniforms[cur])
        path.append(nxt)
        cur = nxt
