"""Pins of the stochastic tree verification oracle (oracle/stochastic.py): the output token
distribution equals the target's (speculative sampling's defining property, checked
statistically with i.i.d. draft children), the degenerate cases (draft = target accepts
every first child; a zero-probability token is never accepted), the inverse-CDF draw
against numpy's searchsorted on hand cases, and the residual rule against a direct
computation."""
import numpy as np
import pytest

from oracle import stochastic as st


def _two_level(V, k, rng, t_logits, d_logits, inv_tt, inv_td):
    """Root with k children whose tokens are i.i.d. draws from the draft's distribution."""
    Q = st.probs(d_logits, inv_td)
    toks = rng.choice(V, size=k, p=Q)
    parents = np.array([-1] + [0] * k)
    tokens = np.array([0] + list(toks))
    T = k + 1
    dl = np.tile(d_logits, (T, 1)).astype(np.float32)
    tl = np.tile(t_logits, (T, 1)).astype(np.float32)
    u = rng.random(T)
    ub = rng.random(T)
    path, L, bonus = st.accept_stochastic(parents, tokens, dl, tl, inv_td, inv_tt, u, ub)
    return int(tokens[path[1]]) if L >= 1 else bonus


@pytest.mark.parametrize("k", [1, 2, 4])
def test_first_token_follows_the_target_distribution(k):
    V = 6
    rng = np.random.default_rng(k)
    t_logits = np.array([1.0, 0.2, -0.5, 2.0, 0.0, -1.0], np.float32)
    d_logits = np.array([0.5, 1.5, 0.0, 0.3, -0.2, 0.8], np.float32)
    inv_tt, inv_td = 1.0 / 0.6, 1.0 / 0.2
    P = st.probs(t_logits, inv_tt)
    n = 20000
    counts = np.zeros(V)
    for _ in range(n):
        counts[_two_level(V, k, rng, t_logits, d_logits, inv_tt, inv_td)] += 1
    sigma = np.sqrt(n * P * (1 - P))
    assert np.all(np.abs(counts - n * P) <= 4 * sigma + 1), (counts / n, P)


def test_draft_equal_to_target_accepts_every_first_child():
    rng = np.random.default_rng(0)
    T, V = 30, 40
    parents = np.array([-1] + [int(rng.integers(0, i)) for i in range(1, T)])
    tokens = rng.integers(0, V, T)
    lg = rng.normal(0, 1, (T, V)).astype(np.float32)
    u = rng.random(T) * 0.999
    path, L, _ = st.accept_stochastic(parents, tokens, lg, lg, 2.0, 2.0, u, rng.random(T))
    # every step takes the lowest-index child (u * Q < P holds when Q == P and u < 1)
    cur, want = 0, [0]
    while True:
        kids = [i for i in range(1, T) if parents[i] == cur]
        if not kids:
            break
        cur = kids[0]
        want.append(cur)
    assert path == want and L == len(want) - 1


def test_token_outside_the_target_support_is_never_accepted():
    V = 5
    tl = np.array([0, 0, -1e30, 0, 0], np.float32)    # token 2 has target probability 0
    dl = np.array([0, 0, 5, 0, 0], np.float32)
    parents, tokens = np.array([-1, 0]), np.array([0, 2])
    for u in (0.0, 1e-9, 0.5):
        path, L, bonus = st.accept_stochastic(parents, tokens, np.stack([dl, dl]), np.stack([tl, tl]), 1.0, 1.0,
                                              np.array([0.5, u]), np.array([0.3, 0.3]))
        assert L == 0 and bonus != 2


def test_inverse_cdf_hand_cases():
    p = np.array([0.1, 0.2, 0.3, 0.4])
    assert st.sample_inverse_cdf(p, 0.0) == 0
    assert st.sample_inverse_cdf(p, 0.0999) == 0
    assert st.sample_inverse_cdf(p, 0.1) == 1          # the cumulative must exceed u
    assert st.sample_inverse_cdf(p, 0.55) == 2
    assert st.sample_inverse_cdf(p, 0.9999999) == 3
    assert st.sample_inverse_cdf(np.array([0.0, 0.0, 2.0]), 0.5) == 2   # unnormalised weights


def test_rejection_uses_the_residual_for_the_bonus():
    # one child, rejected: the bonus comes from norm(max(P - Q, 0)), computed here directly
    V = 4
    tl = np.log(np.array([0.4, 0.3, 0.2, 0.1], np.float32))
    dl = np.log(np.array([0.1, 0.6, 0.2, 0.1], np.float32))
    parents, tokens = np.array([-1, 0]), np.array([0, 1])   # child token 1: P/Q = 0.5
    res = np.array([0.3, 0.0, 0.0, 0.0])                      # max(P - Q, 0), normalised: all on 0
    path, L, bonus = st.accept_stochastic(parents, tokens, np.stack([dl, dl]), np.stack([tl, tl]), 1.0, 1.0,
                                          np.array([0.0, 0.9]), np.array([0.99, 0.99]))
    assert L == 0 and bonus == 0 and res.argmax() == 0
    path, L, _ = st.accept_stochastic(parents, tokens, np.stack([dl, dl]), np.stack([tl, tl]), 1.0, 1.0,
                                      np.array([0.0, 0.49]), np.array([0.5, 0.5]))
    assert L == 1 and path == [0, 1]
