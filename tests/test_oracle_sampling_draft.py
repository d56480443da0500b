"""Pins for the oracle's tree rejection sampling with the drafter's distribution (CPU).

[HB] exercise "trees when sampling": children accepted with min(1, p(x)/q(x)), the
target replaced by norm(max(0, p - q)) after a rejection, q adjusted to the way the
candidates were drawn, the correction drawn from the last residual.  Expected values
come from:
  * the property the rule exists for: when a node's candidates really are drawn from
    q -- independently (q kept) or without replacement (rejected token removed from
    q) -- the first emitted token follows the target row p (Monte Carlo, both modes,
    several candidate counts), and so does the second one below an accepted child;
  * reductions: with q the point mass on a chain node's only child's token the rule
    is the target-only rejection sampling (tree.accept_sample, pinned on its own);
    with one-hot target rows it is the greedy walk (tree.accept_walk) for any q;
  * special cases: q = p accepts the first child that has target mass; a candidate
    with no draft mass but target mass is always accepted; no target mass anywhere
    gives the row's best token.
"""
import numpy as np
import pytest

from oracle import sampling as osm
from oracle import tree as ot
from workloads import gen


def _draw_children(rng, q, m, without_replacement):
    if without_replacement:
        return list(rng.choice(len(q), size=m, replace=False, p=q))
    return list(rng.choice(len(q), size=m, replace=True, p=q))


@pytest.mark.parametrize("without_replacement,m", [(True, 1), (True, 3), (False, 2), (False, 4)])
def test_first_token_follows_the_target(without_replacement, m):
    V = 5
    rng = np.random.default_rng(7 + m + 10 * without_replacement)
    p = rng.dirichlet(np.ones(V))
    q = rng.dirichlet(np.ones(V) * 0.7)
    n = 40_000
    counts = np.zeros(V)
    par = [-1] + [0] * m
    probs = np.stack([p] * (m + 1))
    qs = np.stack([q] * (m + 1))
    for _ in range(n):
        toks = [9] + _draw_children(rng, q, m, without_replacement)
        u = rng.random(m + 1)
        a, path, bonus = osm.accept_sample_draft(toks, par, m + 1, probs, qs, u, 0, 1, without_replacement)
        counts[toks[path[1]] if a else bonus] += 1
    tol = 5 * np.sqrt(0.25 / n)
    np.testing.assert_allclose(counts / n, p, atol=tol)


def test_second_token_follows_the_target_below_an_accepted_child():
    # root -> 2 candidates (without replacement from q0); each candidate c -> 2
    # candidates from q_c.  The token after the first one follows p_c.
    V = 4
    rng = np.random.default_rng(21)
    p = rng.dirichlet(np.ones(V), size=3)
    q = rng.dirichlet(np.ones(V), size=3)
    n = 40_000
    second = np.zeros(V)
    n_second = 0
    par = [-1, 0, 0, 1, 1, 2, 2]
    for _ in range(n):
        t1 = _draw_children(rng, q[0], 2, True)
        t3 = _draw_children(rng, q[1], 2, True)
        t5 = _draw_children(rng, q[2], 2, True)
        toks = [9] + t1 + t3 + t5
        u = rng.random(7)
        a, path, bonus = osm.accept_sample_draft(toks, par, 7, p[[0, 1, 2, 0, 0, 0, 0]], q[[0, 1, 2, 0, 0, 0, 0]], u,
                                                 0, 2, True)
        if a >= 1 and path[1] == 1:           # node 1 accepted: the next token comes from p[1]
            nxt = toks[path[2]] if a >= 2 else bonus
            second[nxt] += 1
            n_second += 1
    tol = 5 * np.sqrt(0.25 / n_second)
    np.testing.assert_allclose(second / n_second, p[1], atol=tol)


@pytest.mark.parametrize("seed", range(4))
def test_point_mass_draft_on_chains_is_target_only_sampling(seed):
    rng = np.random.default_rng(seed)
    T, V = 8, 30
    par = [-1] + list(range(T - 1))                      # a chain
    toks = [3] + list(rng.integers(0, V, T - 1))
    p = rng.dirichlet(np.ones(V) * 0.3, size=T)
    for i in range(T - 1):                               # make acceptance likely somewhere
        if rng.random() < 0.5:
            p[i] = 0.1 * p[i]
            p[i, toks[i + 1]] += 0.9
    q = np.zeros((T, V))
    for i in range(T - 1):
        q[i, toks[i + 1]] = 1.0
    for trial in range(20):
        u = rng.random(T)
        for wr in (True, False):
            d = osm.accept_sample_draft(toks, par, T, p, q, u, 0, 6, wr)
            t = ot.accept_sample(toks, par, T, p, u, 0, 6)
            assert d[0] == t[0] and list(d[1]) == list(t[1]) and d[2] == t[2]


@pytest.mark.parametrize("seed", range(4))
def test_one_hot_targets_are_the_greedy_walk(seed):
    w = gen.make_custom(cfg_id=1300 + seed, B=4, mode="given", given_sizes=[1, 9, 33, 64], given_depth=6, V=40,
                        P=10, accept_prob=0.8)
    tp = gen.synthetic_target_predict(w, w.given_tokens, w.given_parents, w.given_size)
    rng = np.random.default_rng(seed)
    for b in range(w.B):
        onehot = np.zeros((w.T_max, w.V))
        onehot[np.arange(w.T_max), tp[b] % w.V] = 1.0
        q = rng.dirichlet(np.ones(w.V), size=w.T_max) * (rng.random((w.T_max, 1)) < 0.9)   # some q rows all zero
        g = ot.accept_walk(list(w.given_tokens[b]), list(w.given_parents[b]), int(w.given_size[b]), list(tp[b] % w.V),
                           0, w.dcap)
        for wr in (True, False):
            s = osm.accept_sample_draft(list(w.given_tokens[b]), list(w.given_parents[b]), int(w.given_size[b]),
                                        onehot, q, rng.random(w.T_max), 0, w.dcap, wr)
            assert s[0] == g[0] and list(s[1]) == list(g[1]) and s[2] == g[2]


def test_special_cases():
    toks = [7, 2, 0, 4]
    par = [-1, 0, 0, 0]
    V = 5
    p = np.array([[0.1, 0.2, 0.3, 0.0, 0.4]] * 4)
    # q = p: the first child with target mass is accepted for any draw below 1
    a, path, _ = osm.accept_sample_draft(toks, par, 4, p, p, [0.5, 0.999, 0.999, 0.999], 0, 1, True)
    assert a == 1 and path[:2] == [0, 1]
    # a candidate without draft mass but with target mass is always accepted
    q = np.array([[0.0, 0.5, 0.0, 0.5, 0.0]] * 4)
    a, path, _ = osm.accept_sample_draft(toks, par, 4, p, q, [0.5, 0.999, 0.999, 0.999], 0, 1, True)
    assert a == 1 and path[1] == 1
    # no target mass on any child (tokens 2, 0, 4): all rejected.  The first rejection
    # subtracts q (all on token 2, where p is 0) and empties Q; R stays p, so the
    # correction with u0 = 0.5 (target 0.3 of 0.6) is token 3
    p2 = np.array([[0.0, 0.2, 0.0, 0.4, 0.0]] * 4)
    q2 = np.array([[0.0, 0.0, 1.0, 0.0, 0.0]] * 4)
    a, path, bonus = osm.accept_sample_draft(toks, par, 4, p2, q2, [0.5, 0.1, 0.1, 0.1], 0, 1, True)
    assert a == 0 and bonus == 3
    # the residual removes what q covers: p = (0.5, 0.5) on tokens 1, 3, q = (0.5, 0.5)
    # on tokens 2, 3 and a child with token 2 (no target mass) -> rejected;
    # R = max(0, p - q) = 0.5 on token 1 only, whatever u0
    p3 = np.array([[0.0, 0.5, 0.0, 0.5, 0.0]] * 2)
    q3 = np.array([[0.0, 0.0, 0.5, 0.5, 0.0]] * 2)
    for u0 in (0.01, 0.99):
        a, path, bonus = osm.accept_sample_draft([7, 2], [-1, 0], 2, p3, q3, [u0, 0.3], 0, 1, False)
        assert a == 0 and bonus == 1
    # no target mass at all: the row's best token (token 0 on an all-zero row)
    a, path, bonus = osm.accept_sample_draft(toks, par, 4, np.zeros((4, V)), q2, [0.5, 0.1, 0.1, 0.1], 0, 1, True)
    assert a == 0 and bonus == 0
    # bad status and depth cap 0: the correction from the root's full row
    for st, cap in ((ot.ST_PARENTS, 3), (0, 0)):
        a, path, bonus = osm.accept_sample_draft(toks, par, 4, p, p, [0.2, 0.0, 0.0, 0.0], st, cap, True)
        assert a == 0 and path[0] == 0 and bonus == 1    # cumulative 0.1, 0.3: the first above 0.2
