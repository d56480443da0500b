"""Pins for the oracle's tree rejection sampling (target distribution only), CPU.

Expected values come from:
  * the property the method exists for ([HB] exercise "trees when sampling"; [TRT]
    target-only rejection sampling): the emitted tokens follow the target
    distribution -- checked by Monte Carlo on tiny trees at the first and the second
    emitted token, against the target rows themselves;
  * the greedy limit: with one-hot target rows, rejection sampling is the greedy walk
    (pinned on its own) for any uniforms;
  * special cases: a point mass on a child is always accepted, children without mass
    never are, the depth cap and a bad status sample the correction at the current
    node, and u = 0 takes the first child with mass.
"""
import numpy as np
import pytest

from oracle import tree as ot
from workloads import gen


def tiny_tree():
    # node 0 (root) -> children 1 (token 2), 2 (token 0), 3 (token 4); node 1 -> children 4 (token 1), 5 (token 3)
    toks = [7, 2, 0, 4, 1, 3]
    par = [-1, 0, 0, 0, 1, 1]
    return toks, par


def test_first_and_second_token_follow_the_target():
    V = 5
    toks, par = tiny_tree()
    rng = np.random.default_rng(11)
    probs = rng.dirichlet(np.ones(V), size=6)
    n = 120_000
    first = np.zeros(V)
    second_after_2 = np.zeros(V)
    n_after_2 = 0
    for _ in range(n):
        u = rng.random(6)
        a, path, bonus = ot.accept_sample(toks, par, 6, probs, u, 0, dcap=3)
        emitted = [toks[c] for c in path[1:a + 1]] + [bonus]
        first[emitted[0]] += 1
        if emitted[0] == 2 and len(emitted) > 1:   # token 2 = node 1, whose own row is probs[1]
            second_after_2[emitted[1]] += 1
            n_after_2 += 1
    tol = 5 * np.sqrt(0.25 / n)
    np.testing.assert_allclose(first / n, probs[0], atol=tol)
    tol2 = 5 * np.sqrt(0.25 / n_after_2)
    np.testing.assert_allclose(second_after_2 / n_after_2, probs[1], atol=tol2)


@pytest.mark.parametrize("seed", range(6))
def test_one_hot_targets_reduce_to_the_greedy_walk(seed):
    w = gen.make_custom(cfg_id=1100 + seed, B=4, mode="given", given_sizes=[1, 9, 33, 64], given_depth=6, V=40,
                        P=10, accept_prob=0.8)
    tp = gen.synthetic_target_predict(w, w.given_tokens, w.given_parents, w.given_size)
    rng = np.random.default_rng(seed)
    for b in range(w.B):
        onehot = np.zeros((w.T_max, w.V))
        onehot[np.arange(w.T_max), tp[b] % w.V] = 1.0
        g = ot.accept_walk(list(w.given_tokens[b]), list(w.given_parents[b]), int(w.given_size[b]), list(tp[b] % w.V),
                           0, w.dcap)
        s = ot.accept_sample(list(w.given_tokens[b]), list(w.given_parents[b]), int(w.given_size[b]), onehot,
                             rng.random(w.T_max), 0, w.dcap)
        assert s[0] == g[0] and list(s[1]) == list(g[1]) and s[2] == g[2]


def test_special_cases():
    toks, par = tiny_tree()
    V = 5
    probs = np.full((6, V), 0.2)
    # a point mass on child 2's token (0) at the root: accepted for any draw
    pm = probs.copy()
    pm[0] = 0.0
    pm[0, 0] = 1.0
    a, path, bonus = ot.accept_sample(toks, par, 6, pm, [0.0] + [0.999] * 5, 0, dcap=3)
    assert path[:2] == [0, 2] and a == 1
    # no mass on any child's token at the root: never accepted, the correction comes from
    # the root row with nothing removed
    nm = probs.copy()
    nm[0] = [0.0, 0.5, 0.0, 0.5, 0.0]
    a, path, bonus = ot.accept_sample(toks, par, 6, nm, [0.25] + [0.0] * 5, 0, dcap=3)
    assert a == 0 and bonus == 1
    a, path, bonus = ot.accept_sample(toks, par, 6, nm, [0.75] + [0.0] * 5, 0, dcap=3)
    assert a == 0 and bonus == 3
    # u = 0 takes the first child with mass
    a, path, bonus = ot.accept_sample(toks, par, 6, probs, [0.5] + [0.0] * 5, 0, dcap=1)
    assert a == 1 and path[:2] == [0, 1]
    # depth cap 1 stops at node 1: its correction is sampled from its full row (u = 0.5 -> token 2)
    assert bonus == 2
    # dcap 0 and a bad status: the correction is sampled at the root
    a, path, bonus = ot.accept_sample(toks, par, 6, probs, [0.9] + [0.0] * 5, 0, dcap=0)
    assert a == 0 and path == [0] and bonus == 4
    a, path, bonus = ot.accept_sample(toks, par, 6, probs, [0.1] + [0.0] * 5, ot.ST_PARENTS, dcap=3)
    assert a == 0 and path[0] == 0 and bonus == 0
    # every child rejected at the root: tokens 2, 0, 4 removed, the residual is {1, 3}
    a, path, bonus = ot.accept_sample(toks, par, 6, probs, [0.6] + [0.999] * 5, 0, dcap=3)
    assert a == 0 and bonus == 3
    a, path, bonus = ot.accept_sample(toks, par, 6, probs, [0.4] + [0.999] * 5, 0, dcap=3)
    assert a == 0 and bonus == 1
