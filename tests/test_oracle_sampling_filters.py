"""Pins for the oracle's filtering of target logits into probabilities (CPU).

[TRT] "non-greedy: rejection from the target distribution alone": the target's logits
at each tree node become probabilities under the request's temperature, top-k, top-p
and min-p.  Expected values come from:
  * closed forms: no filter is the plain softmax of logits / temperature (scipy);
    top-k is that softmax restricted to the k largest logits and renormalised;
    a temperature <= 0 or top_k = 1 puts all mass on the largest logit;
  * a worked example computed by hand from exp() values (top-p reaching its target
    inside the second token, min-p dropping the tail, top-k + top-p together,
    temperature 2);
  * tie rules: equal logits rank by token id, so top-k / top-p cut ties in token order;
  * invariants: the kept set is a prefix of the ranking, the output sums to 1, min-p
    keeps exactly the tokens whose softmax ratio to the best is >= min_p.
"""
import math

import numpy as np
import pytest
from scipy.special import softmax

from oracle import sampling as osm


def test_no_filter_is_the_softmax():
    rng = np.random.default_rng(0)
    for tau in (0.3, 1.0, 2.5):
        lg = rng.normal(0, 3, 500).astype(np.float32)
        got = osm.sampling_probs_row(lg, tau, 0, 1.0, 0.0)
        ref = softmax(lg.astype(np.float64) / np.float64(np.float32(tau)))
        np.testing.assert_allclose(got, ref, rtol=2e-6, atol=1e-30)
        assert abs(float(got.astype(np.float64).sum()) - 1.0) < 1e-5


@pytest.mark.parametrize("k", [1, 2, 7, 99])
def test_top_k_is_the_softmax_of_the_k_largest(k):
    rng = np.random.default_rng(k)
    lg = rng.normal(0, 2, 100).astype(np.float32)
    got = osm.sampling_probs_row(lg, 0.8, k, 1.0, 0.0)
    top = sorted(range(100), key=lambda v: (-float(lg[v]), v))[:k]
    ref = np.zeros(100)
    ref[top] = softmax(lg[top].astype(np.float64) / np.float64(np.float32(0.8)))
    np.testing.assert_allclose(got, ref, rtol=2e-6, atol=0)


def test_greedy_cases():
    lg = np.array([0.5, 3.0, -1.0, 3.0, 2.0], np.float32)   # the largest logit twice: token 1 wins
    for tau, k, p in ((0.0, 0, 1.0), (-1.0, 0, 1.0), (float("nan"), 0, 1.0), (1.0, 1, 1.0), (1.0, 0, 0.0),
                      (1.0, 0, -0.5)):
        got = osm.sampling_probs_row(lg, tau, k, p, 0.0)
        assert got.tolist() == [0.0, 1.0, 0.0, 0.0, 0.0], (tau, k, p)


def test_worked_example():
    # logits 2, 1, 0, -1 at temperature 1: weights 1, e^-1, e^-2, e^-3
    lg = np.array([2.0, 1.0, 0.0, -1.0], np.float32)
    w = [1.0, math.exp(-1), math.exp(-2), math.exp(-3)]
    W = sum(w)                                       # 1.5530
    # top_p 0.7: target 0.7 W = 1.0871; cumulative 1, 1.3679 -> two tokens kept
    got = osm.sampling_probs_row(lg, 1.0, 0, 0.7, 0.0)
    np.testing.assert_allclose(got, [w[0] / (w[0] + w[1]), w[1] / (w[0] + w[1]), 0, 0], rtol=1e-7)
    assert 0.7 * W > w[0] and w[0] + w[1] >= 0.7 * W
    # min_p 0.3 drops e^-2 = 0.135 and e^-3 (the same two survive)
    got = osm.sampling_probs_row(lg, 1.0, 0, 1.0, 0.3)
    np.testing.assert_allclose(got, [w[0] / (w[0] + w[1]), w[1] / (w[0] + w[1]), 0, 0], rtol=1e-7)
    # top_k 3 then top_p 0.95: target 0.95 (1 + e^-1 + e^-2) = 1.428 > 1.3679 -> all three
    got = osm.sampling_probs_row(lg, 1.0, 3, 0.95, 0.0)
    s3 = w[0] + w[1] + w[2]
    np.testing.assert_allclose(got, [w[0] / s3, w[1] / s3, w[2] / s3, 0], rtol=1e-7)
    # top_p 0.6: target 0.932 < 1 -> the best token alone
    assert osm.sampling_probs_row(lg, 1.0, 0, 0.6, 0.0).tolist() == [1.0, 0.0, 0.0, 0.0]
    # temperature 2: weights exp(-0.5 j)
    got = osm.sampling_probs_row(lg, 2.0, 0, 1.0, 0.0)
    w2 = [math.exp(-0.5 * j) for j in range(4)]
    np.testing.assert_allclose(got, np.array(w2) / sum(w2), rtol=1e-7)
    # min_p at exactly a weight's float32 value keeps it (>=)
    got = osm.sampling_probs_row(lg, 1.0, 0, 1.0, float(np.float32(math.exp(-1))))
    assert (got > 0).tolist() == [True, True, False, False]


def test_top_p_cut_counts_every_tail_weight():
    # Two tokens of weight 1 and 1000 tail tokens of weight ~1e-11 (logit ln 1e-11 at
    # temperature 1).  The exact total is 2 + 1000 w_t, so top_p 0.5 needs more than
    # the first token (1 < 0.5 (2 + 1000 w_t)) and keeps exactly two.  A top-p sum
    # that drops weights below some unit (e.g. 2^-33) would keep one.
    lt = np.float32(math.log(1e-11))
    lg = np.full(1002, lt, np.float32)
    lg[0] = lg[1] = 0.0
    w_t = float(np.float32(math.exp(float(lt))))
    assert 0 < w_t < 2.0 ** -33 and 1.0 < 0.5 * (2.0 + 1000 * w_t)
    for k in (0, 500):                       # the radix path (no top-k) and a top-k survivor list
        got = osm.sampling_probs_row(lg, 1.0, k, 0.5, 0.0)
        assert (got > 0).tolist() == [True, True] + [False] * 1000, k
        assert got[:2].tolist() == [0.5, 0.5]
    # with top_p exactly at a cumulative boundary the cut is inclusive (>=): four equal
    # weights, top_p 0.5 keeps two; the next float32 above 0.5 keeps three
    lg4 = np.zeros(4, np.float32)
    assert (osm.sampling_probs_row(lg4, 1.0, 0, 0.5, 0.0) > 0).tolist() == [True, True, False, False]
    above = float(np.nextafter(np.float32(0.5), np.float32(1.0)))
    assert (osm.sampling_probs_row(lg4, 1.0, 0, above, 0.0) > 0).tolist() == [True, True, True, False]
    # a subnormal weight still counts: 2 + w_s at top_p 0.5 keeps two, 2 alone keeps one
    lgs = np.array([0.0, 0.0, -100.0], np.float32)          # exp(-100) ~ 3.7e-44: a float32 subnormal
    ws = float(np.float32(math.exp(-100.0)))
    assert 0 < ws < 2.0 ** -126
    assert (osm.sampling_probs_row(lgs, 1.0, 0, 0.5, 0.0) > 0).tolist() == [True, True, False]
    assert (osm.sampling_probs_row(lgs[:2], 1.0, 0, 0.5, 0.0) > 0).tolist() == [True, False]


def test_ties_cut_in_token_order():
    lg = np.array([1.0, 2.0, 1.0, 2.0, 1.0, 0.0], np.float32)   # rank: 1, 3, 0, 2, 4, 5
    got = osm.sampling_probs_row(lg, 1.0, 3, 1.0, 0.0)
    assert (got > 0).tolist() == [True, True, False, True, False, False]
    np.testing.assert_allclose(got[[1, 3, 0]], softmax(np.array([2.0, 2.0, 1.0])), rtol=1e-7)
    # top_p inside the tie group at logit 1: weights 1, 1, e^-1 x3, e^-2;
    # target 0.8 W: 2 + e^-1 = 2.37 < 0.8 W = 2.49 <= 2 + 2e^-1 -> tokens 1, 3, 0, 2
    W = 2 + 3 * math.exp(-1) + math.exp(-2)
    assert 2 + math.exp(-1) < 0.8 * W <= 2 + 2 * math.exp(-1)
    got = osm.sampling_probs_row(lg, 1.0, 0, 0.8, 0.0)
    assert (got > 0).tolist() == [True, True, True, True, False, False]
    # -0.0 and +0.0 rank equal (token order decides)
    z = np.array([-0.0, 0.0, -5.0], np.float32)
    assert (osm.sampling_probs_row(z, 1.0, 1, 1.0, 0.0) > 0).tolist() == [True, False, False]


def test_special_logits():
    inf = np.inf
    # +inf logits share all the mass; NaN ranks as -inf
    got = osm.sampling_probs_row(np.array([1.0, inf, np.nan, inf], np.float32), 1.0, 0, 1.0, 0.0)
    assert got.tolist() == [0.0, 0.5, 0.0, 0.5]
    # an all -inf row is uniform
    got = osm.sampling_probs_row(np.full(4, -inf, np.float32), 1.0, 0, 1.0, 0.0)
    assert got.tolist() == [0.25] * 4
    got = osm.sampling_probs_row(np.full(4, -inf, np.float32), 1.0, 2, 1.0, 0.0)
    assert got.tolist() == [0.5, 0.5, 0.0, 0.0]


@pytest.mark.parametrize("seed", range(4))
def test_invariants(seed):
    rng = np.random.default_rng(100 + seed)
    V = 300
    lg = (rng.normal(0, 2, V) * (rng.random(V) < 0.9)).astype(np.float32)   # some exact zeros (ties)
    tau, k, p, m = 0.7 + seed * 0.3, [0, 50, 200, 299][seed], [1.0, 0.9, 0.5, 0.99][seed], [0, 0.01, 0, 0.2][seed]
    got = osm.sampling_probs_row(lg, tau, k, p, m)
    order = sorted(range(V), key=lambda v: (-float(lg[v]), v))
    kept = [v for v in order if got[v] > 0]
    assert kept == order[:len(kept)], "the kept set is a prefix of the ranking"
    assert abs(float(got.astype(np.float64).sum()) - 1.0) < 1e-5
    if k:
        assert len(kept) <= k
    if m:
        ratio = np.exp((lg.astype(np.float64) - lg.max()) / np.float64(np.float32(tau)))
        assert all(ratio[v] >= m * (1 - 1e-6) for v in kept)


def test_batch_rows_and_untouched_rows():
    rng = np.random.default_rng(5)
    B, T_max, V = 3, 4, 20
    lg = rng.normal(0, 1, (B, T_max, V)).astype(np.float32)
    out0 = np.full((B, T_max, V), -7.0, np.float32)
    res = osm.tree_sampling_probs(lg, [4, 2, 3], [0, 0, 1], [1.0, 0.5, 1.0], [0, 5, 0], [0.9, 1.0, 1.0],
                                  [0.0, 0.0, 0.1], out0)
    for b, T in ((0, 4), (1, 2), (2, 1)):       # request 2 has a bad status: its root row only
        assert (res[b, T:] == -7.0).all()
        for i in range(T):
            assert abs(float(res[b, i].astype(np.float64).sum()) - 1.0) < 1e-5
