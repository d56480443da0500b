"""Pins for the oracle's layer-by-layer dynamic build and its fused log-softmax (CPU).

Expected values come from:
  * the batch build (pinned on its own in test_oracle_tree.py): fed the same log-prob
    rows one layer at a time, the layered build gives the same tree bit for bit;
  * brute force over whole rows: each layer's frontier is the K best of all K*V
    (slot, token) extensions of the previous frontier (the joint pruning of the
    EAGLE v2 walkthrough's topK_generate), found by sorting every extension;
  * scipy's log_softmax (an independent library routine) and closed forms for the
    log-softmax of raw logits (a constant row gives -log V; exp of a row sums to 1).
"""
import math

import numpy as np
import pytest
from scipy.special import log_softmax

from oracle import tree as ot
from workloads import gen


def layers_of(rows, K, D):
    """[1 + D*K][V] rows -> [root row] + D blocks of K rows."""
    return [rows[:1]] + [rows[1 + (l - 1) * K:1 + l * K] for l in range(1, D + 1)]


@pytest.mark.parametrize("K,D,TT,peaked", [(10, 6, 60, False), (8, 5, 48, False), (4, 3, 40, True),
                                           (1, 6, 6, False), (3, 0, 2, False), (16, 2, 63, True)])
def test_layered_build_equals_batch_build(K, D, TT, peaked):
    w = gen.make_custom(cfg_id=960 + K + D, B=2, mode="dynamic", K=K, D=D, total_tokens=TT, V=700, peaked=peaked)
    for b in range(w.B):
        ref = ot.build_dynamic(w.logprobs[b], int(w.root_token[b]), K, D, TT, w.T_max)
        got = ot.build_dynamic_layers(layers_of(w.logprobs[b], K, D), int(w.root_token[b]), K, D, TT, w.T_max)
        assert got[0] == ref[0] and got[1] == ref[1] and got[3:5] == ref[3:5]
        assert np.array_equal(np.array(got[2], np.float32).view(np.uint32), np.array(ref[2], np.float32).view(np.uint32))
        assert len(got[5]) == D + 1


def _rank_in_row(row):
    order = np.argsort(-np.asarray(row, np.float32), kind="stable")
    rank = np.empty(len(row), np.int64)
    rank[order] = np.arange(len(row))
    return rank


@pytest.mark.parametrize("peaked", [False, True])
def test_frontiers_are_the_best_extensions_of_whole_rows(peaked):
    K, D, V = 5, 4, 300
    w = gen.make_custom(cfg_id=970, B=1, mode="dynamic", K=K, D=D, total_tokens=30, V=V, peaked=peaked)
    rows = w.logprobs[0]
    fr = ot.build_dynamic_layers(layers_of(rows, K, D), int(w.root_token[0]), K, D, 30, w.T_max)[5]
    # layer 0: the K best tokens of the root row
    r0 = rows[0]
    best0 = sorted(range(V), key=lambda v: (-r0[v], v))[:K]
    assert fr[0][0] == best0
    fscore = [np.float32(r0[v]) for v in best0]
    for l in range(1, D + 1):
        ext = []
        for j in range(K):
            row = rows[1 + (l - 1) * K + j]
            rank = _rank_in_row(row)
            for v in range(V):
                ext.append((-float(np.float32(row[v] + fscore[j])), j, int(rank[v]), v))
        ext.sort()
        top = ext[:K]
        assert fr[l][0] == [e[3] for e in top], f"layer {l}"
        assert fr[l][1] == [e[1] for e in top], f"layer {l}"
        fscore = [np.float32(-e[0]) for e in top]


def test_log_softmax_closed_forms():
    V = 1000
    lp = ot.log_softmax_row(np.full(V, 3.25, np.float32))
    assert (lp == np.float32(-math.log(V))).all()
    z = np.array([0.0, math.log(3.0)], np.float32)       # probabilities 1/4, 3/4
    lp = ot.log_softmax_row(z)
    assert abs(float(lp[0]) - math.log(0.25)) < 1e-6 and abs(float(lp[1]) - math.log(0.75)) < 1e-6
    rng = np.random.default_rng(5)
    z = (rng.standard_normal(32000) * 2).astype(np.float32)
    lp = ot.log_softmax_row(z)
    assert abs(np.exp(lp.astype(np.float64)).sum() - 1.0) < 1e-5
    assert (lp <= 0).all()
    np.testing.assert_array_equal(lp, log_softmax(z.astype(np.float64)).astype(np.float32))


@pytest.mark.parametrize("K,D", [(10, 6), (4, 3), (16, 1)])
def test_logits_build_equals_build_on_library_log_softmax(K, D):
    """Raw logits through the fused log-softmax = the batch build on scipy's log-softmax
    of the same logits (no two kept tokens of a row tie after rounding here)."""
    V = 900
    rng = np.random.default_rng(K * 100 + D)
    B = 2
    for b in range(B):
        z = (rng.standard_normal((1 + D * K, V)) * 2).astype(np.float32)
        lp = log_softmax(z.astype(np.float64), axis=1).astype(np.float32)
        TT = min(K + D * K * K, 63)
        ref = ot.build_dynamic(lp, 7, K, D, TT, 64)
        got = ot.build_dynamic_layers(layers_of(z, K, D), 7, K, D, TT, 64, logits=True)
        assert got[0] == ref[0] and got[1] == ref[1] and got[3:5] == ref[3:5]
        assert np.array_equal(np.array(got[2], np.float32), np.array(ref[2], np.float32))


def test_non_finite_logits_give_the_root_only_tree():
    K, D, V = 3, 2, 50
    z = np.zeros((1 + D * K, V), np.float32)
    z[4, 7] = np.inf
    got = ot.build_dynamic_layers(layers_of(z, K, D), 9, K, D, 5, 16, logits=True)
    assert got[4] == ot.ST_LOGPROB and got[3] == 1 and got[0][0] == 9
