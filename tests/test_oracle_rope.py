"""Pins for the oracle's rotary embedding of the tree's queries (CPU).

Expected values come from the definition's closed forms and the property RoPE is
built for: position 0 is the identity; each (i, i + d/2) pair keeps its length; a
unit vector in pair 0 (frequency 1) at position p becomes (cos p, sin p); and the
score of a rotated query and key depends only on their position difference
(R_m q . R_n k = q . R_(n-m) k).  The attention wrapper is pinned against the
plain attention of pre-rotated queries.
"""
import math

import numpy as np

from oracle import attention as oa
from oracle import tree as ot
from workloads import gen


def test_rope_closed_forms():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 64))
    np.testing.assert_allclose(oa.rope_rotate(x, np.zeros(5), 10000.0), x, rtol=0, atol=0)
    y = oa.rope_rotate(x, np.arange(5) * 37.0, 10000.0)
    np.testing.assert_allclose(x[:, :32] ** 2 + x[:, 32:] ** 2, y[:, :32] ** 2 + y[:, 32:] ** 2, rtol=1e-12)
    e = np.zeros(64)
    e[0] = 1.0
    p = 123.0
    r = oa.rope_rotate(e, np.array(p), 500000.0)
    assert abs(r[0] - math.cos(p)) < 1e-12 and abs(r[32] - math.sin(p)) < 1e-12
    assert np.count_nonzero(np.abs(r) > 1e-15) == 2


def test_rope_scores_depend_on_position_difference():
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    for m, n in [(0, 5), (100, 105), (3000, 3005), (7, 2)]:
        lhs = oa.rope_rotate(q, np.array(m), 10000.0) @ oa.rope_rotate(k, np.array(n), 10000.0)
        rhs = q @ oa.rope_rotate(k, np.array(n - m), 10000.0)
        assert abs(lhs - rhs) < 1e-9


def test_rope_attention_is_attention_of_rotated_queries():
    w = gen.make_custom(cfg_id=1300, B=2, P=[40, 7], mode="given", given_sizes=[9, 5], Hq=4, Hkv=2, d=64,
                        dtype="bf16")
    meta = ot.tree_mask_positions(w.given_parents, w.given_size, w.prefix_len, w.T_max, w.dcap)
    got = oa.tree_attention_rope(w.Q, w.Kc, w.Vc, w.prefix_len, w.given_size, meta["tree_mask"], meta["positions"],
                                 10000.0, status=meta["status"])
    Qr = np.empty(w.Q.shape)
    for b in range(w.B):
        for i in range(w.T_max):
            Qr[b, i] = oa.rope_rotate(w.Q[b, i], np.full(w.Hq, meta["positions"][b, i]), 10000.0)
    ref = oa.tree_attention(Qr, w.Kc, w.Vc, w.prefix_len, w.given_size, meta["tree_mask"], status=meta["status"])
    np.testing.assert_array_equal(got, ref)
