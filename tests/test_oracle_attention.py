"""Pins for the oracle's tree attention (CPU only).

Expected values come from an independent library routine -- torch's
scaled_dot_product_attention on the CPU in float64 -- and from closed forms:
  * the handbook's correctness check: every node's output equals plain attention of
    that node over [prefix ; its own root-to-node chain], computed per node;
  * a one-node tree is single-query decode attention over prefix + root;
  * a chain tree is causal attention shifted by the prefix length;
  * constant V rows give exactly that row; a key aligned with the query and scaled
    up dominates;
  * grouped heads: query head h reads kv head h // (Hq/Hkv);
  * keys that are not ancestors, and cache rows past prefix + tree, do not matter.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle import tree as ot
from workloads import gen


def sdpa(q, k, v, mask=None):
    """q [n][d], k/v [m][d] float64 numpy -> [n][d] via torch SDPA (float64, CPU)."""
    qt = torch.from_numpy(q)[None, None]
    kt = torch.from_numpy(k)[None, None]
    vt = torch.from_numpy(v)[None, None]
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m)[0, 0].numpy()


def build(parents, T, P):
    par = list(parents) + [-1] * (64 - T)
    return ot.mask_positions(par, T, P, 64, 63)


def f64(x):
    return oa.to_f64(x)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_chain_vs_tree_matches_per_chain_sdpa(dtype):
    """The handbook's check, with its six-node tree and a random one."""
    for parents, P in (([-1, 0, 0, 1, 1, 2], 37), (None, 80)):
        w = gen.make_custom(cfg_id=31, P=P, Hq=4, Hkv=2, d=64, dtype=dtype, T_max=64)
        if parents is None:
            rng = np.random.default_rng(3)
            parents = [-1] + [int(rng.integers(0, i)) for i in range(1, 20)]
        T = len(parents)
        meta = build(parents, T, P)
        O = oa.tree_attention(w.Q, w.Kc, w.Vc, w.prefix_len, np.array([T]), meta["tree_mask"][None])
        worst = 0.0
        for i in range(T):
            chain, j = [], i
            while j != -1:
                chain.append(j)
                j = parents[j]
            rows = list(range(P)) + [P + j for j in reversed(chain)]
            for h in range(4):
                g = h // 2
                ref = sdpa(f64(w.Q[0, i, h])[None], f64(w.Kc[0, g, rows]), f64(w.Vc[0, g, rows]))[0]
                worst = max(worst, np.abs(O[0, i, h] - ref).max())
        assert worst < 1e-12


def test_single_node_is_decode_attention():
    w = gen.make_custom(cfg_id=32, P=300, Hq=8, Hkv=2, d=128)
    meta = build([-1], 1, 300)
    O = oa.tree_attention(w.Q, w.Kc, w.Vc, w.prefix_len, np.array([1]), meta["tree_mask"][None])
    for h in range(8):
        ref = sdpa(f64(w.Q[0, 0, h])[None], f64(w.Kc[0, h // 4, :301]), f64(w.Vc[0, h // 4, :301]))[0]
        assert np.abs(O[0, 0, h] - ref).max() < 1e-12
    assert not O[0, 1:].any()                     # rows past the tree are untouched


def test_chain_is_causal_attention_with_offset():
    P, T = 50, 12
    w = gen.make_custom(cfg_id=33, P=P, Hq=2, Hkv=1, d=64, dtype="fp32")
    meta = build([-1] + list(range(T - 1)), T, P)
    O = oa.tree_attention(w.Q, w.Kc, w.Vc, w.prefix_len, np.array([T]), meta["tree_mask"][None])
    causal = np.zeros((T, P + T), bool)
    for i in range(T):
        causal[i, :P + i + 1] = True
    for h in range(2):
        ref = sdpa(f64(w.Q[0, :T, h]), f64(w.Kc[0, 0, :P + T]), f64(w.Vc[0, 0, :P + T]), causal)
        assert np.abs(O[0, :T, h] - ref).max() < 1e-12


def test_constant_values_and_peaked_key():
    P, T = 64, 9
    w = gen.make_custom(cfg_id=34, P=P, Hq=4, Hkv=4, d=64, dtype="fp32")
    parents = [-1, 0, 0, 1, 1, 2, 3, 3, 7]
    meta = build(parents, T, P)
    Vc = np.array(w.Vc)
    c = np.linspace(-1, 1, 64, dtype=np.float32)
    Vc[:] = c
    O = oa.tree_attention(w.Q, w.Kc, Vc, w.prefix_len, np.array([T]), meta["tree_mask"][None])
    assert np.abs(O[0, :T] - c.astype(np.float64)).max() < 1e-12
    # a prefix key 60 * q dominates every other score
    Kc = np.array(w.Kc)
    Kc[0, 1, 17] = 60.0 * w.Q[0, 4, 1]
    O = oa.tree_attention(w.Q, Kc, w.Vc, w.prefix_len, np.array([T]), meta["tree_mask"][None])
    assert np.abs(O[0, 4, 1] - w.Vc[0, 1, 17]).max() < 1e-6


def test_grouped_heads_read_their_kv_head():
    P, T = 20, 5
    w = gen.make_custom(cfg_id=35, P=P, Hq=8, Hkv=2, d=64, dtype="fp32")
    Vc = np.array(w.Vc)
    Vc[0, 0] = 1.0
    Vc[0, 1] = 2.0
    meta = build([-1, 0, 1, 1, 0], T, P)
    O = oa.tree_attention(w.Q, w.Kc, Vc, w.prefix_len, np.array([T]), meta["tree_mask"][None])
    for h in range(8):
        assert np.allclose(O[0, :T, h], 1.0 + h // 4, atol=1e-12)


def test_non_ancestors_and_rows_past_the_tree_do_not_matter():
    P, T = 40, 10
    w = gen.make_custom(cfg_id=36, P=P, Hq=4, Hkv=2, d=64, dtype="bf16")
    parents = [-1, 0, 0, 1, 1, 2, 2, 3, 5, 8]
    meta = build(parents, T, P)
    O = oa.tree_attention(w.Q, w.Kc, w.Vc, w.prefix_len, np.array([T]), meta["tree_mask"][None])
    Kc, Vc = np.array(w.Kc), np.array(w.Vc)
    Kc[0, :, P + 4] ^= 0x1234       # node 4 is an ancestor of nobody but itself
    Vc[0, :, P + 4] ^= 0x0F0F
    Kc[0, :, P + T:] = 0            # rows past the tree
    Vc[0, :, P + T:] = 0
    O2 = oa.tree_attention(w.Q, Kc, Vc, w.prefix_len, np.array([T]), meta["tree_mask"][None])
    rows = [i for i in range(T) if i != 4]
    assert np.array_equal(O[0, rows], O2[0, rows])
    assert not np.array_equal(O[0, 4], O2[0, 4])


def test_nonzero_status_is_root_only():
    P = 16
    w = gen.make_custom(cfg_id=37, P=P, Hq=2, Hkv=1, d=64, dtype="fp32")
    meta = build([-1, 0, 1], 3, P)
    O = oa.tree_attention(w.Q, w.Kc, w.Vc, w.prefix_len, np.array([3]), meta["tree_mask"][None],
                          status=np.array([1]))
    ref = sdpa(f64(w.Q[0, 0, 0])[None], f64(w.Kc[0, 0, :P + 1]), f64(w.Vc[0, 0, :P + 1]))[0]
    assert np.abs(O[0, 0, 0] - ref).max() < 1e-12 and not O[0, 1:].any()


def test_sampled_rows_agree_with_dense():
    w = gen.make_workload(5, batch=3, prefix=300)
    meta = ot.tree_mask_positions(w.given_parents, w.given_size, w.prefix_len, 64, 7)
    O = oa.tree_attention(w.Q, w.Kc, w.Vc, w.prefix_len, w.given_size, meta["tree_mask"])
    samples = [(0, 0, 0), (1, 3, 31), (2, int(w.given_size[2]) - 1, 9)]
    rows = oa.attention_rows(w.Q, w.Kc, w.Vc, w.prefix_len, w.given_size, meta["tree_mask"], samples)
    for (b, i, h), r in zip(samples, rows):
        assert np.abs(O[b, i, h] - r).max() < 1e-12
