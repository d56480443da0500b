"""Pins for the oracle's paged-cache functions (CPU only).

Expected values come from:
  * a hand-worked example (tests/golden/paged_tiny.json): pool slot (block, offset)
    holds 10*block + offset, so every logical row read through the block table, and
    every row the compaction moves, can be checked by eye;
  * the linear oracle, which is pinned on its own: the paged attention of a paged
    copy of a cache equals the linear attention of the cache bit for bit (the same
    float64 arithmetic on the same values), for block sizes from 1 to 64;
  * the compaction commutes with the paging: compacting the paged copy gives the
    paged copy of the compacted linear cache, and blocks no request owns keep their
    bytes.
"""
import json
import os

import numpy as np
import pytest

from oracle import attention as oa
from oracle import kv as okv
from oracle import tree as ot
from workloads import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "paged_tiny.json")


def _golden():
    with open(GOLDEN) as f:
        g = json.load(f)
    nb, bs = g["n_blocks"], g["tokens_per_block"]
    pool = np.zeros((nb, 1, bs, 1), np.float32)
    for blk in range(nb):
        for off in range(bs):
            pool[blk, 0, off, 0] = 10 * blk + off
    return g, pool


def test_golden_paged_rows():
    g, pool = _golden()
    table = np.array(g["block_table"], np.int32)
    n = table.shape[1] * g["tokens_per_block"]
    lin = oa.paged_to_linear(pool, table, g["tokens_per_block"], n)
    assert lin.shape == (2, 1, n, 1)
    np.testing.assert_array_equal(lin[:, 0, :, 0], np.array(g["logical_rows"], np.float32))


def test_golden_paged_compaction():
    g, pool = _golden()
    table = np.array(g["block_table"], np.int32)
    K2, V2, new_len = okv.kv_compact_paged(pool, pool + 100, table, g["tokens_per_block"], g["prefix_len"],
                                           np.array(g["accept_path"]), g["accept_len"])
    np.testing.assert_array_equal(K2[:, 0, :, 0], np.array(g["pool_after"], np.float32))
    np.testing.assert_array_equal(V2[:, 0, :, 0], np.array(g["pool_after"], np.float32) + 100)
    np.testing.assert_array_equal(new_len, g["new_prefix_len"])


def _ragged(mode="given", dtype="bf16", seed=0):
    return gen.make_custom(cfg_id=700 + seed, B=4, P=[0, 37, 100, 64], S_cap=180, mode=mode, given_sizes=[1, 12, 30, 5],
                           Hq=8, Hkv=2, d=64, dtype=dtype)


@pytest.mark.parametrize("bs", [1, 2, 16, 64])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_paged_attention_equals_linear(bs, dtype):
    w = _ragged(dtype=dtype)
    meta = ot.tree_mask_positions(w.given_parents, w.given_size, w.prefix_len, w.T_max, w.dcap)
    ref = oa.tree_attention(w.Q, w.Kc, w.Vc, w.prefix_len, w.given_size, meta["tree_mask"], status=meta["status"])
    pc = gen.paged_layout(w, bs)
    got = oa.tree_attention_paged(w.Q, pc.K_pool, pc.V_pool, pc.block_table, bs, w.prefix_len, w.given_size,
                                  meta["tree_mask"], status=meta["status"])
    assert np.array_equal(got, ref)
    picks = [(1, 3, 5), (2, 29, 0), (0, 0, 7), (3, 4, 2)]
    rows = oa.attention_rows_paged(w.Q, pc.K_pool, pc.V_pool, pc.block_table, bs, w.prefix_len, w.given_size,
                                   meta["tree_mask"], picks, status=meta["status"])
    np.testing.assert_allclose(rows, np.stack([ref[b, i, h] for b, i, h in picks]), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("bs", [1, 8, 32])
def test_paged_compaction_commutes_with_paging(bs):
    w = _ragged()
    meta = ot.tree_mask_positions(w.given_parents, w.given_size, w.prefix_len, w.T_max, w.dcap)
    tp = gen.synthetic_target_predict(w, w.given_tokens, w.given_parents, w.given_size)
    acc = ot.tree_accept(w.given_tokens, w.given_parents, w.given_size, tp, meta["status"], w.dcap)
    assert acc["accept_len"].max() >= 1, "the case should move rows"
    K_lin, V_lin, len_lin = okv.kv_compact(w.Kc, w.Vc, w.prefix_len, acc["accept_path"], acc["accept_len"])
    pc = gen.paged_layout(w, bs)
    K_pg, V_pg, len_pg = okv.kv_compact_paged(pc.K_pool, pc.V_pool, pc.block_table, bs, w.prefix_len,
                                              acc["accept_path"], acc["accept_len"])
    np.testing.assert_array_equal(len_pg, len_lin)
    w_after = gen.Workload(**{**w.__dict__, "Kc": K_lin, "Vc": V_lin})
    expect = gen.paged_layout(w_after, bs)
    assert np.array_equal(K_pg.view(np.uint16), expect.K_pool.view(np.uint16))
    assert np.array_equal(V_pg.view(np.uint16), expect.V_pool.view(np.uint16))
    owned = np.zeros(pc.n_blocks, bool)
    owned[pc.block_table.reshape(-1)] = True
    assert (~owned).any()
    assert np.array_equal(K_pg[~owned].view(np.uint16), pc.K_pool[~owned].view(np.uint16))
