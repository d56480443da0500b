"""GPU parity of the paged-cache calls against the oracle's paged functions.

tree_attention_paged, kv_compact_paged and tree_accept_compact_paged run on a pool
whose blocks are placed at seeded random physical blocks (workloads.gen.paged_layout;
blocks no request owns and rows past a request's cache hold NaN bits, so a wrong
lookup shows).  The bars are those of the linear calls (tests/parity_util.py):
attention within the bf16 tolerance (fp32: 1e-4), the whole pools after compaction
bit for bit.  Block sizes from 1 token (a token-level table) to 256; one request,
ragged batches, more than 64 requests, d = 64 and 128, fp32, the fused compaction,
the full-size large-batch workload the benchmark times, and table entries outside
the pool.
"""
import numpy as np
import pytest

from tests.conftest import gpu_available
from workloads import gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not gpu_available():
        pytest.skip("no GPU")
    from tree_attention_verification_amd import _lib
    _lib.lib()   # raises if the library is missing: no fallback


def run(w, bs, **kw):
    from tests.parity_util import run_pipeline_and_compare
    return run_pipeline_and_compare(w, paged=gen.paged_layout(w, bs), **kw)


def _ragged(cfg_id=930, d=128):
    return gen.make_custom(cfg_id=cfg_id, B=5, P=[3000, 10, 0, 700, 64], mode="given",
                           given_sizes=[40, 3, 1, 64, 17], given_depth=6, T_max=64, dcap=8, Hq=16, Hkv=4, d=d,
                           dtype="bf16", V=50)


@pytest.mark.parametrize("bs", [1, 4, 16, 64, 256])
def test_paged_ragged_batch(bs):
    run(_ragged(), bs)


@pytest.mark.parametrize("bs", [2, 32])
def test_paged_ragged_batch_d64(bs):
    run(_ragged(cfg_id=931, d=64), bs)


def test_paged_single_request_dynamic_tree():
    # one request (capacity-sized splits, the first tile's block numbers read after
    # the sizes): the dynamic-tree workload at batch 1
    run(gen.make_workload(2), 16)


def test_paged_fp32_static_tree():
    run(gen.make_workload(1), 8)


def test_paged_ragged_batch16_full():
    run(gen.make_workload(3), 32)


def test_paged_large_batch_full_size():
    # the large-batch workload at full size, 16 tokens per block, every written row
    run(gen.make_workload(5), 16)


def test_paged_many_requests_d64():
    rng = np.random.default_rng(78)
    B = 70
    P = [int(x) for x in rng.integers(0, 400, size=B)]
    sizes = [int(x) for x in rng.integers(1, 33, size=B)]
    w = gen.make_custom(cfg_id=932, B=B, P=P, mode="given", given_sizes=sizes, given_depth=5, T_max=32, dcap=6,
                        Hq=8, Hkv=2, d=64, dtype="bf16", V=50)
    run(w, 4)


@pytest.mark.parametrize("bs", [1, 16])
def test_paged_fused_calls(bs):
    run(gen.make_workload(5, batch=12, prefix=777), bs, fused=True)
    run(gen.make_workload(2, prefix=500), bs, fused=True)


def test_paged_equals_linear_bit_for_bit():
    """Same keys in the same order: the paged call's output and compaction equal the
    linear call's bit for bit (capacity = S_cap, so both take the same launch plan)."""
    import torch
    from tree_attention_verification_amd.step import TreeVerifyStep
    w = gen.make_custom(cfg_id=933, B=4, P=[1000, 37, 2000, 511], S_cap=2112, mode="given",
                        given_sizes=[64, 9, 30, 1], given_depth=7, Hq=32, Hkv=8, d=128, dtype="bf16", V=50,
                        accept_prob=0.9)
    pc = gen.paged_layout(w, 64)
    assert pc.capacity == w.S_cap
    outs = []
    for paged in (None, pc):
        st = TreeVerifyStep(w, paged=paged)
        st.meta()
        st.attention()
        tp = gen.synthetic_target_predict(w, w.given_tokens, w.given_parents, w.given_size)
        st.set_target_predict(tp)
        st.accept_compact()
        torch.cuda.synchronize()
        outs.append((st.out_host(), st.kv_host(), st.accept_host()))
    (o_lin, (k_lin, v_lin), a_lin), (o_pg, (k_pg, v_pg), a_pg) = outs
    assert np.array_equal(o_lin, o_pg)
    assert a_lin["accept_len"].max() >= 1
    np.testing.assert_array_equal(a_lin["new_prefix_len"], a_pg["new_prefix_len"])
    from oracle import attention as oa
    for lin, pool in ((k_lin, k_pg), (v_lin, v_pg)):
        back = oa.paged_to_linear(pool, pc.block_table, 64, w.S_cap)
        assert np.array_equal(back.view(np.uint16), lin.view(np.uint16))


def test_paged_table_entries_outside_the_pool():
    """Entries outside [0, n_blocks) in request 1's table: nothing is read outside the
    pool, requests 0 and 2 get the oracle's results, and request 1's compaction is
    skipped (rows untouched, new_prefix_len = P + 1)."""
    import torch
    from oracle import attention as oa
    from oracle import kv as okv
    from oracle import tree as ot
    from tests.parity_util import check_attention
    from tree_attention_verification_amd.step import TreeVerifyStep
    w = gen.make_custom(cfg_id=934, B=3, P=[300, 200, 90], mode="given", given_sizes=[20, 30, 12], given_depth=4,
                        Hq=8, Hkv=2, d=128, dtype="bf16", V=50, accept_prob=1.0)
    bs = 16
    pc = gen.paged_layout(w, bs)
    good = gen.PagedCache(**{**pc.__dict__, "block_table": pc.block_table.copy()})
    P1 = int(w.prefix_len[1])
    pc.block_table[1, 3] = -5                          # a prefix block
    pc.block_table[1, (P1 + 1) // bs] = pc.n_blocks + 3  # the block holding row P + 1
    st = TreeVerifyStep(w, paged=pc)
    st.meta()
    st.attention()
    tp = gen.synthetic_target_predict(w, w.given_tokens, w.given_parents, w.given_size)
    st.set_target_predict(tp)
    st.accept()
    st.compact()
    torch.cuda.synchronize()
    meta = ot.tree_mask_positions(w.given_parents, w.given_size, w.prefix_len, w.T_max, w.dcap)
    o_ref = oa.tree_attention_paged(w.Q, good.K_pool, good.V_pool, good.block_table, bs, w.prefix_len, w.given_size,
                                    meta["tree_mask"], status=meta["status"])
    o_gpu = st.out_host()
    for b in (0, 2):
        sub = gen.Workload(**{**w.__dict__, "B": 1})
        check_attention(o_gpu[b:b + 1], o_ref[b:b + 1], sub, w.given_size[b:b + 1], meta["status"][b:b + 1],
                        f"request {b}")
    acc = ot.tree_accept(w.given_tokens, w.given_parents, w.given_size, tp, meta["status"], w.dcap)
    assert acc["accept_len"][1] >= 1
    lens = acc["accept_len"].copy()
    lens[1] = 0                                        # request 1 is left as it was
    K2, V2, newlen = okv.kv_compact_paged(pc.K_pool, pc.V_pool, good.block_table, bs, w.prefix_len,
                                          acc["accept_path"], lens)
    kg, vg = st.kv_host()
    assert np.array_equal(kg.view(np.uint16), K2.view(np.uint16))
    assert np.array_equal(vg.view(np.uint16), V2.view(np.uint16))
    got = st.accept_host()["new_prefix_len"]
    assert got[1] == P1 + 1
    np.testing.assert_array_equal(np.delete(got, 1), np.delete(newlen, 1))
