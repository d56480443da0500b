"""GPU parity of the layer-by-layer dynamic build (tree_build_layer, tree_build_finish).

Each test stages the draft rows one layer at a time, runs tree_build_layer for
layers 0..D and tree_build_finish on the GPU, and compares with the oracle's
layered build (oracle.tree.build_dynamic_layers) on the same bytes: every layer's
frontier (tokens and parent slots), the tree (tokens, parents, float32 score
bits, size, status) and the metadata, all bit for bit.  Rows are log-probs or raw
logits (fused log-softmax); shapes cover the benchmark's dynamic workloads, K = 1
and 16, D = 0, a vocabulary not a multiple of 4, peaked rows, bad values, and a
state reused by a second build.
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


def layers_of(rows, K, D):
    return [rows[:1]] + [rows[1 + (l - 1) * K:1 + l * K] for l in range(1, D + 1)]


def run_layers(w, logits=None, meta=True, step=None):
    import torch
    from oracle import tree as ot
    from tests.parity_util import check_meta
    from tree_attention_verification_amd.step import TreeVerifyStep
    st = step or TreeVerifyStep(w)
    st.prepare_layers(rows=logits, logits=logits is not None)
    st.build_layers(meta=meta)
    torch.cuda.synchronize()
    got = st.tree_host()
    ftok, fpar = st.frontiers_host()
    K, D = w.K, w.D
    rows_all = logits if logits is not None else w.logprobs
    status = np.zeros(w.B, np.int32)
    parents = np.full((w.B, w.T_max), -1, np.int32)
    sizes = np.zeros(w.B, np.int32)
    for b in range(w.B):
        t, p, s, n, stt, fr = ot.build_dynamic_layers(layers_of(rows_all[b], K, D), int(w.root_token[b]), K, D,
                                                      w.total_tokens, w.T_max, logits=logits is not None)
        assert got["status"][b] == stt, f"request {b}"
        assert got["tree_size"][b] == n, f"request {b}"
        np.testing.assert_array_equal(got["draft_tokens"][b], t, err_msg=f"request {b}")
        np.testing.assert_array_equal(got["parents"][b], p, err_msg=f"request {b}")
        assert np.array_equal(got["node_score"][b].view(np.uint32), np.array(s, np.float32).view(np.uint32))
        if stt == 0:
            for l in range(D + 1):
                np.testing.assert_array_equal(ftok[l, b], fr[l][0], err_msg=f"request {b} layer {l} tokens")
                np.testing.assert_array_equal(fpar[l, b], fr[l][1], err_msg=f"request {b} layer {l} parents")
        status[b], parents[b], sizes[b] = stt, p, n
    if meta:
        ref = ot.tree_mask_positions(parents, sizes, w.prefix_len, w.T_max, w.dcap, status)
        check_meta(st.meta_host(), ref)
    return got


def test_layers_dynamic_batch1_logprobs():
    run_layers(gen.make_workload(2, with_attention=False))


def test_layers_dynamic_batch1_logits():
    w = gen.make_workload(2, with_attention=False)
    run_layers(w, logits=gen.draft_logits(2, w.B, w.rows_per_req, w.V))


def test_layers_ragged_batch16_logprobs_and_logits():
    w = gen.make_workload(3, with_attention=False)
    run_layers(w)
    run_layers(w, logits=gen.draft_logits(3, w.B, w.rows_per_req, w.V))


@pytest.mark.parametrize("K,D,TT,V,peaked", [(1, 6, 6, 300, False), (3, 0, 2, 1001, False), (16, 2, 63, 777, True),
                                              (4, 3, 52, 1001, True), (5, 1, 30, 40000, False)])
def test_layers_shapes(K, D, TT, V, peaked):
    w = gen.make_custom(cfg_id=980 + K, B=3, mode="dynamic", K=K, D=D, total_tokens=TT, V=V, P=[10, 0, 90],
                        peaked=peaked)
    run_layers(w)
    run_layers(w, logits=gen.draft_logits(980 + K, w.B, w.rows_per_req, V, peaked=peaked), meta=False)


def test_layers_bad_logits_give_status():
    w = gen.make_custom(cfg_id=990, B=3, mode="dynamic", K=4, D=2, total_tokens=12, V=257, P=33)
    z = gen.draft_logits(990, w.B, w.rows_per_req, w.V)
    z[1, 3, 100] = np.nan
    z[2, 0, 5] = np.inf
    got = run_layers(w, logits=z)
    assert list(got["status"]) == [0, 4, 4]


def test_layers_equal_batch_build_and_reuse_state():
    """The layered build equals tree_build on the stacked rows (bit for bit, on the GPU),
    and a second build on the same state (other rows) is as exact as the first."""
    import torch
    from tree_attention_verification_amd.step import TreeVerifyStep
    w = gen.make_workload(3, with_attention=False)
    st = TreeVerifyStep(w)
    st.build()
    torch.cuda.synchronize()
    batch = st.tree_host()
    layered = run_layers(w, step=st)
    for k in ("draft_tokens", "parents", "tree_size", "status"):
        np.testing.assert_array_equal(layered[k], batch[k])
    assert np.array_equal(layered["node_score"].view(np.uint32), batch["node_score"].view(np.uint32))
    # the same state again, other rows (its contents are the first build's)
    run_layers(w, logits=gen.draft_logits(3, w.B, w.rows_per_req, w.V), step=st)
