"""GPU parity of tree_accept_sample (target-only tree rejection sampling) against the
oracle's accept_sample on the same target distributions and uniform draws.

accept_len, accept_path and bonus_token must match bit for bit.  Both sides take
every decision in float64 from the same float32 inputs (only the order of the sums
differs, so a decision could only flip for a draw within ~1e-16 of its threshold).
Cases: the dynamic-tree workloads' trees, given random trees (depth up to 7) at
several vocabulary sizes (50 to 128256, slices of one entry to ~500), the greedy
limit (one-hot rows: the same result as tree_accept), rows with no mass, tokens
outside the vocabulary, bad statuses and depth caps.
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


def run_sampling(w, probs=None, uniforms=None, status=None, tokens=None, dcap=None):
    import torch
    from oracle import tree as ot
    from tree_attention_verification_amd.step import TreeVerifyStep
    st = TreeVerifyStep(w)
    if w.mode == "given":
        ref_tree = dict(draft_tokens=w.given_tokens, parents=w.given_parents, tree_size=w.given_size)
        st.meta()
    else:
        st.build_meta()
        torch.cuda.synchronize()
        ref_tree = st.tree_host()
    torch.cuda.synchronize()
    if dcap is not None:   # the tree is validated with the workload's cap, the walk runs with this one
        st.dcap = dcap
        st.accept_path = torch.full((w.B, dcap + 1), -7, dtype=torch.int32, device="cuda")
    tok = ref_tree["draft_tokens"] if tokens is None else tokens
    if tokens is not None:
        st.draft_tokens.copy_(torch.from_numpy(np.ascontiguousarray(tokens, dtype=np.int32)))
    if probs is None:
        probs, uniforms = gen.synthetic_target_probs(w, tok, ref_tree["parents"], ref_tree["tree_size"])
    st.set_target_probs(probs, uniforms)
    stat = st.status.cpu().numpy() if status is None else status
    if status is not None:
        st.status.copy_(torch.from_numpy(np.ascontiguousarray(status, dtype=np.int32)))
    ref = ot.tree_accept_sample(tok, ref_tree["parents"], ref_tree["tree_size"], probs, uniforms, stat, st.dcap)
    # with the workspace (every row's sum first, when the rows are few) and without
    for ws in (True, False):
        st.accept_sample(workspace=ws)
        torch.cuda.synchronize()
        got = st.accept_host()
        for k in ("accept_len", "accept_path", "bonus_token"):
            np.testing.assert_array_equal(got[k], ref[k], err_msg=f"{k} (workspace {ws})")
    return got, ref


def test_sampling_dynamic_batch1():
    got, _ = run_sampling(gen.make_workload(2, with_attention=False))


def test_sampling_ragged_batch16():
    run_sampling(gen.make_workload(3, with_attention=False))


@pytest.mark.parametrize("V", [1000, 32000, 128256])
def test_sampling_few_rows_large_vocab(V):
    # few enough rows that the workspace path sums every row first, vocabularies
    # up to 128256 (a partial last piece at 128256 and 1000)
    w = gen.make_custom(cfg_id=1260 + V % 89, B=3, mode="given", given_sizes=[16, 9, 1], given_depth=6, V=V, P=10,
                        accept_prob=0.85, T_max=16)
    assert w.B * w.T_max * V * 4 <= 32 << 20
    got, _ = run_sampling(w)
    assert got["accept_len"].max() >= 1


@pytest.mark.parametrize("V", [50, 1000, 32000, 128256])
def test_sampling_given_trees(V):
    w = gen.make_custom(cfg_id=1200 + V % 97, B=6, mode="given", given_sizes=[1, 5, 20, 40, 64, 64], given_depth=7,
                        V=V, P=10, accept_prob=0.85)
    got, _ = run_sampling(w)
    assert got["accept_len"].max() >= 2, "the case should walk down the tree"


def test_sampling_greedy_limit_matches_tree_accept():
    import torch
    from tree_attention_verification_amd.step import TreeVerifyStep
    w = gen.make_custom(cfg_id=1210, B=5, mode="given", given_sizes=[64, 33, 9, 2, 1], given_depth=6, V=300, P=4,
                        accept_prob=0.8)
    tp = gen.synthetic_target_predict(w, w.given_tokens, w.given_parents, w.given_size)
    onehot = np.zeros((w.B, w.T_max, w.V), np.float32)
    for b in range(w.B):
        onehot[b, np.arange(w.T_max), tp[b]] = 1.0
    uni = np.random.default_rng(3).random((w.B, w.T_max)).astype(np.float32)
    got, _ = run_sampling(w, onehot, uni)
    st = TreeVerifyStep(w)
    st.meta()
    st.set_target_predict(tp)
    st.accept()
    torch.cuda.synchronize()
    greedy = st.accept_host()
    for k in ("accept_len", "accept_path", "bonus_token"):
        np.testing.assert_array_equal(got[k], greedy[k], err_msg=k)


def test_sampling_edge_cases():
    w = gen.make_custom(cfg_id=1220, B=6, mode="given", given_sizes=[30, 30, 30, 30, 30, 12], given_depth=5, V=700,
                        P=4, accept_prob=0.9)
    probs, uni = gen.synthetic_target_probs(w, w.given_tokens, w.given_parents, w.given_size)
    probs[0] = 0.0                                  # no mass anywhere: correction = token 0
    probs[1, 0] = 0.0
    probs[1, 0, 123] = 1.0                          # a point mass off every child at the root
    uni[2] = 0.0                                    # u = 0: every child with mass is taken
    uni[3, 0] = np.float32(np.nextafter(np.float32(1.0), np.float32(0.0)))   # the largest draw below 1
    tokens = w.given_tokens.copy()
    tokens[4, 1:4] = [w.V + 5, -3, 7]               # tokens outside the vocabulary have no mass
    status = np.array([0, 0, 0, 0, 0, 2], np.int32)  # a bad status: the correction at the root
    run_sampling(w, probs, uni, status=status, tokens=tokens)


def test_sampling_wide_nodes():
    # one level under the root: 64 children (the widest node tested a child per
    # lane), 65 and 129 (one child at a time), some with repeated tokens (a
    # repeat brings no mass) and tokens outside the vocabulary
    w = gen.make_custom(cfg_id=1250, B=4, mode="given", given_sizes=[65, 66, 130, 40], given_depth=1, V=300, P=4,
                        T_max=160, dcap=3, accept_prob=0.3)
    assert all(int((w.given_parents[b, 1:w.given_size[b]] == 0).sum()) == w.given_size[b] - 1 for b in range(4))
    tokens = w.given_tokens.copy()
    tokens[1, 1:66] = np.arange(65) % 23            # 65 children, 23 distinct tokens
    tokens[2, 1:130] = np.arange(129) % 50          # 129 children, 50 distinct tokens
    tokens[3, 1:40] = np.arange(39) % 7             # 39 children, 7 distinct tokens
    tokens[3, 5] = -1
    tokens[3, 9] = w.V + 2
    tokens[1, 60] = 250                             # first occurrences past the repeats
    tokens[2, 100] = 299
    probs, uni = gen.synthetic_target_probs(w, tokens, w.given_parents, w.given_size)
    uni[0, 40] = 0.0     # u = 0: taken if no earlier child is and its token has mass
    uni[1, 31] = 0.0     # a repeated token (child 8's): no mass, so not taken
    uni[1, 60] = 0.0
    uni[2, 100] = 0.0    # past the 64th child
    got, _ = run_sampling(w, probs, uni, tokens=tokens)
    assert got["accept_len"].tolist()[:3] == [1, 1, 1]
    # every child rejected (the correction leaves out each distinct rejected token once)
    uni2 = uni.copy()
    uni2[:, 1:] = np.float32(np.nextafter(np.float32(1.0), np.float32(0.0)))
    probs2 = probs.copy()
    probs2[:, 0] *= 0.5                              # less than the full mass on any child
    run_sampling(w, probs2, uni2, tokens=tokens)


@pytest.mark.parametrize("dcap", [0, 1, 3])
def test_sampling_depth_cap(dcap):
    w = gen.make_custom(cfg_id=1230 + dcap, B=4, mode="given", given_sizes=[64, 50, 20, 8], given_depth=7, V=500,
                        P=4, accept_prob=0.95)
    run_sampling(w, dcap=dcap)
