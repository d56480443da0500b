"""GPU parity of tree_accept_sample_draft (tree rejection sampling with the drafter's
distribution q) against the oracle's accept_sample_draft on the same target rows,
draft rows and uniform draws, in both q modes (candidates drawn without
replacement / independently).

accept_len, accept_path and bonus_token must match bit for bit.  Both sides take
every decision in float64 from the same float32 inputs, with each product rounded
on its own; only the order of the sums differs, so a decision could only flip for
a draw within ~1e-16 (relative) of its threshold.  Cases: the dynamic-tree
workloads' trees, given random trees (depth up to 7) at several vocabulary sizes,
trees of 256 nodes, the reductions to tree_accept_sample (point-mass q on chains)
and tree_accept (one-hot targets), and edge cases: q rows without mass, target
rows without mass, tokens outside the vocabulary, bad statuses, depth caps, a
workspace reused across calls.
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


def _dev(x, dtype=None):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x if dtype is None else np.asarray(x, dtype))).cuda()


def gpu_draft(tokens, parents, sizes, probs, q, uni, status, dcap, wr, ws=None):
    import torch
    from tree_attention_verification_amd import _lib as tv
    B, T_max, V = probs.shape
    if ws is None:
        ws = torch.empty(tv.tree_accept_sample_draft_workspace_bytes(B, V), dtype=torch.uint8, device="cuda")
    alen = torch.full((B,), -9, dtype=torch.int32, device="cuda")
    apath = torch.full((B, dcap + 1), -9, dtype=torch.int32, device="cuda")
    bonus = torch.full((B,), -9, dtype=torch.int32, device="cuda")
    tv.tree_accept_sample_draft(B, T_max, dcap, V, _dev(tokens, np.int32), _dev(parents, np.int32),
                                _dev(sizes, np.int32), _dev(probs, np.float32), _dev(q, np.float32),
                                _dev(uni, np.float32), _dev(status, np.int32), wr, alen, apath, bonus, ws)
    torch.cuda.synchronize()
    return dict(accept_len=alen.cpu().numpy(), accept_path=apath.cpu().numpy(), bonus_token=bonus.cpu().numpy())


def compare(tokens, parents, sizes, probs, q, uni, status, dcap, wr, ws=None):
    from oracle import sampling as osm
    got = gpu_draft(tokens, parents, sizes, probs, q, uni, status, dcap, wr, ws)
    ref = osm.tree_accept_sample_draft(tokens, parents, sizes, probs, q, uni, status, dcap, wr)
    for k in ("accept_len", "accept_path", "bonus_token"):
        np.testing.assert_array_equal(got[k], ref[k], err_msg=k)
    return got


def given_case(w):
    probs, uni = gen.synthetic_target_probs(w, w.given_tokens, w.given_parents, w.given_size)
    q = gen.synthetic_draft_probs(w, w.given_tokens, w.given_parents, w.given_size)
    return w.given_tokens, w.given_parents, w.given_size, probs, q, uni, np.zeros(w.B, np.int32)


@pytest.mark.parametrize("wr", [True, False])
@pytest.mark.parametrize("cfg", [2, 3])
def test_draft_sampling_dynamic_trees(cfg, wr):
    import torch
    from tree_attention_verification_amd.step import TreeVerifyStep
    w = gen.make_workload(cfg, with_attention=False)
    st = TreeVerifyStep(w)
    st.build_meta()
    torch.cuda.synchronize()
    tree = st.tree_host()
    probs, uni = gen.synthetic_target_probs(w, tree["draft_tokens"], tree["parents"], tree["tree_size"])
    q = gen.synthetic_draft_probs(w, tree["draft_tokens"], tree["parents"], tree["tree_size"])
    got = compare(tree["draft_tokens"], tree["parents"], tree["tree_size"], probs, q, uni,
                  st.status.cpu().numpy(), st.dcap, wr)
    assert got["accept_len"].max() >= 1


@pytest.mark.parametrize("wr", [True, False])
@pytest.mark.parametrize("V", [50, 1000, 32000, 128256])
def test_draft_sampling_given_trees(V, wr):
    w = gen.make_custom(cfg_id=1700 + V % 83, B=6, mode="given", given_sizes=[1, 5, 20, 40, 64, 64], given_depth=7,
                        V=V, P=10, accept_prob=0.7)
    got = compare(*given_case(w), w.dcap, wr)
    assert got["accept_len"].max() >= 1


def test_draft_sampling_big_trees():
    w = gen.make_custom(cfg_id=1710, B=3, mode="given", given_sizes=[256, 200, 97], given_depth=6, V=2000, P=4,
                        T_max=256, dcap=20, accept_prob=0.8)
    for wr in (True, False):
        compare(*given_case(w), w.dcap, wr)


def test_point_mass_draft_on_chains_equals_target_only():
    """q = the point mass on each chain node's only child: the same walk as
    tree_accept_sample (both library calls, and the oracle)."""
    import torch
    from tree_attention_verification_amd import _lib as tv
    B, T, V = 4, 12, 300
    rng = np.random.default_rng(5)
    par = np.tile(np.arange(-1, T - 1, dtype=np.int32), (B, 1))
    tok = rng.integers(0, V, (B, T)).astype(np.int32)
    w = gen.make_custom(cfg_id=1720, B=B, mode="given", given_sizes=[T] * B, V=V, P=4, T_max=T, dcap=T - 1,
                        accept_prob=0.9)
    probs, uni = gen.synthetic_target_probs(w, tok, par, np.full(B, T, np.int32))
    q = np.zeros((B, T, V), np.float32)
    for b in range(B):
        for i in range(T - 1):
            q[b, i, tok[b, i + 1]] = 1.0
    sizes = np.full(B, T, np.int32)
    status = np.zeros(B, np.int32)
    got = compare(tok, par, sizes, probs, q, uni, status, T - 1, True)
    alen = torch.zeros(B, dtype=torch.int32, device="cuda")
    apath = torch.zeros((B, T), dtype=torch.int32, device="cuda")
    bonus = torch.zeros(B, dtype=torch.int32, device="cuda")
    tv.tree_accept_sample(B, T, T - 1, V, _dev(tok), _dev(par), _dev(sizes), _dev(probs), _dev(uni), _dev(status),
                          alen, apath, bonus)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got["accept_len"], alen.cpu().numpy())
    np.testing.assert_array_equal(got["accept_path"], apath.cpu().numpy())
    np.testing.assert_array_equal(got["bonus_token"], bonus.cpu().numpy())


def test_one_hot_targets_equal_greedy_accept():
    import torch
    from tree_attention_verification_amd.step import TreeVerifyStep
    w = gen.make_custom(cfg_id=1730, B=5, mode="given", given_sizes=[64, 33, 9, 2, 1], given_depth=6, V=300, P=4,
                        accept_prob=0.8)
    tp = gen.synthetic_target_predict(w, w.given_tokens, w.given_parents, w.given_size)
    onehot = np.zeros((w.B, w.T_max, w.V), np.float32)
    for b in range(w.B):
        onehot[b, np.arange(w.T_max), tp[b]] = 1.0
    q = gen.synthetic_draft_probs(w, w.given_tokens, w.given_parents, w.given_size)
    uni = np.random.default_rng(3).random((w.B, w.T_max)).astype(np.float32)
    st = TreeVerifyStep(w)
    st.meta()
    st.set_target_predict(tp)
    st.accept()
    torch.cuda.synchronize()
    greedy = st.accept_host()
    for wr in (True, False):
        got = compare(w.given_tokens, w.given_parents, w.given_size, onehot, q, uni, np.zeros(w.B, np.int32), w.dcap,
                      wr)
        for k in ("accept_len", "accept_path", "bonus_token"):
            np.testing.assert_array_equal(got[k], greedy[k], err_msg=k)


def test_draft_sampling_edge_cases_and_workspace_reuse():
    import torch
    from tree_attention_verification_amd import _lib as tv
    w = gen.make_custom(cfg_id=1740, B=7, mode="given", given_sizes=[30, 30, 30, 30, 30, 12, 25], given_depth=5,
                        V=700, P=4, accept_prob=0.9)
    tokens, parents, sizes, probs, q, uni, status = given_case(w)
    tokens = tokens.copy()
    probs[0] = 0.0                                   # no target mass anywhere: token 0
    q[1] = 0.0                                       # no draft mass: accept iff target mass
    q[2, 0] = 0.0
    q[2, 0, 5] = 1.0                                 # a point mass on a token no child has
    tokens[3, 1:4] = [w.V + 5, -3, 7]                # tokens outside the vocabulary
    status[5] = 2                                    # a bad status: the correction at the root
    uni[6] = 0.0                                     # u = 0: the first child with target mass
    ws = torch.full((tv.tree_accept_sample_draft_workspace_bytes(w.B, w.V),), 255, dtype=torch.uint8, device="cuda")
    for wr in (True, False):
        compare(tokens, parents, sizes, probs, q, uni, status, w.dcap, wr, ws)
    for dcap in (0, 1, 3):                           # depth caps (tree validated with the workload's cap)
        compare(tokens, parents, sizes, probs, q, uni, status, dcap, True, ws)


@pytest.mark.parametrize("V", [700, 32000])
def test_draft_sampling_wide_nodes_and_repeated_tokens(V):
    # one level under the root with 64, 65 and 129 children (the child mask's later
    # words), tokens repeated among siblings (a repeat's mass is already removed
    # without replacement) and outside the vocabulary; V = 700 takes the one
    # workgroup per request kernel, V = 32000 the sliced one
    w = gen.make_custom(cfg_id=1760 + V % 7, B=4, mode="given", given_sizes=[65, 66, 130, 40], given_depth=1,
                        V=V, P=4, T_max=160, dcap=3, accept_prob=0.3)
    tokens, parents, sizes, probs, q, uni, status = given_case(w)
    tokens = tokens.copy()
    tokens[1, 1:66] = np.arange(65) % 23
    tokens[2, 1:130] = np.arange(129) % 50
    tokens[3, 1:40] = np.arange(39) % 7
    tokens[3, 5] = -1
    tokens[3, 9] = V + 2
    q = gen.synthetic_draft_probs(w, tokens, parents, sizes)
    for wr in (True, False):
        compare(tokens, parents, sizes, probs, q, uni, status, w.dcap, wr)
    # every child rejected: the residual after all of a node's updates
    uni2 = uni.copy()
    uni2[:, 1:] = np.float32(np.nextafter(np.float32(1.0), np.float32(0.0)))
    for wr in (True, False):
        got = compare(tokens, parents, sizes, probs, q, uni2, status, w.dcap, wr)
        assert (got["accept_len"] == 0).any()


def test_draft_sampling_largest_vocabulary_and_tiny_trees():
    V = 262144                                      # the call's limit (a 32 KB bitmap of removed tokens)
    w = gen.make_custom(cfg_id=1750, B=2, mode="given", given_sizes=[12, 1], given_depth=3, V=V, P=4, T_max=16,
                        dcap=5, accept_prob=0.6)
    for wr in (True, False):
        compare(*given_case(w), w.dcap, wr)
    # V = 1: every token is token 0, so every child can be accepted
    rng = np.random.default_rng(17)
    parents = np.array([[-1, 0, 0, 1], [-1, 0, -1, -1], [-1, -1, -1, -1]], np.int32)
    tokens = np.where(parents >= 0, 0, -1).astype(np.int32)
    tokens[:, 0] = 0
    sizes = np.array([4, 2, 1], np.int32)
    probs = rng.random((3, 4, 1)).astype(np.float32)
    probs[1, 0, 0] = 0.0                             # no mass: the child is rejected, the correction is token 0
    q = rng.random((3, 4, 1)).astype(np.float32)
    uni = rng.random((3, 4)).astype(np.float32)
    for wr in (True, False):
        compare(tokens, parents, sizes, probs, q, uni, np.zeros(3, np.int32), 3, wr)


@pytest.mark.parametrize("wr", [True, False])
def test_filter_then_draft_sampling(wr):
    """The whole chain with the drafter's q: target logits -> tree_sampling_probs ->
    tree_accept_sample_draft, against the oracle's filter + accept_sample_draft."""
    import torch
    from oracle import sampling as osm
    from tree_attention_verification_amd.step import TreeVerifyStep
    w = gen.make_workload(3, with_attention=False)
    st = TreeVerifyStep(w)
    st.build_meta()
    torch.cuda.synchronize()
    tree = st.tree_host()
    B, T_max, V = w.B, w.T_max, w.V
    lg = gen.synthetic_target_logits(w, tree["tree_size"])
    params = gen.sampling_params(w, B)
    q = gen.synthetic_draft_probs(w, tree["draft_tokens"], tree["parents"], tree["tree_size"])
    _, uni = gen.synthetic_target_probs(w, tree["draft_tokens"], tree["parents"], tree["tree_size"])
    st.set_target_probs(np.zeros((B, T_max, V), np.float32), uni)
    st.set_sampling_inputs(lg, params, q)
    st.sampling_probs()
    st.accept_sample_draft(wr)
    torch.cuda.synchronize()
    got = st.accept_host()
    stat = st.status.cpu().numpy()
    ref_probs = osm.tree_sampling_probs(lg, tree["tree_size"], stat, *params, np.zeros((B, T_max, V), np.float32))
    ref = osm.tree_accept_sample_draft(tree["draft_tokens"], tree["parents"], tree["tree_size"], ref_probs, q, uni,
                                       stat, st.dcap, wr)
    for k in ("accept_len", "accept_path", "bonus_token"):
        np.testing.assert_array_equal(got[k], ref[k], err_msg=k)
