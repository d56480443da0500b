"""GPU parity of tree_sampling_probs (target logits -> filtered probabilities) against
the oracle's sampling_probs_row, and of the chain tree_sampling_probs ->
tree_accept_sample against the oracle's filter + accept_sample.

Bars: the set of kept tokens is bit-exact (the top-k and top-p cuts are exact on
both sides: counts, and exact sums of the same float32 weights); kept
probabilities within 2e-6 relative (one float32 rounding of w / W, W summed in a
different order); rows past a request's tree are untouched.  Cases: several
vocabulary sizes (50 to 128256, i.e. one to ~125 values per thread), mixed
per-request parameters, ties (logits rounded to a coarse grid), NaN / +-inf / -0.0
logits, greedy and off settings of every filter, bad statuses, T_max = 256, and rows
off 16-byte boundaries.
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


def run_filter(logits, tree_size, status, params, offset=0):
    """offset > 0: the logits and the output start `offset` floats into larger
    buffers (rows no longer on 16-byte boundaries)."""
    import torch
    from oracle import sampling as osm
    from tree_attention_verification_amd import _lib as tv
    B, T_max, V = logits.shape
    temp, top_k, top_p, min_p = params
    n = B * T_max * V
    out = torch.full((n + offset,), -7.0, dtype=torch.float32, device="cuda")[offset:].view(B, T_max, V)
    lg = torch.zeros(n + offset, dtype=torch.float32, device="cuda")
    lg[offset:] = _dev(logits).reshape(-1)
    tv.tree_sampling_probs(B, T_max, V, lg[offset:].view(B, T_max, V), _dev(tree_size, np.int32),
                           None if status is None else _dev(status, np.int32), _dev(temp, np.float32),
                           _dev(top_k, np.int32), _dev(top_p, np.float32), _dev(min_p, np.float32), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    st = np.zeros(B, np.int32) if status is None else status
    ref = osm.tree_sampling_probs(logits, tree_size, st, temp, top_k, top_p, min_p,
                                  np.full((B, T_max, V), -7.0, np.float32))
    np.testing.assert_array_equal(got > 0, ref > 0, err_msg="kept tokens")
    np.testing.assert_array_equal(got == -7.0, ref == -7.0, err_msg="untouched rows")
    np.testing.assert_allclose(got, ref, rtol=2e-6, atol=0)
    return got


@pytest.mark.parametrize("V", [50, 1000, 20001, 32000, 128256])
def test_filters_mixed_parameters(V):
    """V = 20001 keeps its keys in LDS but, not a multiple of 4, reads its logits
    one float at a time; V = 32000 reads them four at a time."""
    B = 8 if V <= 32000 else 3
    w = gen.make_custom(cfg_id=1600 + V % 89, B=B, mode="given", given_sizes=[6, 1, 3, 8, 2, 5, 4, 7][:B], V=V, P=4,
                        T_max=8, dcap=6)
    lg = gen.synthetic_target_logits(w, w.given_size)
    params = gen.sampling_params(w, B)
    params[1][0] = min(V - 1, 37)            # make sure top-k, top-p and min-p all run somewhere
    params[2][0], params[3][0], params[0][0] = 0.9, 0.01, 0.8
    run_filter(lg, w.given_size, None, params)


@pytest.mark.parametrize("offset", [1, 2])
def test_filters_rows_off_16_byte_boundaries(offset):
    """V = 32000 with the logits and the output shifted by 4 or 8 bytes: the rows
    keep their keys in LDS but take the one-token passes."""
    V = 32000
    w = gen.make_custom(cfg_id=1660 + offset, B=6, mode="given", given_sizes=[5, 2, 8, 1, 6, 3], V=V, P=4,
                        T_max=8, dcap=6)
    lg = gen.synthetic_target_logits(w, w.given_size)
    params = gen.sampling_params(w, 6)
    params[1][0] = 37
    params[2][0], params[3][0], params[0][0] = 0.9, 0.01, 0.8
    params[1][1], params[2][1], params[3][1], params[0][1] = 0, 0.7, 0.0, 1.1   # radix top-p
    run_filter(lg, w.given_size, None, params, offset=offset)


@pytest.mark.parametrize("tie_step", [0.5, 2.0])
def test_filters_with_ties(tie_step):
    w = gen.make_custom(cfg_id=1610, B=6, mode="given", given_sizes=[4] * 6, V=3000, P=4, T_max=4, dcap=3)
    lg = gen.synthetic_target_logits(w, w.given_size, tie_step=tie_step)
    temp = np.array([1.0, 0.7, 1.3, 1.0, 0.5, 2.0], np.float32)
    top_k = np.array([5, 0, 100, 2999, 0, 40], np.int32)
    top_p = np.array([1.0, 0.8, 0.95, 0.3, 0.99, 1.0], np.float32)
    min_p = np.array([0.0, 0.0, 0.05, 0.0, 0.3, 0.02], np.float32)
    run_filter(lg, w.given_size, None, (temp, top_k, top_p, min_p))


def test_filters_special_values_and_settings():
    V = 700
    w = gen.make_custom(cfg_id=1620, B=10, mode="given", given_sizes=[3] * 10, V=V, P=4, T_max=4, dcap=3)
    lg = gen.synthetic_target_logits(w, w.given_size)
    lg[0, 0, [3, 9, 11]] = np.nan
    lg[0, 1, [5, 6]] = np.inf                   # two +inf: they share the mass
    lg[0, 2, :] = -np.inf                       # an all -inf row: uniform
    lg[1, 0, :] = -0.0
    lg[1, 0, 10:20] = 0.0                       # -0.0 and +0.0 rank equal
    lg[1, 1, ::2] = np.nan
    temp = np.array([1.0, 1.0, 0.0, -1.0, np.nan, 1.0, 1.0, 1.0, 1.0, 0.9], np.float32)
    top_k = np.array([3, 0, 0, 0, 0, 1, V, V + 5, -4, V - 1], np.int32)
    top_p = np.array([1.0, 0.5, 1.0, 1.0, 1.0, 1.0, 0.0, np.nan, 1e-9, 0.999999], np.float32)
    min_p = np.array([0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 1.0, np.nan, 1e-7], np.float32)
    status = np.array([0, 0, 0, 0, 0, 0, 0, 0, 2, 0], np.int32)     # request 8: its root row only
    run_filter(lg, w.given_size, status, (temp, top_k, top_p, min_p))


def test_filters_wide_trees():
    w = gen.make_custom(cfg_id=1630, B=2, mode="given", given_sizes=[256, 130], given_depth=9, V=500, P=4,
                        T_max=256, dcap=20)
    lg = gen.synthetic_target_logits(w, w.given_size)
    params = (np.array([0.8, 1.2], np.float32), np.array([20, 0], np.int32), np.array([0.9, 0.7], np.float32),
              np.array([0.0, 0.05], np.float32))
    run_filter(lg, w.given_size, None, params)


def _tail_rows(V):
    """Rows whose top-p cut depends on weights far below 2^-33 (the exact sums decide):
      0: two tokens of weight 1 + a tail of ~1e-11: top_p 0.5 keeps 2 (1 < 0.5 (2 + tail));
      1: weight 1, four tied tokens of weight 0.5, the same tail: top_p 0.5 needs two of
         the tie group (without the tail, 1 + 0.5 would reach exactly half of 3);
      2: four equal weights, top_p 0.5: the cut lands exactly on a cumulative (2 kept);
      3: as 2 with the next float32 above 0.5 (3 kept);
      4: two tokens of weight 1 and one float32-subnormal weight: top_p 0.5 keeps 2."""
    lt = np.float32(np.log(1e-11))
    rows = np.full((5, V), -np.inf, np.float32)
    rows[0, :] = lt
    rows[0, [7, V - 3]] = 0.0
    rows[1, :] = lt
    rows[1, 11] = 0.0
    rows[1, [2, 30, 40, V - 1]] = np.float32(np.log(0.5))
    rows[2, [0, 5, 9, 13]] = 1.5
    rows[3, [0, 5, 9, 13]] = 1.5
    rows[4, [1, 4]] = 0.0
    rows[4, 8] = -100.0
    top_p = np.array([0.5, 0.5, 0.5, np.nextafter(np.float32(0.5), np.float32(1)), 0.5], np.float32)
    kept = [2, 3, 2, 3, 2]
    return rows, top_p, kept


@pytest.mark.parametrize("many", [False, True])
@pytest.mark.parametrize("top_k", [0, 200, 700])
def test_filters_exact_top_p_cut(many, top_k):
    """The top-p cut follows the exact sums of the float32 weights: tail weights of
    ~1e-11 (and a subnormal) move it.  top_k 0 and 700 take the radix path at 256
    threads per row, 200 the sorted survivor list; 0 the radix path at 1024 threads,
    200 and 700 the survivor list there.  `many` launches >= 512 rows, which selects
    the 256-thread kernel."""
    from oracle import sampling as osm
    V = 3000
    rows, top_p, kept = _tail_rows(V)
    B, T_max = (8, 64) if many else (5, 1)
    lg = np.random.default_rng(7).normal(0, 1, (B, T_max, V)).astype(np.float32)
    tree_size = np.ones(B, np.int32)
    tp = np.full(B, 0.9, np.float32)
    for r in range(5):
        lg[r, 0] = rows[r]
        tp[r] = top_p[r]
        if top_k == 0 or top_k > 3:
            ref = osm.sampling_probs_row(rows[r], 1.0, top_k, top_p[r], 0.0)
            assert int((ref > 0).sum()) == kept[r], r
    params = (np.ones(B, np.float32), np.full(B, top_k, np.int32), tp, np.zeros(B, np.float32))
    run_filter(lg, tree_size, None, params)


@pytest.mark.parametrize("V,many", [(3000, True), (32000, False)])
def test_filters_top_p_cut_on_a_weight_bin_boundary(V, many):
    """top_p x total equal to the exact weight above a level-0 radix bin (weights 1, 1
    in one bin and 0.5 x 4 in the next; top_p 0.5 of the total 4 is exactly the first
    bin's 2): no float64 estimate of the cumulatives can tell on which side the cut
    falls, so the exact bin choice decides (2 kept).  The next float32 above 0.5
    keeps 3, and so does top_p 0.5 once a tail of ~1e-11 weights is added (its
    mass puts the threshold past the boundary).
    Both shapes keep the row's keys in LDS (V = 3000 at 256 threads per row, V = 32000
    at 1024)."""
    from oracle import sampling as osm
    B, T_max = (8, 64) if many else (4, 1)
    lg = np.random.default_rng(11).normal(0, 1, (B, T_max, V)).astype(np.float32)
    half = np.float32(np.log(0.5))
    tp = np.full(B, 0.9, np.float32)
    cases = [(-np.inf, np.float32(0.5), 2), (-np.inf, np.nextafter(np.float32(0.5), np.float32(1)), 3),
             (np.float32(np.log(1e-11)), np.float32(0.5), 3),
             (np.float32(np.log(1e-11)), np.nextafter(np.float32(0.5), np.float32(1)), 3)]
    for r, (fill, p_, kept) in enumerate(cases):
        row = np.full(V, fill, np.float32)
        row[[3, V - 2]] = 0.0
        row[[5, 17, V // 2, V - 1]] = half
        lg[r, 0] = row
        tp[r] = p_
        ref = osm.sampling_probs_row(row, 1.0, 0, p_, 0.0)
        assert int((ref > 0).sum()) == kept, (r, int((ref > 0).sum()))
    tree_size = np.ones(B, np.int32)
    params = (np.ones(B, np.float32), np.zeros(B, np.int32), tp, np.zeros(B, np.float32))
    run_filter(lg, tree_size, None, params)


@pytest.mark.parametrize("tie_step", [0.0, 0.25])
def test_filters_many_rows_large_vocabulary(tie_step):
    """>= 512 rows (the 256-thread kernel) at V = 32000, which keeps every row in
    memory (no register copy): top_k <= 256 takes the sorted survivor list, top_k in
    257..1024 and no top-k take the radix top-p passes; ties from rounded logits."""
    B, T_max, V = 8, 64, 32000
    sizes = np.array([64, 40, 64, 10, 64, 33, 17, 64], np.int32)
    w = gen.make_custom(cfg_id=1650, B=B, mode="given", given_sizes=list(sizes), V=V, P=4, T_max=T_max, dcap=20,
                        given_depth=8)
    lg = gen.synthetic_target_logits(w, w.given_size, tie_step=tie_step)
    temp = np.array([1.0, 0.7, 1.3, 1.0, 0.5, 2.0, 0.9, 1.1], np.float32)
    top_k = np.array([300, 1000, 0, 256, 100, 257, 1024, 0], np.int32)
    top_p = np.array([0.9, 0.95, 0.8, 0.7, 0.99, 0.6, 0.85, 1.0], np.float32)
    min_p = np.array([0.0, 0.0, 0.01, 0.0, 0.0, 0.05, 0.0, 0.02], np.float32)
    run_filter(lg, w.given_size, None, (temp, top_k, top_p, min_p))


@pytest.mark.parametrize("many", [False, True])
@pytest.mark.parametrize("V", [50, 700, 32000])
def test_filters_top_p_value_bins(many, V):
    """Top-p without a small top-k: the first radix level bins the weights by value.
    Temperatures from 0.05 (the weights spread over many bins) to 1e4 (every token in
    the top bin, so the key levels run inside it), coarse ties, and top_k >= V (off)
    and between 1025 and V (the radix top-k, then the bins over its survivors)."""
    B, T_max = (8, 64) if many else (8, 2)
    rng = np.random.default_rng(V + 11 * many)
    lg = rng.normal(0, 2, (B, T_max, V)).astype(np.float32)
    lg[2] = np.round(lg[2] * 2) / 2                      # ties on a grid of 0.5
    lg[5] = np.round(lg[5] * 8) / 8
    tree_size = np.full(B, T_max, np.int32)
    tree_size[[1, 6]] = [3, 1]
    temp = np.array([0.05, 1e4, 1.0, 0.7, 1.0, 2.0, 0.3, 1e4], np.float32)
    top_k = np.array([0, 0, V + 3, V, min(V - 1, 1500), 0, 0, min(V - 1, 2000)], np.int32)
    top_p = np.array([0.9, 0.5, 0.8, 0.95, 0.7, 0.999, 0.1, 0.6], np.float32)
    min_p = np.array([0.0, 0.0, 0.0, 0.01, 0.0, 0.0, 0.0, 0.0], np.float32)
    run_filter(lg, tree_size, None, (temp, top_k, top_p, min_p))


@pytest.mark.parametrize("V,B", [(2000, 512), (32000, 64), (40000, 24)])
def test_filters_weights_bit_exact(V, B):
    """Every weight is fp32(exp((l - l_max) / temperature)) to the bit: one row per
    request, min_p set to the oracle's weight of a chosen token (which must stay)
    or to the next float32 above it (which must go), over weights from ~1 down to
    the subnormal range.  A weight one ulp off on the GPU flips that token."""
    from oracle import sampling as osm
    rng = np.random.default_rng(V + B)
    lg = (rng.normal(0, 1, (B, 1, V)) * rng.uniform(1, 40, (B, 1, 1))).astype(np.float32)
    temp = rng.uniform(0.2, 3.0, B).astype(np.float32)
    min_p = np.zeros(B, np.float32)
    for b in range(B):
        row = osm.rank_order(lg[b, 0])[0]
        w = osm.filter_weights(row, float(temp[b]))
        cand = np.nonzero((w > 0) & (w < 1))[0]
        j = int(cand[rng.integers(0, len(cand))])
        wj = np.float32(w[j])
        min_p[b] = wj if b % 2 == 0 else np.nextafter(wj, np.float32(2))
    params = (temp, np.zeros(B, np.int32), np.ones(B, np.float32), min_p)
    run_filter(lg, np.ones(B, np.int32), None, params)


@pytest.mark.parametrize("cfg", [2, 3])
def test_filter_then_target_only_sampling(cfg):
    """The whole non-greedy chain: logits -> tree_sampling_probs -> tree_accept_sample,
    against the oracle's filter + accept_sample (bit-exact results)."""
    import torch
    from oracle import sampling as osm
    from oracle import tree as ot
    from tree_attention_verification_amd import _lib as tv
    from tree_attention_verification_amd.step import TreeVerifyStep
    w = gen.make_workload(cfg, with_attention=False)
    st = TreeVerifyStep(w)
    st.build_meta()
    torch.cuda.synchronize()
    tree = st.tree_host()
    B, T_max, V = w.B, w.T_max, w.V
    lg = gen.synthetic_target_logits(w, tree["tree_size"])
    params = gen.sampling_params(w, B)
    probs = torch.zeros((B, T_max, V), dtype=torch.float32, device="cuda")
    status = st.status
    tv.tree_sampling_probs(B, T_max, V, _dev(lg), st.tree_size, status, _dev(params[0]), _dev(params[1]),
                           _dev(params[2]), _dev(params[3]), probs)
    _, uni = gen.synthetic_target_probs(w, tree["draft_tokens"], tree["parents"], tree["tree_size"])
    st.set_target_probs(probs.cpu().numpy(), uni)
    st.accept_sample()
    torch.cuda.synchronize()
    got = st.accept_host()
    stat = status.cpu().numpy()
    ref_probs = osm.tree_sampling_probs(lg, tree["tree_size"], stat, *params, np.zeros((B, T_max, V), np.float32))
    ref = ot.tree_accept_sample(tree["draft_tokens"], tree["parents"], tree["tree_size"], ref_probs, uni, stat,
                                st.dcap)
    for k in ("accept_len", "accept_path", "bonus_token"):
        np.testing.assert_array_equal(got[k], ref[k], err_msg=k)


@pytest.mark.parametrize("V", [1, 2, 3])
def test_filters_tiny_vocabularies(V):
    B = 6
    lg = np.random.default_rng(V).normal(0, 1, (B, 1, V)).astype(np.float32)
    lg[5, 0, :] = 0.5                               # all equal
    temp = np.array([1.0, 0.5, 1.0, 1.0, 2.0, 1.0], np.float32)
    top_k = np.array([0, max(V - 1, 0), 1, V, 2, 0], np.int32)
    top_p = np.array([1.0, 0.5, 1.0, 1e-6, 0.9, 0.6], np.float32)
    min_p = np.array([0.0, 0.0, 0.5, 0.0, 0.9, 0.0], np.float32)
    run_filter(lg, np.ones(B, np.int32), None, (temp, top_k, top_p, min_p))


def test_filters_largest_vocabulary():
    V = 262144                                      # the call's limit: 256 slices of 1024 tokens
    w = gen.make_custom(cfg_id=1640, B=2, mode="given", given_sizes=[2, 1], V=V, P=4, T_max=2, dcap=1)
    lg = gen.synthetic_target_logits(w, w.given_size, tie_step=0.25)
    params = (np.array([1.0, 0.7], np.float32), np.array([1000, 0], np.int32), np.array([0.9, 0.95], np.float32),
              np.array([0.0, 0.001], np.float32))
    run_filter(lg, w.given_size, None, params)
