"""GPU parity: the HIP library (through the C ABI) against the CPU oracle.

Every test runs the five calls on the GPU and compares each stage with the oracle
on the same seeded inputs (tests/parity_util.py states the bars).  Sizes: the five
configurations at sizes the oracle finishes in seconds (spanning several key
tiles and a ragged tail), all five at full size in the launch configuration the
benchmark times (every written attention row compared), plus fuzzed shapes and
the degenerate cases of the method.
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


def run(w, **kw):
    from tests.parity_util import run_pipeline_and_compare
    return run_pipeline_and_compare(w, **kw)


# ----------------------------------------------------------------------------- configurations
def test_tiny_static_fp32_p128():
    r = run(gen.make_workload(1))
    assert list(r["tree_size"]) == [11]


def test_eagle2_dynamic_b1_p2048_full():
    r = run(gen.make_workload(2))
    assert list(r["tree_size"]) == [61]


def test_ragged_b16_p512_8192_full():
    r = run(gen.make_workload(3))
    assert (r["tree_size"] == 49).all()


def test_long_context_b4_reduced_prefix():
    run(gen.make_workload(4, batch=2, prefix=3000))


def test_random_trees_b64_reduced():
    run(gen.make_workload(5, batch=12, prefix=777))


def test_long_context_b4_p32768_full_size():
    # every written row (4 requests x 61 nodes x 64 heads over 32829 keys, 8 splits)
    run(gen.make_workload(4))


def test_random_trees_b64_p4096_full_size():
    # every written row of 64 requests with trees of 8..64 nodes over 4096-token prefixes
    run(gen.make_workload(5))


def _scaled_v(w, factor):
    v = (w.Vc.astype(np.uint32) << np.uint32(16)).view(np.float32) * np.float32(factor)
    w.Vc = gen.f32_to_bf16_bits(v)
    return w


@pytest.mark.parametrize("factor", [1e5, 1e-6])
def test_split_partials_keep_the_range_of_v(factor):
    """V scaled far above fp16's largest value (|v| up to ~2e5) and far below its
    normal range (~1e-7): outputs through the split-KV partials (one request over a
    2048-token prefix: 7 splits; two over 9000 tokens: 8 splits) must keep bf16's
    range, like the unsplit path and the oracle.  The bars apply in units of the
    scale (attention is linear in V)."""
    run(_scaled_v(gen.make_workload(2), factor), v_scale=factor)
    run(_scaled_v(gen.make_workload(4, batch=2, prefix=9000), factor), v_scale=factor)
    # the unsplit path (a short prefix: one split) against the same bar
    run(_scaled_v(gen.make_workload(2, prefix=100), factor), v_scale=factor)


# ----------------------------------------------------------------------------- tree shapes
def test_peaked_drafts_give_deep_dynamic_trees():
    w = gen.make_workload(2, peaked=True, prefix=300)
    r = run(w)
    assert r["tree_size"][0] == 61


@pytest.mark.parametrize("K,D,TT", [(1, 6, 6), (3, 0, 2), (2, 2, 10), (16, 2, 63), (4, 3, 52), (5, 1, 30)])
def test_dynamic_build_shapes(K, D, TT):
    w = gen.make_custom(cfg_id=500 + K * 10 + D, mode="dynamic", K=K, D=D, total_tokens=TT, V=777, P=70,
                        Hq=4, Hkv=2, d=64, dtype="bf16")
    run(w)


@pytest.mark.parametrize("br", [[2, 2, 1, 1], [3, 3, 2], [1] * 20, [7], [4, 1, 4]])
def test_static_build_shapes(br):
    w = gen.make_custom(cfg_id=600 + len(br), mode="static", branching=br, V=1003, P=65, Hq=8, Hkv=4, d=128,
                        dtype="bf16", dcap=20)
    run(w)


def test_dynamic_total_tokens_equal_to_all_candidates():
    w = gen.make_custom(cfg_id=650, mode="dynamic", K=3, D=2, total_tokens=3 + 2 * 9, V=64, P=10, T_max=32,
                        dcap=3, Hq=2, Hkv=1, d=64)
    run(w)


# ----------------------------------------------------------------------------- fuzzed given trees
@pytest.mark.parametrize("seed", range(12))
def test_fuzz_given_trees(seed):
    rng = np.random.default_rng(seed)
    Hkv = int(rng.choice([1, 2, 4, 8]))
    rep = int(rng.choice([1, 2, 4, 8]))
    d = int(rng.choice([64, 128]))
    dtype = "bf16" if seed % 4 else "fp32"
    B = int(rng.integers(1, 6))
    P = [int(x) for x in rng.integers(0, 700, size=B)]
    T_max = int(rng.choice([32, 64]))
    sizes = [int(x) for x in rng.integers(1, T_max + 1, size=B)]
    w = gen.make_custom(cfg_id=700 + seed, B=B, P=P, mode="given", given_sizes=sizes, given_depth=int(rng.integers(1, 9)),
                        T_max=T_max, dcap=8, Hq=Hkv * rep, Hkv=Hkv, d=d, dtype=dtype, V=50)
    run(w)


def test_edge_prefix_zero_and_single_node():
    w = gen.make_custom(cfg_id=800, B=4, P=[0, 1, 63, 64], mode="given", given_sizes=[1, 64, 1, 33],
                        Hq=8, Hkv=2, d=128, dtype="bf16", V=40)
    run(w)


def test_edge_chain_of_64_with_full_depth_cap():
    w = gen.make_custom(cfg_id=801, B=2, P=[100, 5], mode="given", given_sizes=[64, 64], given_depth=63, T_max=64,
                        dcap=63, Hq=4, Hkv=4, d=64, dtype="bf16", V=100)
    run(w)


def test_edge_long_prefix_many_splits_bf16_d64():
    w = gen.make_custom(cfg_id=802, B=2, P=[9000, 4321], mode="given", given_sizes=[40, 17], Hq=16, Hkv=2, d=64,
                        dtype="bf16", V=100)
    run(w)


# ----------------------------------------------------------------------------- failure handling
def test_status_codes_and_root_only_fallback():
    """Malformed parents, depth above the cap and out-of-range sizes give the status
    codes the oracle gives, and the root-only tree everywhere downstream."""
    w = gen.make_custom(cfg_id=900, B=6, P=[50, 60, 70, 80, 90, 100], mode="given",
                        given_sizes=[10, 10, 10, 10, 10, 10], given_depth=9, dcap=3, Hq=4, Hkv=2, d=64, V=30)
    w.given_parents[0, 0] = 0            # root with a parent
    w.given_parents[1, 5] = 7            # parent after child
    w.given_parents[2, 3] = 3            # self loop
    w.given_size[3] = 0                  # empty tree
    w.given_size[4] = 65                 # larger than T_max
    w.given_parents[5, 1:10] = np.arange(0, 9)   # a chain deeper than dcap = 3
    w.given_tokens[5, 1:10] = np.arange(1, 10)
    run(w)


def test_bad_logprobs_status():
    w = gen.make_custom(cfg_id=901, B=3, mode="dynamic", K=4, D=2, total_tokens=12, V=257, P=33, d=64)
    w.logprobs[1, 3, 100] = 0.25         # a positive log-prob
    w.logprobs[2, 0, 5] = np.nan
    w.logprobs[0, 2, 7] = -np.inf        # zero probability is fine
    run(w)


def test_prefix_that_does_not_fit_gives_zero_rows():
    import torch
    from tree_attention_verification_amd.step import TreeVerifyStep
    w = gen.make_custom(cfg_id=902, B=2, P=[10, 40], mode="given", given_sizes=[5, 30], Hq=4, Hkv=2, d=64,
                        S_cap=64, V=40)
    st = TreeVerifyStep(w)
    st.O.fill_(1.0)
    st.meta()
    st.attention()
    torch.cuda.synchronize()
    o = st.O.float().cpu().numpy()
    assert (o[1, :30] == 0).all()                    # 40 + 30 > 64: zeros
    assert (o[1, 30:] == 1).all()                    # rows past the tree untouched
    assert np.isfinite(o[0, :5]).all() and (o[0, 5:] == 1).all()


def test_vocab_not_multiple_of_four_and_misaligned_rows():
    w = gen.make_custom(cfg_id=903, B=2, mode="dynamic", K=5, D=2, total_tokens=20, V=1001, P=20, d=64)
    run(w)


def test_heavy_ties_constant_rows_and_two_vocab_tiles():
    # row block 0: every entry of every row tied (the row top-K falls back to its
    # exact bisection); block 1: the 24 best entries of every row are 0.0, so every
    # candidate of the tree ties and the final selection goes by candidate id;
    # block 2: the best entries of half the rows lie past the first 32768 entries
    w = gen.make_custom(cfg_id=904, B=3, mode="dynamic", K=8, D=5, total_tokens=60, V=40000, P=40, d=64)
    w.logprobs[0, :, :] = np.float32(-np.log(40000.0))
    w.logprobs[1, :, :24] = 0.0
    w.logprobs[2, ::2, 33000:33010] = -0.5
    run(w)


def test_large_vocabulary_four_tiles():
    w = gen.make_custom(cfg_id=905, B=2, mode="dynamic", K=10, D=3, total_tokens=40, V=128256, P=50, d=64)
    run(w)


def test_nan_in_unused_cache_rows_and_query_slots():
    # rows past each request's keys and query slots past its tree hold NaN: they
    # may be read (the first key tiles of a split are loaded before the request's
    # sizes are known) but must never reach the output
    w = gen.make_custom(cfg_id=906, B=2, P=[2000, 300], mode="given", given_sizes=[40, 5], Hq=8, Hkv=2, d=128)
    nan_bf16 = np.uint16(0x7FC0)
    for b in range(w.B):
        n = int(w.prefix_len[b]) + int(w.given_size[b])
        w.Kc[b, :, n:, :] = nan_bf16
        w.Vc[b, :, n:, :] = nan_bf16
        w.Q[b, int(w.given_size[b]):] = nan_bf16
    run(w)


@pytest.mark.parametrize("Hq,Hkv,d", [(8, 8, 128), (32, 2, 128), (64, 2, 64), (16, 1, 64)])
def test_gqa_group_sizes(Hq, Hkv, d):
    # plain multi-head (1 query head per kv head) up to 32 and 16 query heads per
    # kv head: the (node, head-in-group) rows of one kv head span 1 to 32 row blocks
    w = gen.make_custom(cfg_id=910 + Hq // Hkv + d, B=3, P=[700, 1500, 64], mode="given", given_sizes=[64, 23, 41],
                        Hq=Hq, Hkv=Hkv, d=d, given_depth=7)
    run(w)


def test_kv_compact_several_layers_with_padded_layer_stride():
    # three layers whose slabs are 64 elements apart beyond their own size; paths
    # with an aliasing source (row P+2 is read for k=1 and written for k=2), an
    # empty acceptance and a longer path.  Every byte of the buffers (padding
    # included) must match the definition applied layer by layer.
    import torch
    from oracle import kv as okv
    from tree_attention_verification_amd import _lib
    n_layers, B, Hkv, S_cap, d, dcap = 3, 3, 2, 100, 64, 7
    per_layer = B * Hkv * S_cap * d
    stride = per_layer + 64
    rng = np.random.default_rng(1234)
    K0 = rng.integers(0, 2 ** 16, size=n_layers * stride, dtype=np.uint16)
    V0 = rng.integers(0, 2 ** 16, size=n_layers * stride, dtype=np.uint16)
    prefix = np.array([10, 20, 40], np.int32)
    paths = np.full((B, dcap + 1), -1, np.int32)
    paths[0, :3] = [0, 2, 3]
    paths[1, :1] = [0]
    paths[2, :4] = [0, 1, 4, 9]
    lens = np.array([2, 0, 3], np.int32)
    dev = "cuda"
    Kt = torch.from_numpy(K0.view(np.int16).copy()).to(dev)
    Vt = torch.from_numpy(V0.view(np.int16).copy()).to(dev)
    newlen = torch.full((B,), -7, dtype=torch.int32, device=dev)
    _lib.kv_compact(B, n_layers, Hkv, d, 2, Kt, Vt, S_cap, stride, torch.from_numpy(prefix).to(dev),
                    torch.from_numpy(paths).to(dev), torch.from_numpy(lens).to(dev), dcap, newlen)
    torch.cuda.synchronize()
    Kg = Kt.cpu().numpy().view(np.uint16)
    Vg = Vt.cpu().numpy().view(np.uint16)

    def layered(x):
        return np.stack([x[l * stride:l * stride + per_layer].reshape(B, Hkv, S_cap, d) for l in range(n_layers)])
    Kr, Vr, nl = okv.kv_compact(layered(K0), layered(V0), prefix, paths, lens)
    np.testing.assert_array_equal(layered(Kg), Kr)
    np.testing.assert_array_equal(layered(Vg), Vr)
    for l in range(n_layers):   # the padding between layers is untouched
        np.testing.assert_array_equal(Kg[l * stride + per_layer:(l + 1) * stride], K0[l * stride + per_layer:(l + 1) * stride])
        np.testing.assert_array_equal(Vg[l * stride + per_layer:(l + 1) * stride], V0[l * stride + per_layer:(l + 1) * stride])
    np.testing.assert_array_equal(newlen.cpu().numpy(), nl)


# ----------------------------------------------------------------------------- fused entry points
def _fused_cases():
    return {
        "tiny-static-fp32": lambda: gen.make_workload(1),
        "eagle2-b1-p2048": lambda: gen.make_workload(2),
        "ragged-b16": lambda: gen.make_workload(3),
        "random-trees-reduced": lambda: gen.make_workload(5, batch=12, prefix=777),
        "dynamic-K16": lambda: gen.make_custom(cfg_id=516, mode="dynamic", K=16, D=2, total_tokens=63, V=777,
                                               P=70, Hq=4, Hkv=2, d=64, dtype="bf16"),
        "dynamic-deeper-than-dcap": lambda: gen.make_custom(cfg_id=517, mode="dynamic", K=1, D=6, total_tokens=6,
                                                            V=300, P=40, dcap=3, Hq=4, Hkv=2, d=64),
        "static-chain-20": lambda: gen.make_custom(cfg_id=620, mode="static", branching=[1] * 20, V=1003, P=65,
                                                   Hq=8, Hkv=4, d=128, dtype="bf16", dcap=20),
        "static-deeper-than-dcap": lambda: gen.make_custom(cfg_id=621, mode="static", branching=[2, 2, 2], V=500,
                                                           P=12, Hq=4, Hkv=2, d=64, dcap=2),
        "given-trees": lambda: gen.make_custom(cfg_id=790, B=3, P=[5, 300, 64], mode="given",
                                               given_sizes=[64, 17, 1], given_depth=7, T_max=64, dcap=8, Hq=8,
                                               Hkv=2, d=128, dtype="bf16", V=50),
    }


@pytest.mark.parametrize("case", list(_fused_cases()))
def test_fused_calls(case):
    """tree_build_meta and tree_accept_compact give the oracle's results."""
    run(_fused_cases()[case](), fused=True)


def test_fused_bad_logprobs_status():
    w = gen.make_custom(cfg_id=901, B=3, mode="dynamic", K=4, D=2, total_tokens=12, V=257, P=33, d=64)
    w.logprobs[1, 3, 100] = 0.25
    w.logprobs[2, 0, 5] = np.nan
    run(w, fused=True)


def test_many_requests_beyond_the_reordered_batch():
    """More than 64 requests: the splits follow the cache capacity (no reordering)."""
    rng = np.random.default_rng(77)
    B = 70
    P = [int(x) for x in rng.integers(0, 400, size=B)]
    sizes = [int(x) for x in rng.integers(1, 33, size=B)]
    w = gen.make_custom(cfg_id=910, B=B, P=P, mode="given", given_sizes=sizes, given_depth=5, T_max=32, dcap=6,
                        Hq=8, Hkv=2, d=128, dtype="bf16", V=50)
    run(w)


def test_ragged_batch_with_short_and_empty_splits():
    """Requests much shorter than the longest: some of their key splits are empty."""
    w = gen.make_custom(cfg_id=911, B=5, P=[3000, 10, 0, 700, 64], mode="given", given_sizes=[40, 3, 1, 64, 17],
                        given_depth=6, T_max=64, dcap=8, Hq=16, Hkv=4, d=128, dtype="bf16", V=50)
    run(w)


def test_single_request_two_stage_plan_d64():
    """One request whose 8-wavefront plan leaves the chip idle: 4-wavefront workgroups with two stage
    buffers, at d = 64 (the benchmark's request covers d = 128)."""
    w = gen.make_custom(cfg_id=912, B=1, P=[1500], mode="given", given_sizes=[50], given_depth=6, T_max=64,
                        dcap=8, Hq=16, Hkv=2, d=64, dtype="bf16", V=50)
    run(w)
