"""GPU parity for trees of more than 64 nodes (T_max up to 256; mask rows of up to
8 words), against the oracle, which has no node limit.

The metadata of such trees comes from a 256-thread workgroup (one thread per node,
pointer jumping through LDS), the greedy walk from a workgroup-wide walk, the
attention mask from a window of up to three mask words per key tile, rejection
sampling from four nodes per lane.  Cases: given random trees of 65..256 nodes
(depth up to 7 and up to 40), dynamic trees of 255 draft nodes (tree_build and
tree_build_meta), static trees of 85 and 121 nodes, T_max = 128 and 256, the
fused calls, rejection sampling, and the paged cache.  Bars as everywhere else.
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


@pytest.mark.parametrize("T_max,sizes,depth", [(256, [256, 200, 65, 1], 7), (256, [256, 180, 90, 33], 40),
                                               (128, [128, 100, 70, 64], 6)])
def test_big_given_trees(T_max, sizes, depth):
    w = gen.make_custom(cfg_id=1500 + depth + T_max, B=len(sizes), P=[1000, 37, 300, 0], mode="given",
                        given_sizes=sizes, given_depth=depth, T_max=T_max, dcap=min(63, T_max - 1), Hq=8, Hkv=2,
                        d=128, dtype="bf16", V=500, accept_prob=0.9)
    r = run(w)
    assert r["tree_size"].max() > 64


@pytest.mark.parametrize("fused", [False, True])
def test_big_dynamic_trees(fused):
    # K = 16, D = 2: 528 candidates, 255 kept (T = 256)
    w = gen.make_custom(cfg_id=1510, B=3, P=[200, 5, 64], mode="dynamic", K=16, D=2, total_tokens=255, V=2000,
                        T_max=256, dcap=8, Hq=16, Hkv=4, d=128, dtype="bf16")
    r = run(w, fused=fused)
    assert (r["tree_size"] == 256).all()


@pytest.mark.parametrize("br", [[4, 4, 4], [3, 3, 3, 3]])
def test_big_static_trees(br):
    w = gen.make_custom(cfg_id=1520 + len(br), B=2, P=[100, 7], mode="static", branching=br, V=300, T_max=128,
                        dcap=6, Hq=8, Hkv=4, d=64, dtype="bf16")
    r = run(w, fused=True)
    assert r["tree_size"].min() > 64


def test_big_trees_fp32_and_paged():
    w = gen.make_custom(cfg_id=1530, B=3, P=[90, 300, 17], mode="given", given_sizes=[150, 256, 80], given_depth=9,
                        T_max=256, dcap=12, Hq=4, Hkv=2, d=64, dtype="fp32", V=300)
    run(w)
    w2 = gen.make_custom(cfg_id=1531, B=3, P=[900, 30, 170], mode="given", given_sizes=[256, 120, 97],
                         given_depth=8, T_max=256, dcap=10, Hq=8, Hkv=2, d=128, dtype="bf16", V=300)
    run(w2, paged=gen.paged_layout(w2, 16))


def test_big_trees_sampling():
    from tests.test_gpu_sampling import run_sampling
    w = gen.make_custom(cfg_id=1540, B=4, mode="given", given_sizes=[256, 200, 130, 66], given_depth=5, V=3000,
                        P=4, T_max=256, dcap=20, accept_prob=0.9)
    got, _ = run_sampling(w)
    assert got["accept_len"].max() >= 2
