"""GPU parity of tree_attention_rope (the queries' rotary embedding fused into the
attention kernel) against the oracle's attention of the queries rotated in float64
at position prefix + depth.  Bars as for tree_attention (bf16: 2e-2 + 1e-2 |ref| per
element and 1e-2 relative Frobenius; fp32: 1e-4).  Positions up to ~32800 (the
long-context workload) check the angle reduction; theta 10^4 and 5*10^5; d = 64 and
128; one request, ragged batches, fp32, the fused calls.
"""
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


def run(w, theta, **kw):
    from tests.parity_util import run_pipeline_and_compare
    return run_pipeline_and_compare(w, rope_theta=theta, **kw)


def test_rope_dynamic_batch1():
    run(gen.make_workload(2), 500000.0)


def test_rope_ragged_batch16():
    run(gen.make_workload(3), 10000.0)


def test_rope_fp32_static_tree():
    run(gen.make_workload(1), 10000.0)


def test_rope_long_context_full_size():
    # positions ~32800, every written row
    run(gen.make_workload(4), 500000.0)


@pytest.mark.parametrize("theta", [10000.0, 1.0e6])
def test_rope_ragged_d64_given_trees(theta):
    w = gen.make_custom(cfg_id=1400, B=5, P=[3000, 10, 0, 700, 64], mode="given", given_sizes=[40, 3, 1, 64, 17],
                        given_depth=6, T_max=64, dcap=8, Hq=16, Hkv=4, d=64, dtype="bf16", V=50)
    run(w, theta)


def test_rope_fused_calls():
    run(gen.make_workload(5, batch=12, prefix=777), 10000.0, fused=True)
