"""GPU: tree_attention_noalloc, the attention entry point that allocates nothing
(for callers that cannot call hipMalloc: its split-KV partials live in a scratch
array the library holds on each GPU), against tree_attention with a caller
workspace.  Two calls in a row, the second on a smaller input (the scratch keeps
the first call's partials), each bit-identical to tree_attention's output (the
same kernels and launch plan) and within the bf16 bar of the oracle."""
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


def _noalloc_against_workspace_call(w):
    import torch
    from oracle import attention as oa
    from tests.parity_util import check_attention
    from tree_attention_verification_amd import _lib as tv
    from tree_attention_verification_amd.step import TreeVerifyStep
    st = TreeVerifyStep(w)
    if w.mode == "given":
        st.meta()
    else:
        st.build_meta()
    torch.cuda.synchronize()
    need = tv.tree_attention_workspace_bytes(st.dtype_code, w.B, w.T_max, w.Hq, w.Hkv, w.d, w.S_cap)
    assert 0 < need <= tv.tree_attention_noalloc_max_bytes(), "the case must use the scratch (split keys)"
    st.attention()                                     # tree_attention, caller workspace
    O2 = torch.zeros_like(st.O)
    tv.tree_attention_noalloc(st.dtype_code, w.B, w.T_max, w.Hq, w.Hkv, w.d, st.Q, st.Kc[0], st.Vc[0], w.S_cap,
                              st.prefix_len, st.tree_size, st.tree_mask, st.status, 0.0, O2)
    torch.cuda.synchronize()
    ref_call = st.out_host()
    got = O2.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref_call), "noalloc output differs from tree_attention's"
    tree, meta = st.tree_host(), st.meta_host()
    ref = oa.tree_attention(w.Q, w.Kc, w.Vc, w.prefix_len, tree["tree_size"], meta["tree_mask"],
                            status=meta["status"])
    check_attention(got, ref, w, tree["tree_size"], meta["status"], "tree_attention_noalloc")


def test_noalloc_two_calls_second_smaller():
    # 1: two requests over 9000-token prefixes, 61-node trees, 64 query heads (8 splits, ~33 MiB of partials)
    _noalloc_against_workspace_call(gen.make_workload(4, batch=2, prefix=9000))
    # 2: one request over 2048 tokens (7 splits, ~4 MiB): reads only what it wrote
    _noalloc_against_workspace_call(gen.make_workload(2))
