"""The C-ABI library without a GPU: it loads, exports every function the header
declares, and rejects invalid arguments on the host before touching the device."""
import ctypes

import pytest

from tree_attention_verification_amd import _lib as tv


def test_library_exports_every_declared_symbol():
    L = tv.lib()
    names = tv.declared_functions()
    assert {"tree_build", "tree_mask_positions", "tree_attention", "tree_accept", "kv_compact"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_error_and_status_strings():
    assert tv.error_string(tv.TV_EINVAL) == "invalid argument"
    assert tv.error_string(tv.TV_EWORKSPACE).startswith("workspace")
    assert tv.status_string(tv.TV_ST_DEPTH).startswith("tree deeper")


X = ctypes.c_void_p(0x1000)   # a non-null dummy; never dereferenced on the error paths below


def test_tree_build_host_validation():
    L = tv.lib()
    br = (ctypes.c_int * 3)(2, 2, 1)
    # B = 0
    assert L.tree_build(0, 0, 100, 4, 2, 5, None, 0, X, 9, X, 64, X, X, X, None, X, X, 1 << 20, None) == tv.TV_EINVAL
    # total_tokens larger than K + D*K^2
    assert L.tree_build(0, 1, 100, 2, 1, 7, None, 0, X, 3, X, 64, X, X, X, None, X, X, 1 << 20, None) == tv.TV_EINVAL
    # rows_per_req != 1 + D*K
    assert L.tree_build(0, 1, 100, 2, 1, 5, None, 0, X, 4, X, 64, X, X, X, None, X, X, 1 << 20, None) == tv.TV_EINVAL
    # K above the supported maximum
    assert L.tree_build(0, 1, 100, 17, 1, 5, None, 0, X, 18, X, 64, X, X, X, None, X, X, 1 << 20,
                        None) == tv.TV_EUNSUPPORTED
    # tree does not fit T_max
    assert L.tree_build(0, 1, 100, 4, 2, 40, None, 0, X, 9, X, 32, X, X, X, None, X, X, 1 << 20, None) == tv.TV_EINVAL
    # workspace too small
    assert L.tree_build(0, 1, 100, 4, 2, 10, None, 0, X, 9, X, 64, X, X, X, None, X, X, 8, None) == tv.TV_EWORKSPACE
    # static: rows_per_req must be the number of expanded nodes (7 for [2,2,1])
    assert L.tree_build(1, 1, 100, 0, 0, 0, br, 3, X, 6, X, 64, X, X, X, None, X, X, 1 << 20, None) == tv.TV_EINVAL
    # null output
    assert L.tree_build(1, 1, 100, 0, 0, 0, br, 3, X, 7, X, 64, None, X, X, None, X, X, 1 << 20, None) == tv.TV_EINVAL


def test_other_calls_host_validation():
    L = tv.lib()
    # tree_mask_positions: dcap must be < T_max, T_max <= 256
    assert L.tree_mask_positions(1, 64, 64, X, X, X, X, X, X, X, X, None, None, None, X, None) == tv.TV_EINVAL
    assert L.tree_mask_positions(1, 257, 7, X, X, X, X, X, X, X, X, None, None, None, X, None) == tv.TV_EUNSUPPORTED
    # tree_attention: Hq % Hkv, head dim, dtype, misaligned pointers, workspace
    args = dict(Q=X, K=X, V=X)
    assert L.tree_attention(0, 1, 64, 6, 4, 128, X, X, X, 4096, X, X, X, X, 0.0, X, None, 0, None) == tv.TV_EINVAL
    assert L.tree_attention(0, 1, 64, 8, 4, 96, X, X, X, 4096, X, X, X, X, 0.0, X, None, 0, None) == tv.TV_EUNSUPPORTED
    assert L.tree_attention(7, 1, 64, 8, 4, 128, X, X, X, 4096, X, X, X, X, 0.0, X, None, 0, None) == tv.TV_EUNSUPPORTED
    odd = ctypes.c_void_p(0x1002)
    assert L.tree_attention(0, 1, 64, 8, 4, 128, odd, X, X, 4096, X, X, X, X, 0.0, X, None, 0, None) == tv.TV_EINVAL
    need = tv.tree_attention_workspace_bytes(0, 1, 64, 32, 8, 128, 65536)
    assert need > 0
    assert L.tree_attention(0, 1, 64, 32, 8, 128, X, X, X, 65536, X, X, X, X, 0.0, X, X, need - 1,
                            None) == tv.TV_EWORKSPACE
    # tree_accept: dcap >= T_max
    assert L.tree_accept(1, 16, 16, X, X, X, X, X, X, X, X, None) == tv.TV_EINVAL
    # kv_compact: row bytes must be a multiple of 16
    assert L.kv_compact(1, 1, 8, 100, 2, X, X, 4096, 0, X, X, X, 7, None, None) == tv.TV_EUNSUPPORTED
    assert L.kv_compact(1, 1, 8, 128, 3, X, X, 4096, 0, X, X, X, 7, None, None) == tv.TV_EINVAL


def test_compaction_refuses_new_prefix_len_aliasing_its_inputs():
    # new_prefix_len written over prefix_len (a prefix grown in place), accept_len or
    # accept_path would race with the workgroups still reading them
    L = tv.lib()
    pre, path, alen, new = (ctypes.c_void_p(a) for a in (0x10000, 0x20000, 0x30000, 0x40000))
    inside = ctypes.c_void_p(0x20000 + 4 * 8 * 3)          # inside accept_path [4][8]
    # kv_compact(B, n_layers, Hkv, d, elem, K, V, S_cap, stride, prefix, path, len, dcap, newlen, stream)
    assert L.kv_compact(4, 1, 8, 128, 2, X, X, 4096, 0, pre, path, alen, 7, pre, None) == tv.TV_EINVAL
    assert L.kv_compact(4, 1, 8, 128, 2, X, X, 4096, 0, pre, path, alen, 7, alen, None) == tv.TV_EINVAL
    assert L.kv_compact(4, 1, 8, 128, 2, X, X, 4096, 0, pre, path, alen, 7, inside, None) == tv.TV_EINVAL
    shifted = ctypes.c_void_p(0x10000 + 12)                # overlapping the last entry
    assert L.kv_compact(4, 1, 8, 128, 2, X, X, 4096, 0, pre, path, alen, 7, shifted, None) == tv.TV_EINVAL
    assert L.kv_compact_paged(4, 1, 8, 128, 2, X, X, 100, 16, X, 10, 0, pre, path, alen, 7, pre,
                              None) == tv.TV_EINVAL
    # tree_accept_compact(B, T_max, dcap, tokens, parents, size, predict, status, len, path, bonus, n_layers, Hkv,
    #                     d, elem, K, V, S_cap, stride, prefix, newlen, stream)
    assert L.tree_accept_compact(4, 16, 7, X, X, X, X, X, alen, path, X, 1, 8, 128, 2, X, X, 4096, 0, pre, pre,
                                 None) == tv.TV_EINVAL
    assert L.tree_accept_compact_paged(4, 16, 7, X, X, X, X, X, alen, path, X, 1, 8, 128, 2, X, X, 100, 16, X, 10,
                                       0, pre, pre, None) == tv.TV_EINVAL


def test_python_binding_refuses_host_tensors():
    import torch
    with pytest.raises(ValueError):
        tv.tree_accept(1, 8, 3, torch.zeros(1, 8, dtype=torch.int32), None, None, None, None, None, None, None)


def test_paged_calls_host_validation():
    L = tv.lib()
    # tree_attention_paged(dtype, B, T_max, Hq, Hkv, d, Q, Kp, Vp, num_blocks, tokens_per_block, table,
    #                      max_blocks, prefix, size, mask, status, scale, O, ws, ws_bytes, stream)
    ok_args = (0, 1, 64, 8, 4, 128, X, X, X, 1000, 16, X, 64, X, X, X, X, 0.0, X, None, 0, None)
    bad_bs = list(ok_args); bad_bs[10] = 24          # not a power of two
    assert L.tree_attention_paged(*bad_bs) == tv.TV_EINVAL
    big_bs = list(ok_args); big_bs[10] = 2048        # above 1024 tokens per block
    assert L.tree_attention_paged(*big_bs) == tv.TV_EINVAL
    no_table = list(ok_args); no_table[11] = None
    assert L.tree_attention_paged(*no_table) == tv.TV_EINVAL
    no_blocks = list(ok_args); no_blocks[9] = 0
    assert L.tree_attention_paged(*no_blocks) == tv.TV_EINVAL
    bad_d = list(ok_args); bad_d[5] = 96
    assert L.tree_attention_paged(*bad_d) == tv.TV_EUNSUPPORTED
    # the capacity max_blocks * tokens_per_block sizes the workspace like S_cap
    need = tv.tree_attention_workspace_bytes(0, 1, 64, 32, 8, 128, 4096 * 16)
    assert need > 0
    small_ws = (0, 1, 64, 32, 8, 128, X, X, X, 100000, 16, X, 4096, X, X, X, X, 0.0, X, X, need - 1, None)
    assert L.tree_attention_paged(*small_ws) == tv.TV_EWORKSPACE
    # kv_compact_paged(B, n_layers, Hkv, d, elem, Kp, Vp, num_blocks, bs, table, max_blocks, stride, prefix,
    #                  path, len, dcap, newlen, stream)
    assert L.kv_compact_paged(1, 1, 8, 128, 2, X, X, 100, 3, X, 10, 0, X, X, X, 7, None, None) == tv.TV_EINVAL
    assert L.kv_compact_paged(1, 1, 8, 128, 2, X, X, 100, 16, None, 10, 0, X, X, X, 7, None, None) == tv.TV_EINVAL
    assert L.kv_compact_paged(1, 1, 8, 100, 2, X, X, 100, 16, X, 10, 0, X, X, X, 7, None, None) == tv.TV_EUNSUPPORTED
    # several layers need a layer stride of at least one pool
    assert L.kv_compact_paged(1, 2, 8, 128, 2, X, X, 100, 16, X, 10, 100 * 8 * 16 * 128 - 8, X, X, X, 7, None,
                              None) == tv.TV_EINVAL
    # tree_accept_compact_paged: tree_accept's checks first (dcap >= T_max)
    assert L.tree_accept_compact_paged(1, 16, 16, X, X, X, X, X, X, X, X, 1, 8, 128, 2, X, X, 100, 16, X, 10, 0,
                                       X, None, None) == tv.TV_EINVAL


def test_layer_calls_host_validation():
    L = tv.lib()
    need = tv.tree_build_layer_workspace_bytes(2, 32000, 10, 6)
    assert need > 0 and tv.tree_build_layer_workspace_bytes(2, 32000, 17, 6) == 0
    # tree_build_layer(layer, B, V, K, D, rows, logits, state, state_bytes, ftok, fpar, stream)
    assert L.tree_build_layer(7, 2, 32000, 10, 6, X, 0, X, need, X, None, None) == tv.TV_EINVAL      # layer > D
    assert L.tree_build_layer(-1, 2, 32000, 10, 6, X, 0, X, need, X, None, None) == tv.TV_EINVAL
    assert L.tree_build_layer(0, 2, 32000, 17, 6, X, 0, X, need, X, None, None) == tv.TV_EUNSUPPORTED
    assert L.tree_build_layer(0, 2, 8, 10, 6, X, 0, X, need, X, None, None) == tv.TV_EINVAL          # K > V
    assert L.tree_build_layer(0, 2, 32000, 10, 6, None, 0, X, need, X, None, None) == tv.TV_EINVAL
    assert L.tree_build_layer(0, 2, 32000, 10, 6, X, 1, X, need - 1, X, None, None) == tv.TV_EWORKSPACE
    # tree_build_finish(B, V, K, D, total, root, T_max, state, bytes, tok, par, size, score, status, dcap, prefix, ...)
    tail = (X, X, X, X, X, X, X, X, None)
    assert L.tree_build_finish(2, 32000, 10, 6, 611, X, 64, X, need, X, X, X, None, X, 7, None,
                               *tail) == tv.TV_EINVAL   # total_tokens > C
    assert L.tree_build_finish(2, 32000, 10, 6, 64, X, 64, X, need, X, X, X, None, X, 7, None,
                               *tail) == tv.TV_EINVAL   # total_tokens + 1 > T_max
    assert L.tree_build_finish(2, 32000, 10, 6, 60, X, 257, X, need, X, X, X, None, X, 7, None,
                               *tail) == tv.TV_EUNSUPPORTED
    assert L.tree_build_finish(2, 32000, 10, 6, 60, X, 64, X, need, X, X, X, None, X, 64, X,
                               *tail) == tv.TV_EINVAL   # dcap >= T_max with metadata
    assert L.tree_build_finish(2, 32000, 10, 6, 60, X, 64, X, need - 1, X, X, X, None, X, 7, None,
                               *tail) == tv.TV_EWORKSPACE


def test_accept_sample_host_validation():
    L = tv.lib()
    # tree_accept_sample(B, T_max, dcap, V, tokens, parents, size, probs, uniforms, status, len, path, bonus,
    #                    ws, ws_bytes, stream)
    assert L.tree_accept_sample(1, 16, 16, 100, X, X, X, X, X, X, X, X, X, None, 0, None) == tv.TV_EINVAL  # dcap
    assert L.tree_accept_sample(1, 257, 7, 100, X, X, X, X, X, X, X, X, X, None, 0, None) == tv.TV_EUNSUPPORTED
    assert L.tree_accept_sample(1, 16, 7, 0, X, X, X, X, X, X, X, X, X, None, 0, None) == tv.TV_EINVAL      # V = 0
    assert L.tree_accept_sample(1, 16, 7, 100, X, X, X, None, X, X, X, X, X, None, 0, None) == tv.TV_EINVAL
    assert L.tree_accept_sample(0, 16, 7, 100, X, X, X, X, X, X, X, X, X, None, 0, None) == tv.TV_EINVAL
    # the optional workspace: B x T_max float64 sums, 8-byte aligned
    assert tv.tree_accept_sample_workspace_bytes(3, 16) == 3 * 16 * 8
    assert tv.tree_accept_sample_workspace_bytes(0, 16) == 0
    ws = ctypes.c_void_p(0x200000)
    assert L.tree_accept_sample(3, 16, 7, 100, X, X, X, X, X, X, X, X, X, ws, 3 * 16 * 8 - 1,
                                None) == tv.TV_EWORKSPACE
    assert L.tree_accept_sample(3, 16, 7, 100, X, X, X, X, X, X, X, X, X, ctypes.c_void_p(0x200004), 4096,
                                None) == tv.TV_EWORKSPACE


def test_rope_call_host_validation():
    L = tv.lib()
    # tree_attention_rope(dtype, B, T_max, Hq, Hkv, d, Q, K, V, S_cap, prefix, size, mask, status, theta, scale, O,
    #                     ws, ws_bytes, stream)
    assert L.tree_attention_rope(0, 1, 64, 8, 4, 128, X, X, X, 4096, X, X, X, X, 0.5, 0.0, X, None, 0,
                                 None) == tv.TV_EINVAL          # theta <= 1
    assert L.tree_attention_rope(0, 1, 64, 8, 4, 128, X, X, X, (1 << 24) + 1, X, X, X, X, 1e4, 0.0, X, None, 0,
                                 None) == tv.TV_EUNSUPPORTED    # positions past 2^24
    assert L.tree_attention_rope(0, 1, 64, 8, 4, 96, X, X, X, 4096, X, X, X, X, 1e4, 0.0, X, None, 0,
                                 None) == tv.TV_EUNSUPPORTED


def test_sampling_calls_host_validation():
    L = tv.lib()
    # tree_sampling_probs(B, T_max, V, logits, size, status, temperature, top_k, top_p, min_p, probs, stream)
    assert L.tree_sampling_probs(0, 4, 100, X, X, None, X, X, X, X, ctypes.c_void_p(0x100000), None) == tv.TV_EINVAL
    assert L.tree_sampling_probs(1, 257, 100, X, X, None, X, X, X, X, ctypes.c_void_p(0x100000),
                                 None) == tv.TV_EUNSUPPORTED
    assert L.tree_sampling_probs(1, 4, 262145, X, X, None, X, X, X, X, ctypes.c_void_p(0x10000000),
                                 None) == tv.TV_EUNSUPPORTED
    assert L.tree_sampling_probs(1, 4, 100, X, X, None, None, X, X, X, ctypes.c_void_p(0x100000),
                                 None) == tv.TV_EINVAL
    # the output overlapping the logits
    assert L.tree_sampling_probs(1, 4, 100, X, X, None, X, X, X, X, ctypes.c_void_p(0x1000 + 400),
                                 None) == tv.TV_EINVAL
    # tree_accept_sample_draft(B, T_max, dcap, V, tokens, parents, size, p, q, u, status, wr, len, path, bonus,
    #                          ws, ws_bytes, stream)
    assert tv.tree_accept_sample_draft_workspace_bytes(3, 1000) == 3 * 1000 * 8
    ws = ctypes.c_void_p(0x200000)
    ok = (1, 16, 7, 100, X, X, X, X, X, X, X, 1, X, X, X, ws, 800, None)
    bad = lambda i, v: tuple(v if j == i else a for j, a in enumerate(ok))
    assert L.tree_accept_sample_draft(*bad(2, 16)) == tv.TV_EINVAL                 # dcap >= T_max
    assert L.tree_accept_sample_draft(*bad(1, 257)) == tv.TV_EUNSUPPORTED
    assert L.tree_accept_sample_draft(*bad(3, 262145)) == tv.TV_EUNSUPPORTED
    assert L.tree_accept_sample_draft(*bad(8, None)) == tv.TV_EINVAL                # no draft rows
    assert L.tree_accept_sample_draft(*bad(16, 799)) == tv.TV_EWORKSPACE            # workspace too small
    assert L.tree_accept_sample_draft(*bad(15, ctypes.c_void_p(0x200004))) == tv.TV_EWORKSPACE   # misaligned
    assert L.tree_accept_sample_draft(*bad(15, None)) == tv.TV_EWORKSPACE


def test_noalloc_attention_refuses_partials_beyond_its_scratch():
    # 511 requests with 256 query rows each and two key splits need ~66 MiB of split
    # partials: more than the 64 MiB scratch, refused before any device call
    L = tv.lib()
    cap = tv.tree_attention_noalloc_max_bytes()
    assert cap == 64 << 20
    assert tv.tree_attention_workspace_bytes(0, 511, 64, 4, 1, 128, 4096) > cap
    assert L.tree_attention_noalloc(0, 511, 64, 4, 1, 128, X, X, X, 4096, X, X, X, X, 0.0, X,
                                    None) == tv.TV_EWORKSPACE
    # the argument checks of tree_attention still apply
    assert L.tree_attention_noalloc(0, 1, 64, 6, 4, 128, X, X, X, 4096, X, X, X, X, 0.0, X, None) == tv.TV_EINVAL
