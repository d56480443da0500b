"""ctypes binding to libtreeverify.so -- argument marshalling only.

Every function has the name and argument order of the C call it wraps
(include/treeverify.h).  Device buffers are passed as torch tensors on the GPU
(their data_ptr() is handed to the library), sizes as Python ints, and the
stream is torch's current HIP stream unless one is given.  No computation of
the step happens here: every step runs in the library's HIP kernels.  There is
no fallback -- if the library is missing or a tensor is not on the GPU the call
raises.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; TREEVERIFY_LIB names another build of the same library (e.g. one
# whose host code is compiled with sanitizers, for the host-validation tests)
LIB_PATH = os.environ.get("TREEVERIFY_LIB") or os.path.join(_HERE, "libtreeverify.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "treeverify.h")

TV_OK, TV_EINVAL, TV_EUNSUPPORTED, TV_EWORKSPACE, TV_ELAUNCH = 0, -1, -2, -3, -4
TV_ST_OK, TV_ST_PARENTS, TV_ST_DEPTH, TV_ST_SIZE, TV_ST_LOGPROB = 0, 1, 2, 3, 4
MODE_DYNAMIC, MODE_STATIC = 0, 1
DTYPE_BF16, DTYPE_FP32 = 0, 1


class TVError(RuntimeError):
    def __init__(self, call: str, code: int):
        super().__init__(f"{call} failed: {error_string(code)} ({code})")
        self.code = code


_lib = None

P = ctypes.c_void_p
I = ctypes.c_int
LL = ctypes.c_longlong
SZ = ctypes.c_size_t
F = ctypes.c_float

_SIGS = {
    "tree_build_workspace_bytes": (SZ, [I, I, I, I, I]),
    "tree_build": (I, [I, I, I, I, I, I, P, I, P, I, P, I, P, P, P, P, P, P, SZ, P]),
    "tree_mask_positions": (I, [I, I, I, P, P, P, P, P, P, P, P, P, P, P, P, P]),
    "tree_build_meta": (I, [I, I, I, I, I, I, P, I, P, I, P, I, P, P, P, P, P, P, SZ, I, P, P, P, P, P, P, P, P, P]),
    "tree_attention_workspace_bytes": (SZ, [I, I, I, I, I, I, LL]),
    "tree_attention": (I, [I, I, I, I, I, I, P, P, P, LL, P, P, P, P, F, P, P, SZ, P]),
    "tree_attention_noalloc": (I, [I, I, I, I, I, I, P, P, P, LL, P, P, P, P, F, P, P]),
    "tree_attention_noalloc_max_bytes": (SZ, []),
    "tree_accept": (I, [I, I, I, P, P, P, P, P, P, P, P, P]),
    "kv_compact": (I, [I, I, I, I, I, P, P, LL, LL, P, P, P, I, P, P]),
    "tree_accept_compact": (I, [I, I, I, P, P, P, P, P, P, P, P, I, I, I, I, P, P, LL, LL, P, P, P]),
    "tree_attention_paged": (I, [I, I, I, I, I, I, P, P, P, LL, I, P, I, P, P, P, P, F, P, P, SZ, P]),
    "kv_compact_paged": (I, [I, I, I, I, I, P, P, LL, I, P, I, LL, P, P, P, I, P, P]),
    "tree_accept_compact_paged": (I, [I, I, I, P, P, P, P, P, P, P, P, I, I, I, I, P, P, LL, I, P, I, LL, P, P, P]),
    "tree_build_layer_workspace_bytes": (SZ, [I, I, I, I]),
    "tree_build_layer": (I, [I, I, I, I, I, P, I, P, SZ, P, P, P]),
    "tree_build_finish": (I, [I, I, I, I, I, P, I, P, SZ, P, P, P, P, P, I, P, P, P, P, P, P, P, P, P]),
    "tree_accept_sample_workspace_bytes": (SZ, [I, I]),
    "tree_accept_sample": (I, [I, I, I, I, P, P, P, P, P, P, P, P, P, P, SZ, P]),
    "tree_attention_rope": (I, [I, I, I, I, I, I, P, P, P, LL, P, P, P, P, F, F, P, P, SZ, P]),
    "tree_sampling_probs": (I, [I, I, I, P, P, P, P, P, P, P, P, P]),
    "tree_accept_sample_draft_workspace_bytes": (SZ, [I, I]),
    "tree_accept_sample_draft": (I, [I, I, I, I, P, P, P, P, P, P, P, I, P, P, P, P, SZ, P]),
    "tv_error_string": (ctypes.c_char_p, [I]),
    "tv_status_string": (ctypes.c_char_p, [I]),
}


def lib():
    """Load the in-tree library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m tree_attention_verification_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def declared_functions():
    """Names of the functions include/treeverify.h declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def error_string(code: int) -> str:
    return lib().tv_error_string(int(code)).decode()


def status_string(st: int) -> str:
    return lib().tv_status_string(int(st)).decode()


def _dev(t, name):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name}: tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name}: tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ws(ws):
    if ws is None:
        return None, 0
    return _dev(ws, "workspace"), ws.numel() * ws.element_size()


def _check(name, rc):
    if rc != TV_OK:
        raise TVError(name, rc)


def tree_build_workspace_bytes(mode, B, V, K, rows_per_req) -> int:
    return int(lib().tree_build_workspace_bytes(mode, B, V, K, rows_per_req))


def tree_build(mode, B, V, K, D, total_tokens, branching, logprobs, rows_per_req, root_token, T_max,
               draft_tokens, parents, tree_size, node_score, status, workspace, stream=None):
    br = None
    n_levels = 0
    if branching:
        n_levels = len(branching)
        br = (ctypes.c_int * n_levels)(*[int(x) for x in branching])
    wp, wn = _ws(workspace)
    rc = lib().tree_build(mode, B, V, K, D, total_tokens, br, n_levels, _dev(logprobs, "logprobs"), rows_per_req,
                          _dev(root_token, "root_token"), T_max, _dev(draft_tokens, "draft_tokens"),
                          _dev(parents, "parents"), _dev(tree_size, "tree_size"), _dev(node_score, "node_score"),
                          _dev(status, "status"), wp, wn, _stream(stream))
    _check("tree_build", rc)


def tree_build_meta(mode, B, V, K, D, total_tokens, branching, logprobs, rows_per_req, root_token, T_max,
                    draft_tokens, parents, tree_size, node_score, status, workspace, dcap, prefix_len, tree_mask,
                    tree_position_ids, positions, retrieve_indices, leaf_count, first_child, next_sibling,
                    stream=None):
    br = None
    n_levels = 0
    if branching:
        n_levels = len(branching)
        br = (ctypes.c_int * n_levels)(*[int(x) for x in branching])
    wp, wn = _ws(workspace)
    rc = lib().tree_build_meta(mode, B, V, K, D, total_tokens, br, n_levels, _dev(logprobs, "logprobs"),
                               rows_per_req, _dev(root_token, "root_token"), T_max,
                               _dev(draft_tokens, "draft_tokens"), _dev(parents, "parents"),
                               _dev(tree_size, "tree_size"), _dev(node_score, "node_score"), _dev(status, "status"),
                               wp, wn, dcap, _dev(prefix_len, "prefix_len"), _dev(tree_mask, "tree_mask"),
                               _dev(tree_position_ids, "tree_position_ids"), _dev(positions, "positions"),
                               _dev(retrieve_indices, "retrieve_indices"), _dev(leaf_count, "leaf_count"),
                               _dev(first_child, "first_child"), _dev(next_sibling, "next_sibling"),
                               _stream(stream))
    _check("tree_build_meta", rc)


def tree_mask_positions(B, T_max, dcap, parents, tree_size, prefix_len, tree_mask, tree_position_ids, positions,
                        retrieve_indices, leaf_count, first_child, next_sibling, status_in, status_out, stream=None):
    rc = lib().tree_mask_positions(B, T_max, dcap, _dev(parents, "parents"), _dev(tree_size, "tree_size"),
                                   _dev(prefix_len, "prefix_len"), _dev(tree_mask, "tree_mask"),
                                   _dev(tree_position_ids, "tree_position_ids"), _dev(positions, "positions"),
                                   _dev(retrieve_indices, "retrieve_indices"), _dev(leaf_count, "leaf_count"),
                                   _dev(first_child, "first_child"), _dev(next_sibling, "next_sibling"),
                                   _dev(status_in, "status_in"), _dev(status_out, "status_out"), _stream(stream))
    _check("tree_mask_positions", rc)


def tree_attention_workspace_bytes(dtype, B, T_max, Hq, Hkv, d, S_cap) -> int:
    return int(lib().tree_attention_workspace_bytes(dtype, B, T_max, Hq, Hkv, d, S_cap))


def tree_attention(dtype, B, T_max, Hq, Hkv, d, Q, Kc, Vc, S_cap, prefix_len, tree_size, tree_mask, status, scale,
                   O, workspace, stream=None):
    wp, wn = _ws(workspace)
    rc = lib().tree_attention(dtype, B, T_max, Hq, Hkv, d, _dev(Q, "Q"), _dev(Kc, "Kc"), _dev(Vc, "Vc"), S_cap,
                              _dev(prefix_len, "prefix_len"), _dev(tree_size, "tree_size"),
                              _dev(tree_mask, "tree_mask"), _dev(status, "status"), float(scale), _dev(O, "O"),
                              wp, wn, _stream(stream))
    _check("tree_attention", rc)


def tree_attention_noalloc_max_bytes() -> int:
    return int(lib().tree_attention_noalloc_max_bytes())


def tree_attention_noalloc(dtype, B, T_max, Hq, Hkv, d, Q, Kc, Vc, S_cap, prefix_len, tree_size, tree_mask, status,
                           scale, O, stream=None):
    rc = lib().tree_attention_noalloc(dtype, B, T_max, Hq, Hkv, d, _dev(Q, "Q"), _dev(Kc, "Kc"), _dev(Vc, "Vc"),
                                      S_cap, _dev(prefix_len, "prefix_len"), _dev(tree_size, "tree_size"),
                                      _dev(tree_mask, "tree_mask"), _dev(status, "status"), float(scale),
                                      _dev(O, "O"), _stream(stream))
    _check("tree_attention_noalloc", rc)


def tree_accept(B, T_max, dcap, draft_tokens, parents, tree_size, target_predict, status, accept_len, accept_path,
                bonus_token, stream=None):
    rc = lib().tree_accept(B, T_max, dcap, _dev(draft_tokens, "draft_tokens"), _dev(parents, "parents"),
                           _dev(tree_size, "tree_size"), _dev(target_predict, "target_predict"),
                           _dev(status, "status"), _dev(accept_len, "accept_len"), _dev(accept_path, "accept_path"),
                           _dev(bonus_token, "bonus_token"), _stream(stream))
    _check("tree_accept", rc)


def kv_compact(B, n_layers, Hkv, d, elem_bytes, Kc, Vc, S_cap, layer_stride_elems, prefix_len, accept_path,
               accept_len, dcap, new_prefix_len, stream=None):
    rc = lib().kv_compact(B, n_layers, Hkv, d, elem_bytes, _dev(Kc, "Kc"), _dev(Vc, "Vc"), S_cap, layer_stride_elems,
                          _dev(prefix_len, "prefix_len"), _dev(accept_path, "accept_path"),
                          _dev(accept_len, "accept_len"), dcap, _dev(new_prefix_len, "new_prefix_len"),
                          _stream(stream))
    _check("kv_compact", rc)


def tree_accept_compact(B, T_max, dcap, draft_tokens, parents, tree_size, target_predict, status, accept_len,
                        accept_path, bonus_token, n_layers, Hkv, d, elem_bytes, Kc, Vc, S_cap, layer_stride_elems,
                        prefix_len, new_prefix_len, stream=None):
    rc = lib().tree_accept_compact(B, T_max, dcap, _dev(draft_tokens, "draft_tokens"), _dev(parents, "parents"),
                                   _dev(tree_size, "tree_size"), _dev(target_predict, "target_predict"),
                                   _dev(status, "status"), _dev(accept_len, "accept_len"),
                                   _dev(accept_path, "accept_path"), _dev(bonus_token, "bonus_token"), n_layers, Hkv,
                                   d, elem_bytes, _dev(Kc, "Kc"), _dev(Vc, "Vc"), S_cap, layer_stride_elems,
                                   _dev(prefix_len, "prefix_len"), _dev(new_prefix_len, "new_prefix_len"),
                                   _stream(stream))
    _check("tree_accept_compact", rc)


def tree_attention_paged(dtype, B, T_max, Hq, Hkv, d, Q, K_pool, V_pool, num_blocks, tokens_per_block, block_table,
                         max_blocks_per_seq, prefix_len, tree_size, tree_mask, status, scale, O, workspace,
                         stream=None):
    wp, wn = _ws(workspace)
    rc = lib().tree_attention_paged(dtype, B, T_max, Hq, Hkv, d, _dev(Q, "Q"), _dev(K_pool, "K_pool"),
                                    _dev(V_pool, "V_pool"), num_blocks, tokens_per_block,
                                    _dev(block_table, "block_table"), max_blocks_per_seq,
                                    _dev(prefix_len, "prefix_len"), _dev(tree_size, "tree_size"),
                                    _dev(tree_mask, "tree_mask"), _dev(status, "status"), float(scale), _dev(O, "O"),
                                    wp, wn, _stream(stream))
    _check("tree_attention_paged", rc)


def kv_compact_paged(B, n_layers, Hkv, d, elem_bytes, K_pool, V_pool, num_blocks, tokens_per_block, block_table,
                     max_blocks_per_seq, layer_stride_elems, prefix_len, accept_path, accept_len, dcap,
                     new_prefix_len, stream=None):
    rc = lib().kv_compact_paged(B, n_layers, Hkv, d, elem_bytes, _dev(K_pool, "K_pool"), _dev(V_pool, "V_pool"),
                                num_blocks, tokens_per_block, _dev(block_table, "block_table"), max_blocks_per_seq,
                                layer_stride_elems, _dev(prefix_len, "prefix_len"), _dev(accept_path, "accept_path"),
                                _dev(accept_len, "accept_len"), dcap, _dev(new_prefix_len, "new_prefix_len"),
                                _stream(stream))
    _check("kv_compact_paged", rc)


def tree_accept_compact_paged(B, T_max, dcap, draft_tokens, parents, tree_size, target_predict, status, accept_len,
                              accept_path, bonus_token, n_layers, Hkv, d, elem_bytes, K_pool, V_pool, num_blocks,
                              tokens_per_block, block_table, max_blocks_per_seq, layer_stride_elems, prefix_len,
                              new_prefix_len, stream=None):
    rc = lib().tree_accept_compact_paged(B, T_max, dcap, _dev(draft_tokens, "draft_tokens"),
                                         _dev(parents, "parents"), _dev(tree_size, "tree_size"),
                                         _dev(target_predict, "target_predict"), _dev(status, "status"),
                                         _dev(accept_len, "accept_len"), _dev(accept_path, "accept_path"),
                                         _dev(bonus_token, "bonus_token"), n_layers, Hkv, d, elem_bytes,
                                         _dev(K_pool, "K_pool"), _dev(V_pool, "V_pool"), num_blocks,
                                         tokens_per_block, _dev(block_table, "block_table"), max_blocks_per_seq,
                                         layer_stride_elems, _dev(prefix_len, "prefix_len"),
                                         _dev(new_prefix_len, "new_prefix_len"), _stream(stream))
    _check("tree_accept_compact_paged", rc)


def tree_build_layer_workspace_bytes(B, V, K, D) -> int:
    return int(lib().tree_build_layer_workspace_bytes(B, V, K, D))


def tree_build_layer(layer, B, V, K, D, rows, rows_are_logits, state, frontier_tokens, frontier_parents=None,
                     stream=None):
    sp, sn = _ws(state)
    rc = lib().tree_build_layer(layer, B, V, K, D, _dev(rows, "rows"), int(bool(rows_are_logits)), sp, sn,
                                _dev(frontier_tokens, "frontier_tokens"), _dev(frontier_parents, "frontier_parents"),
                                _stream(stream))
    _check("tree_build_layer", rc)


def tree_build_finish(B, V, K, D, total_tokens, root_token, T_max, state, draft_tokens, parents, tree_size,
                      node_score, status, dcap=0, prefix_len=None, tree_mask=None, tree_position_ids=None,
                      positions=None, retrieve_indices=None, leaf_count=None, first_child=None, next_sibling=None,
                      stream=None):
    sp, sn = _ws(state)
    rc = lib().tree_build_finish(B, V, K, D, total_tokens, _dev(root_token, "root_token"), T_max, sp, sn,
                                 _dev(draft_tokens, "draft_tokens"), _dev(parents, "parents"),
                                 _dev(tree_size, "tree_size"), _dev(node_score, "node_score"), _dev(status, "status"),
                                 dcap, _dev(prefix_len, "prefix_len"), _dev(tree_mask, "tree_mask"),
                                 _dev(tree_position_ids, "tree_position_ids"), _dev(positions, "positions"),
                                 _dev(retrieve_indices, "retrieve_indices"), _dev(leaf_count, "leaf_count"),
                                 _dev(first_child, "first_child"), _dev(next_sibling, "next_sibling"),
                                 _stream(stream))
    _check("tree_build_finish", rc)


def tree_accept_sample_workspace_bytes(B, T_max) -> int:
    return int(lib().tree_accept_sample_workspace_bytes(B, T_max))


def tree_accept_sample(B, T_max, dcap, V, draft_tokens, parents, tree_size, target_probs, uniforms, status,
                       accept_len, accept_path, bonus_token, workspace=None, stream=None):
    wp, wn = _ws(workspace)
    rc = lib().tree_accept_sample(B, T_max, dcap, V, _dev(draft_tokens, "draft_tokens"), _dev(parents, "parents"),
                                  _dev(tree_size, "tree_size"), _dev(target_probs, "target_probs"),
                                  _dev(uniforms, "uniforms"), _dev(status, "status"), _dev(accept_len, "accept_len"),
                                  _dev(accept_path, "accept_path"), _dev(bonus_token, "bonus_token"), wp, wn,
                                  _stream(stream))
    _check("tree_accept_sample", rc)


def tree_sampling_probs(B, T_max, V, logits, tree_size, status, temperature, top_k, top_p, min_p, probs,
                        stream=None):
    rc = lib().tree_sampling_probs(B, T_max, V, _dev(logits, "logits"), _dev(tree_size, "tree_size"),
                                   _dev(status, "status"), _dev(temperature, "temperature"), _dev(top_k, "top_k"),
                                   _dev(top_p, "top_p"), _dev(min_p, "min_p"), _dev(probs, "probs"),
                                   _stream(stream))
    _check("tree_sampling_probs", rc)


def tree_accept_sample_draft_workspace_bytes(B, V) -> int:
    return int(lib().tree_accept_sample_draft_workspace_bytes(B, V))


def tree_accept_sample_draft(B, T_max, dcap, V, draft_tokens, parents, tree_size, target_probs, draft_probs,
                             uniforms, status, without_replacement, accept_len, accept_path, bonus_token, workspace,
                             stream=None):
    wp, wn = _ws(workspace)
    rc = lib().tree_accept_sample_draft(B, T_max, dcap, V, _dev(draft_tokens, "draft_tokens"),
                                        _dev(parents, "parents"), _dev(tree_size, "tree_size"),
                                        _dev(target_probs, "target_probs"), _dev(draft_probs, "draft_probs"),
                                        _dev(uniforms, "uniforms"), _dev(status, "status"),
                                        1 if without_replacement else 0, _dev(accept_len, "accept_len"),
                                        _dev(accept_path, "accept_path"), _dev(bonus_token, "bonus_token"), wp, wn,
                                        _stream(stream))
    _check("tree_accept_sample_draft", rc)


def tree_attention_rope(dtype, B, T_max, Hq, Hkv, d, Q, Kc, Vc, S_cap, prefix_len, tree_size, tree_mask, status,
                        rope_theta, scale, O, workspace, stream=None):
    wp, wn = _ws(workspace)
    rc = lib().tree_attention_rope(dtype, B, T_max, Hq, Hkv, d, _dev(Q, "Q"), _dev(Kc, "Kc"), _dev(Vc, "Vc"), S_cap,
                                   _dev(prefix_len, "prefix_len"), _dev(tree_size, "tree_size"),
                                   _dev(tree_mask, "tree_mask"), _dev(status, "status"), float(rope_theta),
                                   float(scale), _dev(O, "O"), wp, wn, _stream(stream))
    _check("tree_attention_rope", rc)
