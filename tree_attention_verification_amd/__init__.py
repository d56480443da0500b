"""MI355X-native tree-verification step for EAGLE-2/3 dynamic-tree speculative decoding.

The work is done by libtreeverify.so (hand-written HIP for gfx950, C ABI in
include/treeverify.h); `_lib` is the ctypes binding with the same call names and
`step.TreeVerifyStep` holds one batch's device buffers and runs the five calls.
"""
from . import _lib
from ._lib import (tree_build, tree_build_workspace_bytes, tree_build_meta, tree_mask_positions, tree_attention,
                   tree_attention_workspace_bytes, tree_accept, kv_compact, tree_accept_compact,
                   tree_attention_paged, kv_compact_paged, tree_accept_compact_paged,
                   tree_build_layer_workspace_bytes, tree_build_layer, tree_build_finish,
                   tree_accept_sample_workspace_bytes, tree_accept_sample, tree_attention_rope, tree_sampling_probs, tree_accept_sample_draft_workspace_bytes,
                   tree_accept_sample_draft, TVError)

__all__ = ["tree_build", "tree_build_workspace_bytes", "tree_build_meta", "tree_mask_positions", "tree_attention",
           "tree_attention_workspace_bytes", "tree_accept", "kv_compact", "tree_accept_compact",
           "tree_attention_paged", "kv_compact_paged", "tree_accept_compact_paged",
           "tree_build_layer_workspace_bytes", "tree_build_layer", "tree_build_finish",
           "tree_accept_sample_workspace_bytes", "tree_accept_sample", "tree_attention_rope", "tree_sampling_probs", "tree_accept_sample_draft_workspace_bytes",
           "tree_accept_sample_draft", "TVError"]
