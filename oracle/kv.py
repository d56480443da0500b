"""Oracle: compaction of the accepted path's K/V rows.

Test infrastructure only (see oracle/__init__.py).

[HB] (after the tree_spec.py listing) and [TRT] ("after acceptance: KV from tree
layout back to linear"): the K/V of the accepted nodes were already computed at
the right positions during verification, so they are not recomputed; they are
moved so the sequence is contiguous again and the rejected rows are dropped.
Tree node j of request b sits at cache row P_b + j; the root (node 0) is already
at row P_b.  For k = 1..L (L = accept_len[b]) row P_b + k receives the row
P_b + path[k], in every layer and kv head, for K and V.  A source row can be a
row that an earlier k overwrites (path [0, 2, 3] reads row P+2, which k = 2
writes), so all sources are read before anything is written.  Rows outside
P_b+1..P_b+L are untouched.  new_prefix_len = P_b + L + 1.
"""
from __future__ import annotations

import numpy as np


def kv_compact(Kc: np.ndarray, Vc: np.ndarray, prefix_len, accept_path, accept_len):
    """Kc, Vc: [n_layers][B][Hkv][S_cap][d] (or [B][Hkv][S_cap][d]); returns new copies
    and new_prefix_len."""
    K2, V2 = np.array(Kc, copy=True), np.array(Vc, copy=True)
    squeeze = K2.ndim == 4
    if squeeze:
        K2, V2 = K2[None], V2[None]
    B = K2.shape[1]
    new_len = np.zeros(B, np.int32)
    for b in range(B):
        P, L = int(prefix_len[b]), int(accept_len[b])
        src = [P + int(accept_path[b][k]) for k in range(1, L + 1)]
        for T in (K2, V2):
            snapshot = [T[:, b, :, s].copy() for s in src]          # read every source first
            for k, rows in enumerate(snapshot, start=1):
                T[:, b, :, P + k] = rows
        new_len[b] = P + L + 1
    if squeeze:
        K2, V2 = K2[0], V2[0]
    return K2, V2, new_len


def kv_compact_paged(K_pool, V_pool, block_table, tokens_per_block, prefix_len, accept_path, accept_len):
    """The same compaction on a paged cache ([TRT]: the relocation walks the block
    table and copies inside blocks): logical row s of request b is
    pool[block_table[b][s // tokens_per_block], :, s % tokens_per_block].
    K_pool, V_pool: [n_layers][n_blocks][Hkv][bs][d] (or without the layer axis);
    returns new copies and new_prefix_len."""
    K2, V2 = np.array(K_pool, copy=True), np.array(V_pool, copy=True)
    squeeze = K2.ndim == 4
    if squeeze:
        K2, V2 = K2[None], V2[None]
    bs = int(tokens_per_block)
    B = len(prefix_len)
    new_len = np.zeros(B, np.int32)

    def slot(b, s):
        return int(block_table[b][s // bs]), s % bs

    for b in range(B):
        P, L = int(prefix_len[b]), int(accept_len[b])
        src = [slot(b, P + int(accept_path[b][k])) for k in range(1, L + 1)]
        dst = [slot(b, P + k) for k in range(1, L + 1)]
        for T in (K2, V2):
            snapshot = [T[:, blk, :, off].copy() for blk, off in src]     # read every source first
            for (blk, off), rows in zip(dst, snapshot):
                T[:, blk, :, off] = rows
        new_len[b] = P + L + 1
    if squeeze:
        K2, V2 = K2[0], V2[0]
    return K2, V2, new_len
