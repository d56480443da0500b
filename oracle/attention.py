"""Oracle: tree-masked grouped-query attention, dense softmax in float64.

Test infrastructure only (see oracle/__init__.py).

What is computed ([HB] tree_spec.py forward_with_mask and the correctness check;
[E2] section 4 tree_decoding; [TRT] packed ancestor mask): for request b, query head
h and tree node i < T_b the visible keys are every committed prefix row
0..P_b-1 of kv head g = h // (Hq/Hkv) (the KV heads are repeated across the
query-head group) plus the tree rows P_b + j for which node j is node i itself
or one of its ancestors (bit j of the packed mask row i).  The output is
softmax(q . k * scale) . v over those keys, scale = 1/sqrt(d) by default (the
scaled-dot-product default).  Q and K are taken after any rotary embedding.

Inputs are fed exactly as the library receives them: bf16 bit patterns (uint16)
or float32.  bf16 -> float64 is exact; all arithmetic is float64; a matmul from
numpy is the only library primitive.  Rows i >= T_b of the output are left as
given; a request with non-zero status is the root-only tree (T_b = 1).
"""
from __future__ import annotations

import math

import numpy as np


def to_f64(x: np.ndarray) -> np.ndarray:
    """Decode the stored element type exactly: uint16 arrays are bfloat16 bit patterns
    (the upper 16 bits of a float32), anything else is cast."""
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def visible_tree_nodes(mask_row: np.ndarray, T: int):
    """Node ids j < T whose bit is set in a packed mask row (bit j&31 of word j>>5)."""
    return [j for j in range(T) if (int(mask_row[j >> 5]) >> (j & 31)) & 1]


def full_mask(tree_mask_b: np.ndarray, T: int, P: int) -> np.ndarray:
    """[T][P+T] boolean visibility for one request, built as [HB] forward_with_mask
    builds it: every node sees all P prefix columns, followed by the T x T tree mask
    (unpacked from the packed rows)."""
    m = np.zeros((T, P + T), dtype=bool)
    m[:, :P] = True
    for i in range(T):
        for j in visible_tree_nodes(tree_mask_b[i], T):
            m[i, P + j] = True
    return m


def tree_attention(Q, Kc, Vc, prefix_len, tree_size, tree_mask, status=None, scale=None, out=None,
                   requests=None):
    """Returns float64 O shaped like Q.  ``requests`` limits the work to a subset of
    request ids (the others are left as in ``out``, default zero).

    Per request and kv head the scores of all T*rep query rows against all P+T keys
    are one float64 matmul; masked entries get -inf; each row is soft-maxed
    (max-subtracted) and multiplied by V -- the dense masked attention of the
    definition."""
    B, T_max, Hq, d = Q.shape
    Hkv = Kc.shape[1]
    rep = Hq // Hkv
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(d)
    O = np.zeros(Q.shape, np.float64) if out is None else np.array(out, dtype=np.float64, copy=True)
    for b in (range(B) if requests is None else requests):
        T = int(tree_size[b])
        if status is not None and int(status[b]) != 0:
            T = 1
        P = int(prefix_len[b])
        vis = full_mask(tree_mask[b], T, P)                            # [T][P+T]
        for g in range(Hkv):
            keys = to_f64(Kc[b, g, :P + T])                            # [P+T][d]
            vals = to_f64(Vc[b, g, :P + T])
            q = to_f64(Q[b, :T, g * rep:(g + 1) * rep])                # [T][rep][d]
            s = (q.reshape(T * rep, d) @ keys.T).reshape(T, rep, P + T) * scale   # [T][rep][P+T]
            s = np.where(vis[:, None, :], s, -np.inf)
            p = np.exp(s - s.max(axis=2, keepdims=True))
            O[b, :T, g * rep:(g + 1) * rep] = (p @ vals) / p.sum(axis=2, keepdims=True)
    return O


def attention_rows(Q, Kc, Vc, prefix_len, tree_size, tree_mask, samples, scale=None, status=None):
    """Oracle output for a list of sampled (b, i, h) rows only (for full-size checks)."""
    B, T_max, Hq, d = Q.shape
    rep = Hq // Kc.shape[1]
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(d)
    res = []
    for b, i, h in samples:
        T = int(tree_size[b])
        if status is not None and int(status[b]) != 0:
            T = 1
        P = int(prefix_len[b])
        g = h // rep
        vis = list(range(P)) + [P + j for j in visible_tree_nodes(tree_mask[b, i], T)]
        k_i = to_f64(Kc[b, g][vis])
        v_i = to_f64(Vc[b, g][vis])
        s = (k_i @ to_f64(Q[b, i, h])) * scale
        p = np.exp(s - s.max())
        res.append((p @ v_i) / p.sum())
    return np.array(res)


def paged_to_linear(pool, block_table, tokens_per_block, n_rows):
    """The linear cache [B][Hkv][n_rows][d] a paged pool describes ([TRT] "after
    acceptance: KV from tree layout back to linear": a token's physical slot is its
    request's block-table entry plus the offset inside the block).  Row s of request b
    is pool[block_table[b][s // tokens_per_block], :, s % tokens_per_block]; pool is
    [n_blocks][Hkv][tokens_per_block][d]."""
    table = np.asarray(block_table)
    s = np.arange(n_rows)
    blk = table[:, s // tokens_per_block]                      # [B][n_rows]
    off = np.broadcast_to(s % tokens_per_block, blk.shape)     # [B][n_rows]
    rows = pool[blk, :, off]                                   # [B][n_rows][Hkv][d]
    return np.ascontiguousarray(rows.transpose(0, 2, 1, 3))


def tree_attention_paged(Q, K_pool, V_pool, block_table, tokens_per_block, prefix_len, tree_size, tree_mask,
                         status=None, scale=None, requests=None):
    """tree_attention over a paged cache: the rows each request reads (P_b + T_b of them)
    are gathered through its block table, then the dense definition above applies."""
    n = max(int(prefix_len[b]) + max(int(tree_size[b]), 1) for b in range(Q.shape[0]))
    n = min(n, np.asarray(block_table).shape[1] * tokens_per_block)
    Kc = paged_to_linear(K_pool, block_table, tokens_per_block, n)
    Vc = paged_to_linear(V_pool, block_table, tokens_per_block, n)
    return tree_attention(Q, Kc, Vc, prefix_len, tree_size, tree_mask, status=status, scale=scale,
                          requests=requests)


def attention_rows_paged(Q, K_pool, V_pool, block_table, tokens_per_block, prefix_len, tree_size, tree_mask,
                         samples, scale=None, status=None):
    """attention_rows over a paged cache (rows gathered through the block table)."""
    B, T_max = Q.shape[:2]
    n = min(int(np.max(np.asarray(prefix_len))) + T_max, np.asarray(block_table).shape[1] * tokens_per_block)
    Kc = paged_to_linear(K_pool, block_table, tokens_per_block, n)
    Vc = paged_to_linear(V_pool, block_table, tokens_per_block, n)
    return attention_rows(Q, Kc, Vc, prefix_len, tree_size, tree_mask, samples, scale=scale, status=status)


def rope_rotate(x, positions, theta):
    """Rotary position embedding of the last axis of x at the given positions ([HB]
    forward_with_mask applies it to the tree's queries and keys at position
    prefix + depth).  Pairs (i, i + d/2) rotate by angle pos * theta**(-2i/d) (the
    rotate-half layout): out_i = x_i cos - x_(i+d/2) sin, out_(i+d/2) = x_(i+d/2) cos
    + x_i sin.  x: [..., d] (float64 after to_f64), positions broadcast against x's
    leading axes.  All in float64."""
    x = to_f64(x) if np.asarray(x).dtype == np.uint16 else np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    inv = theta ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    ang = np.asarray(positions, dtype=np.float64)[..., None] * inv
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def tree_attention_rope(Q, Kc, Vc, prefix_len, tree_size, tree_mask, positions, theta, status=None, scale=None):
    """tree_attention with the queries given before their rotary embedding: each node's
    query heads are rotated at its position (positions [B][T_max] = prefix + depth, as
    tree_mask_positions writes them), then the dense definition applies.  The cache
    holds keys after their rotary embedding."""
    Qr = rope_rotate(Q, np.asarray(positions)[:, :, None], theta)    # [B][T_max][Hq][d]
    return tree_attention(Qr, Kc, Vc, prefix_len, tree_size, tree_mask, status=status, scale=scale)
