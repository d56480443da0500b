"""Pins for the oracle's greedy acceptance and KV compaction (CPU only).

Expected values come from:
  * plain greedy decoding with a toy deterministic target (the handbook's claim that
    tree speculative decoding reproduces greedy output token for token): the accepted
    tokens plus the bonus token are the next greedy tokens after the root;
  * brute-force enumeration of every root path (the accepted length is the longest
    path that is a greedy prefix);
  * the second formulation of the EAGLE v2 walkthrough (cumprod along retrieve rows,
    best row with lowest index on ties);
  * special cases: nothing matches -> 0; a chain is all-or-cut;
  * compaction: rows labelled by their own index land where the definition says,
    every other byte is untouched, and attention of the last accepted node over the
    compacted contiguous prefix equals its tree-attention output before compaction.
"""
import hashlib

import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle import kv as okv
from oracle import tree as ot
from workloads import gen


def toy_target(seq, V):
    """Deterministic stand-in for a target model's greedy next token."""
    h = hashlib.blake2b(bytes(str(tuple(seq)), "ascii"), digest_size=8).digest()
    return int.from_bytes(h, "little") % V


def path_tokens(tokens, parents, i):
    out = []
    while i != -1:
        out.append(tokens[i])
        i = parents[i]
    return out[::-1]


def random_tree(rng, T, V, max_depth=7):
    """Random tree with distinct sibling tokens (parents precede children)."""
    parents, depth, nkids = [-1], [0], [0]
    for i in range(1, T):
        elig = [j for j in range(i) if depth[j] < max_depth and nkids[j] < V]
        p = elig[int(rng.integers(0, len(elig)))]
        parents.append(p)
        depth.append(depth[p] + 1)
        nkids[p] += 1
        nkids.append(0)
    tokens = [int(rng.integers(0, V))] + [0] * (T - 1)
    for i in range(T):
        kids = [c for c in range(1, T) if parents[c] == i]
        if kids:
            for c, t in zip(kids, rng.choice(V, size=len(kids), replace=False)):
                tokens[c] = int(t)
    return tokens, parents


def test_accept_equals_plain_greedy_decode():
    rng = np.random.default_rng(11)
    V, dcap = 4, 7
    for trial in range(500):
        T = int(rng.integers(1, 40))
        tokens, parents = random_tree(rng, T, V)
        prompt = [int(x) for x in rng.integers(0, V, size=5)]
        pred = [toy_target(prompt + path_tokens(tokens, parents, i), V) for i in range(T)]
        alen, apath, bonus = ot.accept_walk(tokens, parents, T, pred, 0, dcap)
        # plain greedy from prompt + root
        seq = prompt + [tokens[0]]
        greedy = []
        for _ in range(alen + 1):
            nxt = toy_target(seq, V)
            greedy.append(nxt)
            seq.append(nxt)
        got = [tokens[n] for n in apath[1:alen + 1]] + [bonus]
        assert got == greedy, trial
        # brute force over every root path: longest greedy-consistent prefix
        best = 0
        for leaf in range(T):
            chain = path_tokens(tokens, parents, leaf)
            s, k = prompt + [chain[0]], 0
            for t in chain[1:]:
                if toy_target(s, V) != t:
                    break
                s.append(t)
                k += 1
            best = max(best, k)
        assert alen == best
        # second formulation: cumprod along retrieve rows
        meta = ot.mask_positions(parents + [-1] * (64 - T), T, 0, 64, dcap)
        plen, ppath = ot.accept_posterior(tokens + [-1] * (64 - T), meta["retrieve_indices"],
                                          meta["leaf_count"], pred + [-1] * (64 - T))
        assert plen == alen and ppath == apath[:alen + 1]


def test_all_mismatch_and_chain_all_or_cut():
    tokens = [5, 1, 2, 3, 4]
    parents = [-1, 0, 1, 2, 3]
    assert ot.accept_walk(tokens, parents, 5, [9] * 5, 0, 7) == (0, [0] + [-1] * 7, 9)
    # chain: accepted up to the first mismatch, then cut
    pred = [1, 2, 7, 4, 8]
    alen, apath, bonus = ot.accept_walk(tokens, parents, 5, pred, 0, 7)
    assert (alen, apath[:3], bonus) == (2, [0, 1, 2], 7)
    pred = [1, 2, 3, 4, 8]
    assert ot.accept_walk(tokens, parents, 5, pred, 0, 7)[0] == 4
    # status != 0 -> root only
    assert ot.accept_walk(tokens, parents, 5, pred, 1, 7) == (0, [0] + [-1] * 7, 1)
    # the walk never goes deeper than dcap
    assert ot.accept_walk(tokens, parents, 5, pred, 0, 2)[0] == 2


def test_compaction_moves_labelled_rows():
    B, H, S, d, P = 3, 2, 40, 8, [5, 12, 0]
    K = np.zeros((2, B, H, S, d), np.float32)       # two layers
    for r in range(S):
        K[..., r, :] = r
    V = -K
    path = np.array([[0, 2, 3, 7, -1], [0, 1, -1, -1, -1], [0, 4, 9, 10, 11]], np.int32)
    alen = np.array([3, 0, 4], np.int32)
    K2, V2, new = okv.kv_compact(K, V, P, path, alen)
    assert list(new) == [5 + 4, 12 + 1, 0 + 5]
    for b in range(B):
        exp = np.arange(S, dtype=np.float32)
        for k in range(1, alen[b] + 1):
            exp[P[b] + k] = P[b] + path[b][k]
        assert np.array_equal(K2[:, b, :, :, 0], np.broadcast_to(exp[:, None].T, (2, H, S)))
        assert np.array_equal(V2[:, b], -K2[:, b])


def test_compacted_prefix_reproduces_the_accepted_nodes_attention():
    w = gen.make_custom(cfg_id=41, P=60, Hq=4, Hkv=2, d=64, dtype="fp32", mode="given",
                        given_sizes=[30], V=6)
    T = int(w.given_size[0])
    meta = ot.tree_mask_positions(w.given_parents, w.given_size, w.prefix_len, 64, 7)
    rng = np.random.default_rng(2)
    # force a long accepted path: predict the first child everywhere
    pred = np.full((1, 64), -7, np.int32)
    for i in range(T):
        if meta["first_child"][0, i] != -1:
            pred[0, i] = w.given_tokens[0, meta["first_child"][0, i]]
    acc = ot.tree_accept(w.given_tokens, w.given_parents, w.given_size, pred, meta["status"], 7)
    L = int(acc["accept_len"][0])
    assert L >= 2
    O = oa.tree_attention(w.Q, w.Kc, w.Vc, w.prefix_len, w.given_size, meta["tree_mask"])
    K2, V2, new = okv.kv_compact(w.Kc, w.Vc, w.prefix_len, acc["accept_path"], acc["accept_len"])
    last = int(acc["accept_path"][0, L])
    n = int(new[0])
    for h in range(4):
        g = h // 2
        q = oa.to_f64(w.Q[0, last, h])
        s = oa.to_f64(K2[0, g, :n]) @ q / np.sqrt(64)
        p = np.exp(s - s.max())
        ref = p @ oa.to_f64(V2[0, g, :n]) / p.sum()
        assert np.abs(O[0, last, h] - ref).max() < 1e-12
