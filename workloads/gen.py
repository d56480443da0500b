"""Seeded synthetic inputs for the tree-verification step.

This module only draws random numbers and lays them out in the buffers the
library and the oracle both read.  It computes none of the method's outputs:
no top-k, no tree selection, no mask, no attention, no acceptance.  Both the
HIP path and the CPU oracle are fed the *same bytes* from here.

Every stream is a PCG64 generator seeded with ``[cfg_id, stream, b]``:
  0 draft logits, 1 Q, 2 K, 3 V, 4 target draws, 5 shapes/topology, 6 root
  tokens, 7 paged-cache block placement, 8 target distributions for sampling.

Workload shapes follow the five configurations the tree-verification step is
measured on (tree sizes as in the EAGLE-2 walkthrough's ``topK_generate``
section: top_k, depth, total_tokens = 60; GQA attention shapes of Llama-3-8B /
70B layers).  Where the configuration text leaves a value open the choice is
stated next to it.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np

(STREAM_LOGITS, STREAM_Q, STREAM_K, STREAM_V, STREAM_TARGET, STREAM_SHAPE, STREAM_ROOT, STREAM_PAGES, STREAM_PROBS,
 STREAM_TLOGITS, STREAM_DRAFTQ) = range(11)

T_MAX_DEFAULT = 64
DCAP_DEFAULT = 7


def rng(cfg_id: int, stream: int, b: int = 0) -> np.random.Generator:
    return np.random.default_rng([int(cfg_id), int(stream), int(b)])


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bfloat16 (round to nearest, ties to even); returns uint16 bit patterns.
    Inputs here are finite normal draws, so NaN handling is not needed."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


@dataclasses.dataclass
class Workload:
    """One batch of inputs for a full pass of the verification step."""
    name: str
    cfg_id: int
    B: int
    mode: str                      # 'dynamic' | 'static' | 'given'
    V: int
    K: int                         # top_k (dynamic) or max(branching) (static)
    D: int                         # expansion rounds after the base layer (dynamic)
    total_tokens: int              # draft nodes kept, root excluded (dynamic)
    branching: List[int]           # static mode level widths
    T_max: int
    dcap: int
    # draft side
    logprobs: Optional[np.ndarray]  # float32 [B][R][V]
    root_token: np.ndarray          # int32 [B]
    # given-topology mode only (the drafter's tree is an input)
    given_parents: Optional[np.ndarray] = None   # int32 [B][T_max]
    given_tokens: Optional[np.ndarray] = None    # int32 [B][T_max]
    given_size: Optional[np.ndarray] = None      # int32 [B]
    # attention side
    prefix_len: np.ndarray = None   # int32 [B]
    Hq: int = 0
    Hkv: int = 0
    d: int = 0
    dtype: str = "bf16"             # 'bf16' (uint16 bit patterns) or 'fp32'
    S_cap: int = 0
    Q: np.ndarray = None            # [B][T_max][Hq][d]
    Kc: np.ndarray = None           # [B][Hkv][S_cap][d]
    Vc: np.ndarray = None           # [B][Hkv][S_cap][d]
    # synthetic target model draws
    accept_prob: float = 0.6
    tgt_u: np.ndarray = None        # float64 [B][T_max]
    tgt_choice: np.ndarray = None   # int64 [B][T_max]
    tgt_rand: np.ndarray = None     # int32 [B][T_max]

    @property
    def rows_per_req(self) -> int:
        return 0 if self.logprobs is None else self.logprobs.shape[1]

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4


def _draft_logprobs(cfg_id: int, B: int, R: int, V: int, std: float, peaked: bool) -> np.ndarray:
    """Draft distributions: logits ~ N(0, std^2) per row, optionally with +12 added to one
    random token per row; log-probs = fp32(logits - logsumexp(logits)) computed in fp64."""
    out = np.empty((B, R, V), dtype=np.float32)
    for b in range(B):
        g = rng(cfg_id, STREAM_LOGITS, b)
        z = g.standard_normal((R, V)) * std
        if peaked:
            hot = g.integers(0, V, size=R)
            z[np.arange(R), hot] += 12.0
        zmax = z.max(axis=1, keepdims=True)
        lse = zmax + np.log(np.exp(z - zmax).sum(axis=1, keepdims=True))
        out[b] = (z - lse).astype(np.float32)
    return out


def draft_logits(cfg_id: int, B: int, R: int, V: int, std: float = 2.0, peaked: bool = False) -> np.ndarray:
    """The raw draft logits behind _draft_logprobs (same draws), rounded to float32:
    the input of the layer-by-layer build's fused log-softmax."""
    out = np.empty((B, R, V), dtype=np.float32)
    for b in range(B):
        g = rng(cfg_id, STREAM_LOGITS, b)
        z = g.standard_normal((R, V)) * std
        if peaked:
            hot = g.integers(0, V, size=R)
            z[np.arange(R), hot] += 12.0
        out[b] = z.astype(np.float32)
    return out


def _attn_tensors(cfg_id: int, B: int, T_max: int, Hq: int, Hkv: int, d: int, S_cap: int,
                  scale: float, dtype: str):
    Q = np.empty((B, T_max, Hq, d), dtype=np.uint16 if dtype == "bf16" else np.float32)
    Kc = np.empty((B, Hkv, S_cap, d), dtype=Q.dtype)
    Vc = np.empty((B, Hkv, S_cap, d), dtype=Q.dtype)
    for b in range(B):
        for arr, stream in ((Q, STREAM_Q), (Kc, STREAM_K), (Vc, STREAM_V)):
            x = rng(cfg_id, stream, b).standard_normal(arr.shape[1:], dtype=np.float32)
            if scale != 1.0:
                x *= np.float32(scale)
            arr[b] = f32_to_bf16_bits(x) if dtype == "bf16" else x
    return Q, Kc, Vc


def _target_draws(cfg_id: int, B: int, T_max: int, V: int):
    u = np.empty((B, T_max), dtype=np.float64)
    ch = np.empty((B, T_max), dtype=np.int64)
    rt = np.empty((B, T_max), dtype=np.int32)
    for b in range(B):
        g = rng(cfg_id, STREAM_TARGET, b)
        u[b] = g.random(T_max)
        ch[b] = g.integers(0, 1 << 30, size=T_max)
        rt[b] = g.integers(0, V, size=T_max)
    return u, ch, rt


def _root_tokens(cfg_id: int, B: int, V: int) -> np.ndarray:
    return np.array([rng(cfg_id, STREAM_ROOT, b).integers(0, V) for b in range(B)], dtype=np.int32)


def _random_topology(cfg_id: int, b: int, T: int, V: int, max_depth: int, T_max: int):
    """Random tree of T nodes (root included) with node depth <= max_depth.

    Nodes are created one by one; node k picks its parent uniformly among the
    already created nodes whose level is below max_depth and that have fewer
    than V children (a node's level is known when it is created: parent's
    level + 1).  Nodes are then renumbered
    level by level (breadth-first: within a level, by new parent index then
    creation order), so parents precede children.  Sibling tokens are drawn
    without replacement from [0, V)."""
    g = rng(cfg_id, STREAM_SHAPE, b)
    par = [-1]
    lev = [0]
    nkid = [0]
    for k in range(1, T):
        elig = [j for j in range(k) if lev[j] < max_depth and nkid[j] < V]
        p = elig[int(g.integers(0, len(elig)))]
        par.append(p)
        lev.append(lev[p] + 1)
        nkid[p] += 1
        nkid.append(0)
    # breadth-first renumbering
    new_of = {0: 0}
    order = [0]
    for level in range(1, max_depth + 1):
        members = [k for k in range(T) if lev[k] == level]
        members.sort(key=lambda k: (new_of[par[k]], k))
        for k in members:
            new_of[k] = len(order)
            order.append(k)
    parents = np.full(T_max, -1, dtype=np.int32)
    tokens = np.full(T_max, -1, dtype=np.int32)
    for old in order:
        parents[new_of[old]] = -1 if old == 0 else new_of[par[old]]
    tokens[0] = int(g.integers(0, V))
    for nd in range(T):
        kids = [c for c in range(T) if parents[c] == nd and c != 0]
        if kids:
            toks = g.choice(V, size=len(kids), replace=False)
            for c, t in zip(kids, toks):
                tokens[c] = int(t)
    return parents, tokens


def make_workload(cfg_id: int, *, peaked: bool = False, batch: Optional[int] = None,
                  prefix: Optional[int] = None, T_max: int = T_MAX_DEFAULT,
                  dcap: int = DCAP_DEFAULT, seed_offset: int = 0,
                  with_attention: bool = True, tree_nodes: Optional[int] = None) -> Workload:
    """Build one of the five measured configurations (1..5).

    ``batch`` / ``prefix`` shrink a configuration for CPU-sized tests while
    keeping its tree and head shapes; ``seed_offset`` moves every stream;
    ``with_attention=False`` skips the Q/K/V draws (tree-only tests);
    ``tree_nodes`` (65..256) grows the trees: dynamic configurations keep
    tree_nodes - 1 draft nodes, the random-tree configuration draws sizes in
    [8, tree_nodes]; T_max becomes tree_nodes."""
    if tree_nodes is not None:
        T_max = int(tree_nodes)
    sid = cfg_id + 1000 * seed_offset
    attn = _attn_tensors if with_attention else (lambda *a: (None, None, None))
    if cfg_id == 1:
        # Tiny chain-vs-tree check: static branching [2,2,1], P=128, Hq4/Hkv2/d64 fp32, V=1000.
        B, P, V = 1, 128, 1000
        branching = [2, 2, 1]
        R = 1 + 2 + 4                      # nodes expanded by the static builder
        lp = _draft_logprobs(sid, B, R, V, 2.0, peaked)
        T = 1 + 2 + 4 + 4
        S_cap = P + T_max
        Q, Kc, Vc = attn(sid, B, T_max, 4, 2, 64, S_cap, 1.0, "fp32")
        u, ch, rt = _target_draws(sid, B, T_max, V)
        return Workload("tiny-static-[2,2,1]-P128-fp32", cfg_id, B, "static", V, max(branching), 0, T - 1,
                        branching, T_max, dcap, lp, _root_tokens(sid, B, V),
                        prefix_len=np.full(B, P, np.int32), Hq=4, Hkv=2, d=64, dtype="fp32",
                        S_cap=S_cap, Q=Q, Kc=Kc, Vc=Vc, accept_prob=0.7, tgt_u=u, tgt_choice=ch, tgt_rand=rt)
    if cfg_id in (2, 3, 4):
        if cfg_id == 2:
            B, K, D, TT, Hq = 1, 10, 6, 60, 32
            P = np.full(B, 2048, np.int32)
        elif cfg_id == 3:
            B, K, D, TT, Hq = 16, 8, 5, 48, 32
            P = np.array([rng(sid, STREAM_SHAPE, b).integers(512, 8193) for b in range(B)], np.int32)
        else:
            B, K, D, TT, Hq = 4, 10, 6, 60, 64
            P = np.full(B, 32768, np.int32)
        if tree_nodes is not None:
            TT = int(tree_nodes) - 1
        if batch is not None:
            B = batch
            P = P[:B] if len(P) >= B else np.resize(P, B)
        if prefix is not None:
            P = np.minimum(P, prefix).astype(np.int32)
        V = 32000
        R = 1 + D * K
        lp = _draft_logprobs(sid, B, R, V, 2.0, peaked)
        S_cap = int(P.max()) + T_max
        Q, Kc, Vc = attn(sid, B, T_max, Hq, 8, 128, S_cap, 0.5, "bf16")
        u, ch, rt = _target_draws(sid, B, T_max, V)
        names = {2: "eagle2-dynamic-b1-P2048-K10-D6-T60-llama3-8b",
                 3: "ragged-b16-P512..8192-K8-D5-T48",
                 4: "long-b4-P32768-K10-D6-T60-70b-gqa"}
        return Workload(names[cfg_id], cfg_id, B, "dynamic", V, K, D, TT, [], T_max, dcap, lp,
                        _root_tokens(sid, B, V), prefix_len=P, Hq=Hq, Hkv=8, d=128, dtype="bf16",
                        S_cap=S_cap, Q=Q, Kc=Kc, Vc=Vc, accept_prob=0.6, tgt_u=u, tgt_choice=ch, tgt_rand=rt)
    if cfg_id == 5:
        B = 64 if batch is None else batch
        V = 32000
        P = np.full(B, 4096 if prefix is None else prefix, np.int32)
        top = 64 if tree_nodes is None else int(tree_nodes)
        sizes = np.array([rng(sid, STREAM_SHAPE, 10_000 + b).integers(8, top + 1) for b in range(B)], np.int32)
        sizes = np.minimum(sizes, T_max).astype(np.int32)
        par = np.full((B, T_max), -1, np.int32)
        tok = np.full((B, T_max), -1, np.int32)
        for b in range(B):
            par[b], tok[b] = _random_topology(sid, b, int(sizes[b]), V, 7, T_max)
        S_cap = int(P.max()) + T_max
        Q, Kc, Vc = attn(sid, B, T_max, 32, 8, 128, S_cap, 0.5, "bf16")
        u, ch, rt = _target_draws(sid, B, T_max, V)
        return Workload("large-b64-P4096-random-trees-T8..64", cfg_id, B, "given", V, 0, 0, 0, [], T_max, dcap,
                        None, tok[:, 0].copy(), given_parents=par, given_tokens=tok, given_size=sizes,
                        prefix_len=P, Hq=32, Hkv=8, d=128, dtype="bf16", S_cap=S_cap, Q=Q, Kc=Kc, Vc=Vc,
                        accept_prob=0.5, tgt_u=u, tgt_choice=ch, tgt_rand=rt)
    raise ValueError(f"unknown configuration {cfg_id}")


def make_custom(*, cfg_id: int = 900, B: int = 1, P=128, mode: str = "dynamic", V: int = 64,
                K: int = 3, D: int = 2, total_tokens: int = 8, branching=(2, 2, 1), T_max: int = 64,
                dcap: int = 7, Hq: int = 4, Hkv: int = 2, d: int = 64, dtype: str = "bf16",
                qkv_scale: float = 0.5, accept_prob: float = 0.6, peaked: bool = False,
                logit_std: float = 2.0, given_sizes=None, given_depth: int = 7,
                S_cap: Optional[int] = None) -> Workload:
    """Arbitrary small shapes for fuzz and edge-case tests (same recipe as the configurations)."""
    sid = cfg_id
    Parr = np.array(P if np.ndim(P) else [P] * B, dtype=np.int32)
    if S_cap is None:
        S_cap = int(Parr.max()) + T_max
    lp = None
    par = tok = sizes = None
    if mode == "dynamic":
        lp = _draft_logprobs(sid, B, 1 + D * K, V, logit_std, peaked)
    elif mode == "static":
        nrow, width = 1, 1
        for w in branching[:-1]:
            width *= w
            nrow += width
        lp = _draft_logprobs(sid, B, nrow, V, logit_std, peaked)
        K = max(branching)
    else:
        sizes = np.array(given_sizes if given_sizes is not None else
                         [rng(sid, STREAM_SHAPE, 10_000 + b).integers(1, T_max + 1) for b in range(B)], np.int32)
        par = np.full((B, T_max), -1, np.int32)
        tok = np.full((B, T_max), -1, np.int32)
        for b in range(B):
            par[b], tok[b] = _random_topology(sid, b, int(sizes[b]), V, given_depth, T_max)
    Q, Kc, Vc = _attn_tensors(sid, B, T_max, Hq, Hkv, d, S_cap, qkv_scale, dtype)
    u, ch, rt = _target_draws(sid, B, T_max, V)
    root = tok[:, 0].copy() if mode == "given" else _root_tokens(sid, B, V)
    return Workload(f"custom-{mode}", cfg_id, B, mode, V, K, D, total_tokens, list(branching), T_max, dcap,
                    lp, root, given_parents=par, given_tokens=tok, given_size=sizes, prefix_len=Parr,
                    Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, S_cap=S_cap, Q=Q, Kc=Kc, Vc=Vc,
                    accept_prob=accept_prob, tgt_u=u, tgt_choice=ch, tgt_rand=rt)


def synthetic_target_predict(w: Workload, draft_tokens: np.ndarray, parents: np.ndarray,
                             tree_size: np.ndarray) -> np.ndarray:
    """Stand-in for the target model's per-node argmax (the target forward is not part of
    the step).  For node i with children (nodes c < tree_size with parents[c] == i, in
    ascending order): with probability ``accept_prob`` predict the token of child number
    ``choice % n_children``; otherwise (and at leaves) predict a uniform random token.
    The tree it reads is whatever tree the side under test was given or built; it is
    identical on both sides because the builds are compared bit for bit first."""
    B, T_max = draft_tokens.shape
    out = np.full((B, T_max), -1, dtype=np.int32)
    for b in range(B):
        T = int(tree_size[b])
        if T < 1 or T > T_max:          # a malformed tree is verified as its root alone
            T = 1
        for i in range(T):
            kids = [c for c in range(1, T) if parents[b, c] == i]
            if kids and w.tgt_u[b, i] < w.accept_prob:
                out[b, i] = draft_tokens[b, kids[int(w.tgt_choice[b, i]) % len(kids)]]
            else:
                out[b, i] = w.tgt_rand[b, i]
    return out



@dataclasses.dataclass
class PagedCache:
    """A paged copy of a workload's K/V cache (pure data placement, nothing computed).

    K_pool, V_pool [n_blocks][Hkv][tokens_per_block][d]: block_table[b][j] is the
    physical block that holds logical rows j*tokens_per_block .. (j+1)*tokens_per_block-1
    of request b (all kv heads).  Blocks no request owns, and rows of a request's last
    block past the linear cache's S_cap, hold NaN bit patterns."""
    tokens_per_block: int
    max_blocks: int
    n_blocks: int
    block_table: np.ndarray   # int32 [B][max_blocks]
    K_pool: np.ndarray
    V_pool: np.ndarray

    @property
    def capacity(self) -> int:
        return self.max_blocks * self.tokens_per_block


def nan_bits(dtype) -> object:
    """A quiet-NaN fill value of the stored element type (uint16 = bfloat16 bits)."""
    return np.uint16(0x7FC0) if np.dtype(dtype) == np.uint16 else np.float32(np.nan)


def paged_layout(w: Workload, tokens_per_block: int, spare_blocks: Optional[int] = None) -> PagedCache:
    """Place w.Kc / w.Vc block by block at seeded random physical blocks of a pool with
    ``spare_blocks`` extra blocks (default B*max_blocks/8, at least 1) that no request owns."""
    B, Hkv, S_cap, d = w.Kc.shape
    bs = int(tokens_per_block)
    max_blocks = -(-S_cap // bs)
    n_used = B * max_blocks
    spare = max(1, n_used // 8) if spare_blocks is None else int(spare_blocks)
    n_blocks = n_used + spare
    perm = rng(w.cfg_id, STREAM_PAGES, 0).permutation(n_blocks)[:n_used].astype(np.int32)
    table = perm.reshape(B, max_blocks)
    pools = []
    for lin in (w.Kc, w.Vc):
        pool = np.full((n_blocks, Hkv, bs, d), nan_bits(lin.dtype), dtype=lin.dtype)
        padded = np.full((B, Hkv, max_blocks * bs, d), nan_bits(lin.dtype), dtype=lin.dtype)
        padded[:, :, :S_cap] = lin
        # [B][Hkv][max_blocks][bs][d] -> [B][max_blocks][Hkv][bs][d], one physical block each
        blocks = padded.reshape(B, Hkv, max_blocks, bs, d).transpose(0, 2, 1, 3, 4)
        pool[table.reshape(-1)] = blocks.reshape(n_used, Hkv, bs, d)
        pools.append(pool)
    return PagedCache(bs, max_blocks, n_blocks, table, pools[0], pools[1])


def synthetic_target_probs(w: Workload, draft_tokens: np.ndarray, parents: np.ndarray, tree_size: np.ndarray,
                           concentration: float = 0.3):
    """Stand-in for the target model's (filtered) next-token distribution at every node,
    and the uniform draws of rejection sampling.  Row i of a tree node is Gamma(
    concentration) noise normalised to sum 1 - m plus mass m ~ U[0.5, 0.95] on the
    token of one of node i's children (chosen uniformly) with probability
    accept_prob; rows of padding nodes are zero.  Returns float32 probs
    [B][T_max][V] and float32 uniforms [B][T_max] in [0, 1)."""
    B, T_max = draft_tokens.shape
    V = w.V
    probs = np.zeros((B, T_max, V), np.float32)
    uni = np.zeros((B, T_max), np.float32)
    for b in range(B):
        g = rng(w.cfg_id, STREAM_PROBS, b)
        T = int(tree_size[b])
        T = 1 if T < 1 or T > T_max else T
        for i in range(T):
            noise = g.gamma(concentration, size=V)
            kids = [c for c in range(1, T) if parents[b, c] == i]
            row = noise / noise.sum()
            if kids and g.random() < w.accept_prob:
                m = g.uniform(0.5, 0.95)
                x = int(draft_tokens[b, kids[int(g.integers(0, len(kids)))]])
                if 0 <= x < V:
                    row = row * (1.0 - m)
                    row[x] += m
            probs[b, i] = row.astype(np.float32)
        uni[b] = g.random(T_max).astype(np.float32)
    return probs, uni


def synthetic_target_logits(w: Workload, tree_size: np.ndarray, std_range=(0.5, 4.0), tie_step: float = 0.0):
    """Stand-in for the target model's raw logits at every tree node: N(0, s^2) with s
    drawn per request from std_range; with tie_step > 0 the values are rounded to
    multiples of it (many equal logits).  Rows of padding nodes are N(0, 1) too (they
    must not be read or written by the consumer).  float32 [B][T_max][V]."""
    B, T_max, V = len(tree_size), w.T_max, w.V
    out = np.zeros((B, T_max, V), np.float32)
    for b in range(B):
        g = rng(w.cfg_id, STREAM_TLOGITS, b)
        s = g.uniform(*std_range)
        x = g.standard_normal((T_max, V)) * s
        if tie_step > 0:
            x = np.round(x / tie_step) * tie_step
        out[b] = x.astype(np.float32)
    return out


def sampling_params(w: Workload, B: int):
    """Per-request sampling parameters, a mix of the usual settings: temperature in
    [0.3, 1.5] (0 = greedy for about one request in eight), top_k 0 (off) or in
    [1, min(V, 100)], top_p 1 (off) or in [0.5, 0.99], min_p 0 (off) or in
    [0.001, 0.2].  Returns float32 temperature, int32 top_k, float32 top_p, min_p."""
    g = rng(w.cfg_id, STREAM_TLOGITS, 10_000)
    temp = np.where(g.random(B) < 0.125, 0.0, g.uniform(0.3, 1.5, B)).astype(np.float32)
    top_k = np.where(g.random(B) < 0.5, 0, g.integers(1, min(w.V, 100) + 1, B)).astype(np.int32)
    top_p = np.where(g.random(B) < 0.4, 1.0, g.uniform(0.5, 0.99, B)).astype(np.float32)
    min_p = np.where(g.random(B) < 0.6, 0.0, g.uniform(0.001, 0.2, B)).astype(np.float32)
    return temp, top_k, top_p, min_p


def synthetic_draft_probs(w: Workload, draft_tokens: np.ndarray, parents: np.ndarray, tree_size: np.ndarray,
                          concentration: float = 0.3):
    """Stand-in for the drafter's distribution q at every node (the one its children
    were proposed from): Gamma(concentration) noise normalised to 1 - m plus mass
    m ~ U[0.3, 0.9] spread over the node's children's tokens with Dirichlet(1)
    weights (the drafter proposes tokens it likes); rows of nodes without children
    are noise only, rows of padding nodes zero.  float32 [B][T_max][V]."""
    B, T_max = draft_tokens.shape
    V = w.V
    q = np.zeros((B, T_max, V), np.float32)
    for b in range(B):
        g = rng(w.cfg_id, STREAM_DRAFTQ, b)
        T = int(tree_size[b])
        T = 1 if T < 1 or T > T_max else T
        for i in range(T):
            noise = g.gamma(concentration, size=V)
            row = noise / noise.sum()
            kids = [int(draft_tokens[b, c]) for c in range(1, T) if parents[b, c] == i]
            kids = [x for x in kids if 0 <= x < V]
            if kids:
                m = g.uniform(0.3, 0.9)
                row = row * (1.0 - m)
                wts = g.dirichlet(np.ones(len(kids)))
                for x, wt in zip(kids, wts):
                    row[x] += m * wt
            q[b, i] = row.astype(np.float32)
    return q
