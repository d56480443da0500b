"""Oracle: draft-tree build, tree metadata and greedy acceptance (plain Python/numpy).

Test infrastructure only (see oracle/__init__.py).  Everything here works on one
request at a time with Python lists; the batch wrappers at the bottom loop over
requests and produce the padded arrays the library's calls produce.

Conventions fixed where the pages leave them open (each is listed with its reason
in the design notes):
  * ranking everywhere is the total order (value descending, index ascending);
    -0.0 ranks equal to +0.0;
  * dynamic scores are float32 sums of log-probs, one round-to-nearest add per level,
    root score 0;
  * after the final selection the kept candidates are numbered in ascending
    candidate id (node 0 is the root), which is level order;
  * tree_size counts the root;
  * padding: tokens / parents / retrieve entries -1, scores -inf, mask bits 0,
    positions 0.
Status codes: 0 ok, 1 malformed parents, 2 depth above the cap, 3 tree size out of
range, 4 non-finite or positive log-prob or a kept node whose parent was not kept.
A request with non-zero status is treated as the root-only tree downstream.
"""
from __future__ import annotations

import numpy as np

ST_OK, ST_PARENTS, ST_DEPTH, ST_SIZE, ST_LOGPROB = 0, 1, 2, 3, 4


# ---------------------------------------------------------------------------
# per-row top-k
# ---------------------------------------------------------------------------
def row_topk(row: np.ndarray, k: int):
    """The k best tokens of one draft row by (log-prob descending, token ascending).

    [E2] section 3 takes torch.topk of the draft model's log-probs for every expanded
    node; [HB] build_draft_tree takes logits.topk(width).  Ties are left open by both;
    the lower token id wins here.  A stable argsort of the negated values gives
    exactly that order (equal values keep ascending index; -0.0 equals +0.0)."""
    row = np.asarray(row, dtype=np.float32)
    order = np.argsort(-row, kind="stable")[:k]
    return [int(t) for t in order], [np.float32(row[t]) for t in order]


def row_is_valid(row: np.ndarray) -> bool:
    """Log-probs must be <= 0 and not NaN (-inf, a zero-probability token, is allowed)."""
    row = np.asarray(row, dtype=np.float32)
    return not (np.isnan(row).any() or (row > 0).any())


def _root_only(root_token, T_max):
    tokens = [-1] * T_max
    parents = [-1] * T_max
    scores = [np.float32(-np.inf)] * T_max
    tokens[0] = int(root_token)
    scores[0] = np.float32(0.0)
    return tokens, parents, scores, 1


# ---------------------------------------------------------------------------
# dynamic tree build ([E2] section 3; [TRT] _select_topk_draft_tokens)
# ---------------------------------------------------------------------------
def build_dynamic(logprobs: np.ndarray, root_token: int, K: int, D: int, total_tokens: int, T_max: int):
    """EAGLE-2 dynamic tree for one request.

    logprobs[R][V], R = 1 + D*K: row 0 is the draft distribution after the root;
    row 1 + (l-1)*K + j is the distribution after frontier slot j of layer l
    (l = 1..D), i.e. what the draft forward on that frontier node would give.

    Steps ([E2] section 3, first/second/third step):
      base layer: the K best tokens of row 0 become candidates 0..K-1 (parent = root,
        score = their log-prob) and, in rank order, the first frontier;
      each of D rounds: every frontier slot j expands into its row's K best tokens
        r = 0..K-1 with cumulative score fl32(logprob + score of slot j); the K*K
        new candidates get ids K + (l-1)K^2 + jK + r and the K best of them (score
        descending, jK+r ascending) become the next frontier (the global, joint
        pruning over K*K, cu_scores = topk_p + scores);
      final: of all C = K + D*K^2 candidates keep the total_tokens best (score
        descending, id ascending), number them 1..T-1 in ascending id, node 0 is
        the root, and rewrite every parent as a node index.
    [TRT] forms the same cumulative score as a product of probabilities; the sum of
    log-probs orders identically in exact arithmetic and is used here.
    Returns tokens, parents, scores (lists of length T_max), tree_size, status."""
    R = 1 + D * K
    if not all(row_is_valid(logprobs[r]) for r in range(R)):
        return (*_root_only(root_token, T_max), ST_LOGPROB)
    cand_score, cand_token, cand_parent = [], [], []      # parent: candidate id or -1 (root)
    toks, vals = row_topk(logprobs[0], K)
    for r in range(K):
        cand_score.append(vals[r])
        cand_token.append(toks[r])
        cand_parent.append(-1)
    frontier = list(range(K))
    fscore = list(vals)
    for l in range(1, D + 1):
        base = len(cand_score)
        layer_scores = []
        for j in range(K):
            toks, vals = row_topk(logprobs[1 + (l - 1) * K + j], K)
            for r in range(K):
                s = np.float32(vals[r] + fscore[j])        # one float32 add, round to nearest
                cand_score.append(s)
                cand_token.append(toks[r])
                cand_parent.append(frontier[j])
                layer_scores.append(s)
        order = sorted(range(K * K), key=lambda q: (-layer_scores[q], q))
        frontier = [base + q for q in order[:K]]
        fscore = [layer_scores[q] for q in order[:K]]
    return _select_and_number(cand_score, cand_token, cand_parent, root_token, total_tokens, T_max)


def _select_and_number(cand_score, cand_token, cand_parent, root_token, total_tokens, T_max):
    """The final step of [E2] section 3: keep the total_tokens best candidates (score
    descending, id ascending), number them 1..T-1 in ascending id, node 0 = root,
    rewrite parents as node indices (a kept node whose parent was dropped -> status 4)."""
    C = len(cand_score)
    order = sorted(range(C), key=lambda c: (-cand_score[c], c))
    chosen = sorted(order[:total_tokens])
    node_of = {c: 1 + n for n, c in enumerate(chosen)}
    tokens, parents, scores, _ = _root_only(root_token, T_max)
    for n, c in enumerate(chosen, start=1):
        p = cand_parent[c]
        if p != -1 and p not in node_of:                     # kept node whose parent was dropped
            return (*_root_only(root_token, T_max), ST_LOGPROB)
        tokens[n] = cand_token[c]
        parents[n] = 0 if p == -1 else node_of[p]
        scores[n] = cand_score[c]
    return tokens, parents, scores, 1 + len(chosen), ST_OK


# ---------------------------------------------------------------------------
# layer-by-layer dynamic build ([E2] section 3: the draft model runs on the
# current frontier between rounds, so a round's rows exist only once the round
# before it has chosen its frontier)
# ---------------------------------------------------------------------------
def log_softmax_row(z: np.ndarray) -> np.ndarray:
    """fp32 logits -> fp32 log-probs: fp32(z - lse), lse = m + log(sum(exp(z - m))) in
    float64 with m = max(z) (the draft head's log-softmax, [E2] section 3)."""
    z64 = np.asarray(z, dtype=np.float32).astype(np.float64)
    m = z64.max()
    with np.errstate(invalid="ignore", over="ignore"):   # non-finite rows are rejected by the caller
        lse = m + np.log(np.exp(z64 - m).sum())
        return (z64 - lse).astype(np.float32)


def logits_row_topk(z: np.ndarray, k: int):
    """The k best tokens of a row of fp32 logits by (logit descending, token ascending),
    which is the order of the row's log-softmax before its values are rounded, and
    their log-probs (log_softmax_row)."""
    toks, _ = row_topk(z, k)
    lp = log_softmax_row(z)
    return toks, [np.float32(lp[t]) for t in toks]


def logits_row_is_valid(z: np.ndarray) -> bool:
    return bool(np.isfinite(np.asarray(z, dtype=np.float32)).all())


def build_dynamic_layers(layers, root_token: int, K: int, D: int, total_tokens: int, T_max: int,
                         logits: bool = False):
    """build_dynamic taking its rows one layer at a time, as a draft loop produces them.

    layers[0] is the root's row ([V] or [1][V]); layers[l] (l = 1..D) is [K][V], row j
    the draft distribution after frontier slot j of layer l.  With logits=True the rows
    are raw logits: each row is ranked by logit and scored by its log-softmax
    (logits_row_topk).  Same rounds and final selection as build_dynamic.
    Returns tokens, parents, scores, tree_size, status, and frontiers: frontiers[l] =
    (tokens [K], parent slots [K]) of the frontier chosen at layer l, the parent slot
    being the slot of layer l-1's frontier it extends (-1 at layer 0)."""
    topk = logits_row_topk if logits else row_topk
    valid = logits_row_is_valid if logits else row_is_valid
    rows0 = np.asarray(layers[0]).reshape(-1, np.asarray(layers[0]).shape[-1])
    all_rows = [rows0[0]] + [np.asarray(layers[l])[j] for l in range(1, D + 1) for j in range(K)]
    ok = all(valid(r) for r in all_rows)
    cand_score, cand_token, cand_parent = [], [], []
    toks, vals = topk(rows0[0], K)
    for r in range(K):
        cand_score.append(vals[r])
        cand_token.append(toks[r])
        cand_parent.append(-1)
    frontier, fscore = list(range(K)), list(vals)
    frontiers = [(list(toks), [-1] * K)]
    for l in range(1, D + 1):
        base = len(cand_score)
        layer_scores, layer_tokens = [], []
        for j in range(K):
            toks, vals = topk(np.asarray(layers[l])[j], K)
            for r in range(K):
                s = np.float32(vals[r] + fscore[j])
                cand_score.append(s)
                cand_token.append(toks[r])
                cand_parent.append(frontier[j])
                layer_scores.append(s)
                layer_tokens.append(toks[r])
        order = sorted(range(K * K), key=lambda q: (-layer_scores[q], q))[:K]
        frontier = [base + q for q in order]
        fscore = [layer_scores[q] for q in order]
        frontiers.append(([layer_tokens[q] for q in order], [q // K for q in order]))
    if not ok:
        return (*_root_only(root_token, T_max), ST_LOGPROB, frontiers)
    return (*_select_and_number(cand_score, cand_token, cand_parent, root_token, total_tokens, T_max), frontiers)


# ---------------------------------------------------------------------------
# static tree build ([HB] build_draft_tree)
# ---------------------------------------------------------------------------
def build_static(logprobs: np.ndarray, root_token: int, branching, T_max: int):
    """Static branching tree: starting from the root, every node of the current
    frontier (in order) appends the top-branching[l] tokens of its own draft row as
    children; the new nodes, in append order, are the next frontier.  Row n of
    logprobs is the draft distribution after node n (the nodes that get expanded
    are exactly 0..R-1 because nodes are appended level by level).
    The score of a node is fl32(its log-prob + its parent's score), root 0."""
    R = logprobs.shape[0]
    tokens, parents, scores = [int(root_token)], [-1], [np.float32(0.0)]
    frontier = [0]
    for width in branching:
        nxt = []
        for node in frontier:
            if node >= R or not row_is_valid(logprobs[node]):
                return (*_root_only(root_token, T_max), ST_LOGPROB)
            toks, vals = row_topk(logprobs[node], width)
            for t, v in zip(toks, vals):
                tokens.append(t)
                parents.append(node)
                scores.append(np.float32(v + scores[node]))
                nxt.append(len(tokens) - 1)
        frontier = nxt
    T = len(tokens)
    if T > T_max:
        raise ValueError(f"static tree of {T} nodes exceeds T_max={T_max}")
    pad = T_max - T
    return (tokens + [-1] * pad, parents + [-1] * pad, scores + [np.float32(-np.inf)] * pad, T, ST_OK)


# ---------------------------------------------------------------------------
# tree metadata ([HB] tree_mask / depths; [E2] section 3 third step; [TRT] build op)
# ---------------------------------------------------------------------------
def validate(parents, tree_size: int, T_max: int, dcap: int) -> int:
    """Structural checks: 3 if tree_size is outside [1, T_max]; 1 if parents[0] != -1
    or some parents[i] (1 <= i < T) is outside [0, i); 2 if a node is deeper than dcap."""
    T = int(tree_size)
    if T < 1 or T > T_max:
        return ST_SIZE
    if parents[0] != -1:
        return ST_PARENTS
    for i in range(1, T):
        if not (0 <= parents[i] < i):
            return ST_PARENTS
    depth = [0] * T
    for i in range(1, T):
        depth[i] = depth[parents[i]] + 1
        if depth[i] > dcap:
            return ST_DEPTH
    return ST_OK


def ancestor_sets(parents, T: int):
    """Row i of the tree mask as an integer bitset: node i and all of its ancestors
    ([HB] tree_mask; [TRT] packed ancestor mask).  The ancestor relation is the
    transitive closure of the parent relation; since a validated tree numbers every
    parent before its children, the closure follows in one pass in node order:
    A(i) = {i} united with A(parent of i)."""
    rows = []
    for i in range(T):
        rows.append((1 << i) | (rows[parents[i]] if parents[i] >= 0 else 0))
    return rows


def depths(parents, T: int):
    """Depth of every node ([HB] depths; [E2] tree_position_ids): the number of its
    ancestors other than itself, read off the ancestor bitsets."""
    return [bin(a).count("1") - 1 for a in ancestor_sets(parents, T)]


def mask_positions(parents, tree_size: int, prefix_len: int, T_max: int, dcap: int, status_in: int = 0):
    """Everything the tree-build kernel of [TRT] derives from parent pointers, for one
    request: packed ancestor mask ([TRT] packed mask, 32 nodes per uint32, bit j&31
    of word j>>5), per-node depth (tree_position_ids, [E2]) and absolute position
    prefix_len + depth ([HB]: position = committed length + depth; siblings share it),
    retrieve_indices (one row per leaf, leaves in ascending id, root..leaf along the
    parent chain, [E2] section 3), first-child / next-sibling lists ([TRT]).
    A request that fails validation (or arrives with non-zero status) gets the
    root-only tree."""
    W = (T_max + 31) // 32
    status = status_in if status_in != ST_OK else validate(parents, tree_size, T_max, dcap)
    if status != ST_OK:
        T, par = 1, [-1]
    else:
        T, par = int(tree_size), list(parents[:tree_size])
    rows = ancestor_sets(par, T)
    dep = depths(par, T)
    mask = np.zeros((T_max, W), dtype=np.uint32)
    for i in range(T):
        for w in range(W):
            mask[i, w] = np.uint32((rows[i] >> (32 * w)) & 0xFFFFFFFF)
    tpos = np.zeros(T_max, np.int32)
    pos = np.zeros(T_max, np.int32)
    for i in range(T):
        tpos[i] = dep[i]
        pos[i] = prefix_len + dep[i]
    children = [[c for c in range(1, T) if par[c] == i] for i in range(T)]
    leaves = [i for i in range(T) if not children[i]]
    ri = np.full((T_max, dcap + 1), -1, np.int32)
    for r, leaf in enumerate(leaves):
        chain = []
        j = leaf
        while j != -1:
            chain.append(j)
            j = par[j]
        for k, n in enumerate(reversed(chain)):
            ri[r, k] = n
    first_child = np.full(T_max, -1, np.int32)
    next_sibling = np.full(T_max, -1, np.int32)
    for i in range(T):
        kids = children[i]
        if kids:
            first_child[i] = kids[0]
        for a, b in zip(kids, kids[1:]):
            next_sibling[a] = b
    return dict(tree_mask=mask, tree_position_ids=tpos, positions=pos, retrieve_indices=ri,
                leaf_count=len(leaves), first_child=first_child, next_sibling=next_sibling, status=status)


# ---------------------------------------------------------------------------
# greedy acceptance ([HB] tree_speculative_generate walk; [TRT] greedy verification;
# [E2] section 5 evaluate_posterior)
# ---------------------------------------------------------------------------
def accept_walk(draft_tokens, parents, tree_size: int, target_predict, status: int, dcap: int):
    """From the root, repeatedly move to the lowest-index child whose draft token equals
    the target's prediction at the current node; stop when no child matches.
    accept_len counts accepted draft nodes (root excluded); the path starts at the
    root; the bonus token is the target's prediction at the last node of the path."""
    path = [0]
    if status == ST_OK:
        T = int(tree_size)
        # (parent, token) -> the lowest-index child of that parent carrying that token
        step = {}
        for c in range(1, T):
            step.setdefault((int(parents[c]), int(draft_tokens[c])), c)
        while len(path) <= dcap:
            nxt = step.get((path[-1], int(target_predict[path[-1]])))
            if nxt is None:
                break
            path.append(nxt)
    padded = path + [-1] * (dcap + 1 - len(path))
    return len(path) - 1, padded, int(target_predict[path[-1]])


def _residual_sample(row, removed, u):
    """A token from norm(row with the `removed` tokens' mass taken out): the smallest v
    whose cumulative residual mass exceeds u times the residual total (float64, in
    token order); if rounding leaves no such v, the last token with residual mass, and
    with no residual mass at all the row's best token (probability desc, token asc)."""
    r = np.asarray(row, dtype=np.float64).copy()
    if removed:
        r[sorted(removed)] = 0.0
    total = r.sum()
    if not total > 0.0:
        return int(np.argsort(-np.asarray(row, np.float32), kind="stable")[0])
    cum = np.cumsum(r)
    hit = np.nonzero(cum > u * total)[0]
    if len(hit):
        return int(hit[0])
    return int(np.nonzero(r > 0.0)[0][-1])


def accept_sample(draft_tokens, parents, tree_size: int, target_probs, uniforms, status: int, dcap: int):
    """Tree rejection sampling with the target distribution only ([TRT] "non-greedy:
    rejection sampling from the target distribution alone"; [HB] exercise "trees
    when sampling": at a node, consider its children in order, accept each with
    min(1, p(x)/q(x)); on rejection continue with norm(max(0, p - q)); if every child
    is rejected, sample the correction token from the final residual).

    The tree's candidates are the drafter's deterministic top-K picks, so q for a
    candidate is the point mass on its token: the acceptance test is p(x) against
    the remaining mass, and the residual is p with the rejected tokens' mass removed.
    target_probs[i] is the target's (already filtered) distribution at node i;
    uniforms[c] (c >= 1) is the draw for child c's test, uniforms[0] the draw for the
    correction token.  At node n with row p, Z = sum(p) and R = the mass of the tokens
    rejected so far at n (float64): child c (ascending id) with token x is accepted iff
    uniforms[c] * (Z - R) < p(x) (p(x) = 0 for an already-rejected token).  The walk
    stops at depth dcap (the correction is then sampled from the full row there).
    Returns accept_len, the padded path (root first) and the correction (bonus) token."""
    path = [0]
    node = 0
    removed = set()
    if status == ST_OK:
        T = int(tree_size)
        while True:
            removed = set()
            if len(path) > dcap:
                break
            row = np.asarray(target_probs[node], dtype=np.float64)
            Z = row.sum()
            R = 0.0
            nxt = None
            for c in (c for c in range(1, T) if parents[c] == node):
                x = int(draft_tokens[c])
                inside = 0 <= x < len(row)                  # a token outside the vocabulary has no mass
                px = 0.0 if (x in removed or not inside) else float(row[x])
                if float(uniforms[c]) * (Z - R) < px:
                    nxt = c
                    break
                if inside and x not in removed:
                    R += px
                    removed.add(x)
            if nxt is None:
                break
            path.append(nxt)
            node = nxt
    bonus = _residual_sample(target_probs[node], removed, float(uniforms[0]))
    padded = path + [-1] * (dcap + 1 - len(path))
    return len(path) - 1, padded, bonus


def accept_posterior(draft_tokens, retrieve_rows, leaf_count: int, target_predict):
    """[E2] section 5: for every retrieve row (a root-to-leaf path) mark position k >= 1
    accepted when the draft token there equals the target's argmax at position k-1;
    the cumulative product along the row counts the leading accepted positions; the
    best row is the one with the most, the lowest row index on ties."""
    best_len, best_row = -1, 0
    for r in range(leaf_count):
        row = [n for n in retrieve_rows[r] if n != -1]
        flags = [1 if draft_tokens[row[k]] == target_predict[row[k - 1]] else 0 for k in range(1, len(row))]
        run = int(np.cumprod([1] + flags).sum()) - 1
        if run > best_len:
            best_len, best_row = run, r
    row = [n for n in retrieve_rows[best_row] if n != -1]
    return best_len, row[:best_len + 1]


# ---------------------------------------------------------------------------
# batch wrappers (padded arrays, the library's layouts)
# ---------------------------------------------------------------------------
def tree_build(w):
    """Batch tree build for a workload object (dynamic / static / given)."""
    B, T_max = w.B, w.T_max
    tok = np.full((B, T_max), -1, np.int32)
    par = np.full((B, T_max), -1, np.int32)
    score = np.full((B, T_max), -np.inf, np.float32)
    size = np.zeros(B, np.int32)
    status = np.zeros(B, np.int32)
    for b in range(B):
        if w.mode == "dynamic":
            t, p, s, n, st = build_dynamic(w.logprobs[b], int(w.root_token[b]), w.K, w.D, w.total_tokens, T_max)
        elif w.mode == "static":
            t, p, s, n, st = build_static(w.logprobs[b], int(w.root_token[b]), w.branching, T_max)
        else:
            t, p, n, st = list(w.given_tokens[b]), list(w.given_parents[b]), int(w.given_size[b]), ST_OK
            s = [np.float32(-np.inf)] * T_max
        tok[b], par[b], score[b], size[b], status[b] = t, p, s, n, st
    return dict(draft_tokens=tok, parents=par, node_score=score, tree_size=size, status=status)


def tree_mask_positions(parents, tree_size, prefix_len, T_max: int, dcap: int, status_in=None):
    B = parents.shape[0]
    W = (T_max + 31) // 32
    out = dict(tree_mask=np.zeros((B, T_max, W), np.uint32), tree_position_ids=np.zeros((B, T_max), np.int32),
               positions=np.zeros((B, T_max), np.int32),
               retrieve_indices=np.full((B, T_max, dcap + 1), -1, np.int32),
               leaf_count=np.zeros(B, np.int32), first_child=np.full((B, T_max), -1, np.int32),
               next_sibling=np.full((B, T_max), -1, np.int32), status=np.zeros(B, np.int32))
    for b in range(B):
        st_in = 0 if status_in is None else int(status_in[b])
        r = mask_positions(list(parents[b]), int(tree_size[b]), int(prefix_len[b]), T_max, dcap, st_in)
        for k, v in r.items():
            out[k][b] = v
    return out


def tree_accept_sample(draft_tokens, parents, tree_size, target_probs, uniforms, status, dcap: int):
    B = draft_tokens.shape[0]
    alen = np.zeros(B, np.int32)
    apath = np.full((B, dcap + 1), -1, np.int32)
    bonus = np.zeros(B, np.int32)
    for b in range(B):
        a, p, bt = accept_sample(list(draft_tokens[b]), list(parents[b]), int(tree_size[b]), target_probs[b],
                                 uniforms[b], int(status[b]), dcap)
        alen[b], apath[b], bonus[b] = a, p, bt
    return dict(accept_len=alen, accept_path=apath, bonus_token=bonus)


def tree_accept(draft_tokens, parents, tree_size, target_predict, status, dcap: int):
    B = draft_tokens.shape[0]
    alen = np.zeros(B, np.int32)
    apath = np.full((B, dcap + 1), -1, np.int32)
    bonus = np.zeros(B, np.int32)
    for b in range(B):
        a, p, bt = accept_walk(list(draft_tokens[b]), list(parents[b]), int(tree_size[b]),
                               list(target_predict[b]), int(status[b]), dcap)
        alen[b], apath[b], bonus[b] = a, p, bt
    return dict(accept_len=alen, accept_path=apath, bonus_token=bonus)
