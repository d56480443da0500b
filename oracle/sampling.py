"""Oracle: the sampling side of verification (plain Python/numpy, float64 decisions).

Test infrastructure only (see oracle/__init__.py).

  * sampling_probs_row / tree_sampling_probs -- [TRT] section "non-greedy: rejection
    from the target distribution alone": before the rejection step the target's
    logits at every tree node are turned into probabilities with the request's
    sampling parameters (temperature, top-k, top-p, min-p); the per-request
    parameters are repeated over the request's nodes, each node filtered on its own.
  * accept_sample_draft / tree_accept_sample_draft -- [HB] exercise "trees when
    sampling": at a node the children (the drafter's candidates) are tried in turn,
    each accepted with probability min(1, p(x)/q(x)); after a rejection the target
    distribution becomes norm(max(0, p - q)) and q is adjusted to the way the
    candidates were drawn; when every child is rejected the correction token is
    drawn from the last residual and the walk ends.

Readings where the pages are silent (each listed with its reason in the design notes):
  filtering
  * the filters apply in the order temperature, top-k, top-p, min-p, each to what the
    previous one left;
  * tokens rank by (logit descending, token ascending) on the float32 logits; NaN
    ranks as -inf and -0.0 equals +0.0;
  * a temperature <= 0 (or NaN) is greedy: all mass on the first-ranked token;
  * a token's weight is exp((l - l_max) / temperature) in float64, exactly 1 for every
    token whose logit equals the largest (this defines +inf logits and an all -inf
    row), rounded to float32;
  * top-k (1 <= k < V) keeps the first k ranks;
  * top-p (< 1; NaN = off) keeps the shortest rank prefix of the top-k survivors whose
    cumulative weight reaches top_p x their total weight (so at least one token), in
    exact arithmetic: the cumulative and the total are the exact sums of the float32
    weights, and cumulative >= top_p x total is decided exactly with top_p's own
    float32 value (every float32 is an integer multiple of 2^-149, so Python integers
    in that unit hold the sums, and the comparison is one of integers);
  * min-p (> 0) drops tokens whose weight is below min_p x the largest weight (which is
    1); the first-ranked token is always kept;
  * the output is w / (sum of the kept w), float64 rounded to float32; dropped tokens
    get 0.
  draft-distribution acceptance
  * draft_probs[n] is q at node n: the drafter's distribution that node n's children
    were proposed from;
  * R and Q are the unnormalised target and draft residuals (R = p, Q = q when a node
    is entered), ZR and ZQ their float64 sums (recomputed after every change);
  * child c (ascending id) with token x, r = R(x) and s = Q(x) (both 0 for a token
    outside the vocabulary), is accepted iff r > 0 and (s == 0 or u_c s ZR < r ZQ),
    i.e. u_c < min(1, (r / ZR) / (s / ZQ)); products are rounded one at a time;
  * after a rejection R <- max(0, R ZQ - Q ZR) elementwise, which is norm(max(0, p'-q'))
    up to a positive factor (R is kept when ZQ = 0); with without_replacement the
    rejected token's draft mass is removed, Q(x) <- 0 (candidates drawn without
    replacement), otherwise Q is kept (candidates drawn independently);
  * the correction token is drawn from the final R exactly as tree.accept_sample draws
    it from its residual: the smallest v whose cumulative R (token order) exceeds
    u_0 x sum(R); if rounding leaves none, the last token with R > 0; with no residual
    mass, the node's best token by (p descending, token ascending).  At the depth cap
    the correction comes from the node's full row p.
"""
from __future__ import annotations

import numpy as np

from oracle.tree import ST_OK


# ---------------------------------------------------------------------------
# target logits -> filtered probabilities
# ---------------------------------------------------------------------------
def rank_order(logits):
    """Token order (logit descending, token ascending) of one float32 logit row, NaN
    ranked as -inf.  Returns (the cleaned float32 row, the order)."""
    lg = np.array(logits, dtype=np.float32)
    lg[np.isnan(lg)] = -np.inf
    lg[lg == 0.0] = 0.0                      # -0.0 -> +0.0 (they rank equal)
    order = np.lexsort((np.arange(lg.size), -lg.astype(np.float64)))
    return lg, order


def filter_weights(lg, temperature):
    """float32-rounded weights exp((l - l_max) / temperature), 1 at the largest logit."""
    lmax = lg.max()
    with np.errstate(invalid="ignore", over="ignore", under="ignore"):
        z = (lg.astype(np.float64) - np.float64(lmax)) / np.float64(temperature)
        w = np.where(lg == lmax, 1.0, np.exp(z))
    return w.astype(np.float32).astype(np.float64)


def sampling_probs_row(logits, temperature, top_k, top_p, min_p):
    """Filtered probabilities of one node's target logits ([TRT] probabilities from
    logits with temperature, top-k, top-p and min-p; readings in the module header)."""
    lg, order = rank_order(logits)
    V = lg.size
    out = np.zeros(V, np.float32)
    tau = float(np.float32(temperature))
    if not tau > 0.0:                        # greedy (NaN included)
        out[order[0]] = 1.0
        return out
    w = filter_weights(lg, tau)
    n = int(top_k) if 1 <= int(top_k) < V else V
    surv = order[:n]
    tp = float(np.float32(top_p))
    if tp < 1.0:
        # exact sums: w * 2^149 is an integer for every float32 w (the scaling by a
        # power of two is exact in float64), and top_p = num / den exactly
        units = [int(x * 2.0 ** 149) for x in w[surv]]
        num, den = tp.as_integer_ratio()
        target = num * sum(units)             # cumulative >= top_p x total  <=>  den x cumulative >= target
        cum = 0
        for n, x in enumerate(units):
            cum += x
            if den * cum >= target:
                surv = surv[:n + 1]
                break
    keep = np.zeros(V, bool)
    keep[surv] = True
    mp = float(np.float32(min_p))
    if mp > 0.0:
        keep &= w >= mp
        keep[order[0]] = True
    out[keep] = (w[keep] / w[keep].sum()).astype(np.float32)
    return out


def tree_sampling_probs(logits, tree_size, status, temperature, top_k, top_p, min_p, out):
    """Batch form: rows 0..T_b-1 of request b (T_b = 1 for a bad status or size) are
    filtered with request b's parameters; the other rows of `out` are left as given."""
    B, T_max, _ = logits.shape
    res = np.array(out, dtype=np.float32, copy=True)
    for b in range(B):
        T = int(tree_size[b])
        if int(status[b]) != ST_OK or T < 1 or T > T_max:
            T = 1
        for i in range(T):
            res[b, i] = sampling_probs_row(logits[b, i], temperature[b], top_k[b], top_p[b], min_p[b])
    return res


# ---------------------------------------------------------------------------
# acceptance with the drafter's distribution
# ---------------------------------------------------------------------------
def draw_from_residual(residual, row, u):
    """The correction token from an unnormalised residual (float64, token order)."""
    r = np.asarray(residual, dtype=np.float64)
    total = r.sum()
    if not total > 0.0:
        return int(np.argsort(-np.asarray(row, np.float32), kind="stable")[0])
    cum = np.cumsum(r)
    hit = np.nonzero(cum > u * total)[0]
    if len(hit):
        return int(hit[0])
    return int(np.nonzero(r > 0.0)[0][-1])


def accept_sample_draft(draft_tokens, parents, tree_size: int, target_probs, draft_probs, uniforms, status: int,
                        dcap: int, without_replacement: bool):
    """Tree rejection sampling with the drafter's distribution q ([HB] exercise
    "trees when sampling"; readings in the module header).  uniforms[c] (c >= 1) is
    child c's draw, uniforms[0] the correction's.  Returns accept_len, the padded
    path (root first) and the correction (bonus) token."""
    path = [0]
    node = 0
    R = None
    if status == ST_OK:
        T = int(tree_size)
        while len(path) <= dcap:
            p = np.asarray(target_probs[node], dtype=np.float64)
            V = p.size
            R = p.copy()
            Q = np.asarray(draft_probs[node], dtype=np.float64).copy()
            ZR, ZQ = R.sum(), Q.sum()
            nxt = None
            for c in (c for c in range(1, T) if parents[c] == node):
                x = int(draft_tokens[c])
                inside = 0 <= x < V
                r = float(R[x]) if inside else 0.0
                s = float(Q[x]) if inside else 0.0
                if r > 0.0 and (s == 0.0 or float(uniforms[c]) * s * ZR < r * ZQ):
                    nxt = c
                    break
                if ZQ > 0.0:
                    R = np.maximum(0.0, R * ZQ - Q * ZR)
                    ZR = R.sum()
                if without_replacement and inside:
                    Q[x] = 0.0
                    ZQ = Q.sum()
            if nxt is None:
                break
            path.append(nxt)
            node = nxt
            R = None
    row = target_probs[node]
    residual = R if R is not None else np.asarray(row, dtype=np.float64)
    bonus = draw_from_residual(residual, row, float(uniforms[0]))
    padded = path + [-1] * (dcap + 1 - len(path))
    return len(path) - 1, padded, bonus


def tree_accept_sample_draft(draft_tokens, parents, tree_size, target_probs, draft_probs, uniforms, status,
                             dcap: int, without_replacement: bool):
    B = draft_tokens.shape[0]
    alen = np.zeros(B, np.int32)
    apath = np.full((B, dcap + 1), -1, np.int32)
    bonus = np.zeros(B, np.int32)
    for b in range(B):
        a, p, bt = accept_sample_draft(list(draft_tokens[b]), list(parents[b]), int(tree_size[b]), target_probs[b],
                                       draft_probs[b], uniforms[b], int(status[b]), dcap, without_replacement)
        alen[b], apath[b], bonus[b] = a, p, bt
    return dict(accept_len=alen, accept_path=apath, bonus_token=bonus)
