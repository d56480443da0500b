"""Pins for the oracle's tree build and tree metadata (CPU only).

What fixes the expected values (none of them come from the oracle itself):
  * the handbook's printed six-node mask and its exercise node counts (tests/golden);
  * a dynamic tree worked by hand (tests/golden/hand_dynamic_tree.json);
  * closed forms: K-ary trees (parent (i-1)//K, the dummy-slot tree of the
    TensorRT-LLM dissection) and the chain (top_k = 1);
  * special cases: K = 1 gives the chain of row argmaxes, total_tokens = C keeps every
    candidate, D = 0 keeps the top tokens of the root row;
  * an independent brute-force restatement of the dynamic build (recursive over
    token paths, scores summed along each path) on many tiny random inputs;
  * invariants of ancestor masks on random trees.
"""
import json
import os

import numpy as np
import pytest

from oracle import tree as ot
from workloads import gen

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def mask_bits(mask_rows, T):
    return ["".join("1" if (int(r[j >> 5]) >> (j & 31)) & 1 else "0" for j in range(T)) for r in mask_rows[:T]]


# ----------------------------------------------------------------------------- golden
def test_handbook_six_node_mask():
    g = load("handbook_six_node_mask.json")
    par = g["parents"] + [-1] * (64 - 6)
    r = ot.mask_positions(par, 6, 100, 64, 7)
    assert r["status"] == 0
    assert mask_bits(r["tree_mask"], 6) == g["mask_rows"]
    # siblings share a position: nodes 1, 2 (children of 0) and 3, 4 (children of 1)
    assert list(r["positions"][:6]) == [100, 101, 101, 102, 102, 102]


def test_handbook_node_counts():
    for case in load("handbook_node_counts.json")["cases"]:
        br = case["branching"]
        nrow = 1 + sum(int(np.prod(br[:l + 1])) for l in range(len(br) - 1))
        lp = np.log(np.full((nrow, 50), 1 / 50, np.float64)).astype(np.float32)
        lp += np.linspace(0, -1, 50, dtype=np.float32)
        tok, par, sc, T, st = ot.build_static(lp, 7, br, 64)
        assert st == 0 and T - 1 == case["draft_nodes"]
        # level widths multiply as the branching list says
        d = ot.depths(par, T)
        for l, w in enumerate(br):
            assert d.count(l + 1) == int(np.prod(br[:l + 1]))


def test_hand_worked_dynamic_tree():
    g = load("hand_dynamic_tree.json")
    lp = np.array(g["rows"], np.float32)
    for tt, exp in g["expected"].items():
        tt = int(tt)
        tok, par, sc, T, st = ot.build_dynamic(lp, g["root_token"], g["K"], g["D"], tt, 64)
        assert st == 0 and T == tt + 1
        assert tok[:T] == exp["tokens"]
        assert par[:T] == exp["parents"]
        assert [float(s) for s in sc[:T]] == exp["scores"]
        assert all(t == -1 for t in tok[T:]) and all(p == -1 for p in par[T:])
        if "mask_rows" in exp:
            r = ot.mask_positions(par, T, 0, 64, 7)
            assert mask_bits(r["tree_mask"], T) == exp["mask_rows"]
            assert list(r["tree_position_ids"][:T]) == exp["depths"]
            rows = [[n for n in row if n != -1] for row in r["retrieve_indices"][:r["leaf_count"]]]
            assert rows == exp["retrieve"]


# ----------------------------------------------------------------------------- closed forms
def kary_depth(i, K):
    """Level of node i in a complete K-ary tree numbered level by level:
    the first L levels hold 1 + K + ... + K^(L-1) nodes."""
    level, first = 0, 0
    while True:
        width = K ** level
        if i < first + width:
            return level
        first += width
        level += 1


@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_kary_tree_closed_form(K):
    T = 40 if K > 1 else 8
    par = [-1] + [(i - 1) // K for i in range(1, T)] + [-1] * (64 - T)
    r = ot.mask_positions(par, T, 10, 64, 63)
    assert r["status"] == 0
    for i in range(T):
        assert r["tree_position_ids"][i] == kary_depth(i, K)
        assert r["positions"][i] == 10 + kary_depth(i, K)
    if K == 1:  # the chain: full lower-triangular mask and one path
        assert mask_bits(r["tree_mask"], T) == ["1" * (i + 1) + "0" * (T - i - 1) for i in range(T)]
        assert r["leaf_count"] == 1
        assert list(r["retrieve_indices"][0][:T]) == list(range(T))


def test_chain_from_k1_dynamic_build():
    rng = np.random.default_rng(5)
    D, V = 5, 30
    lp = np.log(rng.dirichlet(np.ones(V), size=1 + D)).astype(np.float32)
    tok, par, sc, T, st = ot.build_dynamic(lp, 11, 1, D, D + 1, 64)
    assert st == 0 and T == D + 2
    assert par[:T] == [-1] + list(range(T - 1))
    assert tok[1:T] == [int(np.argmax(lp[r])) for r in range(1 + D)]


def test_keep_everything_and_depth_zero():
    rng = np.random.default_rng(6)
    K, D, V = 3, 2, 12
    C = K + D * K * K
    lp = np.log(rng.dirichlet(np.ones(V), size=1 + D * K)).astype(np.float32)
    tok, par, sc, T, st = ot.build_dynamic(lp, 0, K, D, C, 64)
    assert st == 0 and T == C + 1
    d = ot.depths(par, T)
    assert [d.count(l) for l in range(D + 2)] == [1, K] + [K * K] * D
    # D = 0: root plus the top tokens of row 0, in rank order (ascending candidate id)
    tok, par, sc, T, st = ot.build_dynamic(lp[:1], 0, K, 0, 2, 64)
    order = np.argsort(-lp[0], kind="stable")
    assert T == 3 and tok[1:3] == [int(order[0]), int(order[1])] and par[:3] == [-1, 0, 0]


# ----------------------------------------------------------------------------- brute force
def brute_dynamic(lp, root, K, D, total):
    """Independent restatement: a candidate is identified by its path of (row, token)
    choices; its score is the float32 running sum of the row log-probs along the
    path; each round ranks all children of the current frontier at once."""
    def ranked(row):
        return sorted(range(len(row)), key=lambda t: (-float(row[t]), t))[:K]

    everything = []        # (score, creation index, path tuple of tokens, parent path)
    base = [((t,), np.float32(lp[0][t])) for t in ranked(lp[0])]
    for p, s in base:
        everything.append((s, len(everything), p, ()))
    frontier = base
    for l in range(1, D + 1):
        kids = []
        for j, (p, s) in enumerate(frontier):
            row = lp[1 + (l - 1) * K + j]
            for t in ranked(row):
                kids.append((p + (t,), np.float32(np.float32(row[t]) + s), p))
        for q, (p, s, parent) in enumerate(kids):
            everything.append((s, len(everything), p, parent))
        best = sorted(range(len(kids)), key=lambda q: (-float(kids[q][1]), q))[:K]
        frontier = [(kids[q][0], kids[q][1]) for q in best]
    keep = sorted(sorted(everything, key=lambda e: (-float(e[0]), e[1]))[:total], key=lambda e: e[1])
    index = {e[2]: n + 1 for n, e in enumerate(keep)}
    tokens = [root] + [e[2][-1] for e in keep]
    parents = [-1] + [index[e[3]] if e[3] else 0 for e in keep]
    return tokens, parents, [0.0] + [float(e[0]) for e in keep]


def test_dynamic_build_brute_force():
    rng = np.random.default_rng(2024)
    n = 0
    for trial in range(400):
        K = int(rng.integers(1, 4))
        D = int(rng.integers(0, 3))
        V = int(rng.integers(K, 9))
        C = K + D * K * K
        total = int(rng.integers(1, C + 1))
        # coarse values on a dyadic grid force plenty of ties
        lp = -(rng.integers(0, 6, size=(1 + D * K, V)) / 4.0).astype(np.float32)
        tok, par, sc, T, st = ot.build_dynamic(lp, 1, K, D, total, 64)
        bt, bp, bs = brute_dynamic(lp, 1, K, D, total)
        assert st == 0
        assert tok[:T] == bt and par[:T] == bp and [float(s) for s in sc[:T]] == bs, trial
        n += 1
    assert n == 400


def brute_static(lp, root, branching):
    """Independent restatement of the static build: a node is named by its tuple of
    child ranks from the root; nodes are numbered level by level with the tuples in
    lexicographic order (= frontier order); tokens are then filled depth-first,
    each node reading the draft row with its own number."""
    all_keys = [()]
    for l, width in enumerate(branching):
        all_keys += sorted(k + (r,) for k in all_keys if len(k) == l for r in range(width))
    all_keys.sort(key=lambda k: (len(k), k))
    num = {k: n for n, k in enumerate(all_keys)}
    tok = {(): root}

    def fill(key):
        if len(key) == len(branching):
            return
        row = lp[num[key]]
        ranked = sorted(range(len(row)), key=lambda t: (-float(row[t]), t))
        for r in range(branching[len(key)]):
            tok[key + (r,)] = ranked[r]
            fill(key + (r,))
    fill(())
    tokens = [tok[k] for k in all_keys]
    parents = [-1] + [num[k[:-1]] for k in all_keys[1:]]
    return tokens, parents


def test_static_build_brute_force():
    rng = np.random.default_rng(99)
    for trial in range(200):
        br = [int(x) for x in rng.integers(1, 4, size=int(rng.integers(1, 4)))]
        nrow = 1 + sum(int(np.prod(br[:l + 1])) for l in range(len(br) - 1))
        lp = -(rng.integers(0, 5, size=(nrow, 7)) / 2.0).astype(np.float32)
        tok, par, sc, T, st = ot.build_static(lp, 3, br, 64)
        bt, bp = brute_static(lp, 3, br)
        assert st == 0 and tok[:T] == bt and par[:T] == bp, trial


def test_dynamic_build_properties_on_config_shapes():
    """Properties of a kept set on a full-size draft: ancestor-closed, BFS order, scores
    non-increasing along paths, every kept score >= every dropped one (top-T), kept
    children of a node are a prefix of that node's ranked children."""
    w = gen.make_workload(2)
    r = ot.tree_build(w)
    T = int(r["tree_size"][0])
    par, sc = list(r["parents"][0]), list(r["node_score"][0])
    assert T == 61 and r["status"][0] == 0
    for i in range(1, T):
        assert 0 <= par[i] < i
        assert sc[i] <= sc[par[i]]
    d = ot.depths(par, T)
    assert d == sorted(d)                                   # level order


# ----------------------------------------------------------------------------- invariants
def random_parents(rng, T):
    return [-1] + [int(rng.integers(0, i)) for i in range(1, T)]


def test_mask_invariants_random_trees():
    rng = np.random.default_rng(7)
    for trial in range(300):
        T = int(rng.integers(1, 65))
        par = random_parents(rng, T)
        r = ot.mask_positions(par + [-1] * (64 - T), T, 33, 64, 63)
        assert r["status"] == 0
        bits = mask_bits(r["tree_mask"], T)
        d = r["tree_position_ids"]
        for i in range(T):
            assert bits[i][i] == "1" and bits[i][0] == "1"          # self and root
            assert bits[i][i + 1:] == "0" * (T - i - 1)             # lower-triangular
            assert bits[i].count("1") == d[i] + 1                   # popcount = depth + 1
            if i:
                # row i = row of parent plus bit i
                assert bits[i][:i] + "0" == bits[par[i]][:i + 1]
                assert r["positions"][i] == r["positions"][par[i]] + 1
        # padding rows / bits are zero
        assert not r["tree_mask"][T:].any()
        kids = {i: [c for c in range(1, T) if par[c] == i] for i in range(T)}
        leaves = [i for i in range(T) if not kids[i]]
        assert r["leaf_count"] == len(leaves)
        covered = set()
        for k, leaf in enumerate(leaves):
            row = [n for n in r["retrieve_indices"][k] if n != -1]
            assert row[0] == 0 and row[-1] == leaf
            for a, b in zip(row, row[1:]):
                assert par[b] == a
            covered |= set(row)
        assert covered == set(range(T))
        assert (r["retrieve_indices"][len(leaves):] == -1).all()
        # child / sibling lists enumerate each node's children in ascending order
        for i in range(T):
            walk, c = [], r["first_child"][i]
            while c != -1:
                walk.append(int(c))
                c = r["next_sibling"][c]
            assert walk == kids[i]


@pytest.mark.parametrize("bad,code", [
    ({"parents": [0, 0, 1]}, ot.ST_PARENTS),            # root parent must be -1
    ({"parents": [-1, 1, 0]}, ot.ST_PARENTS),           # self loop
    ({"parents": [-1, 0, 3, 1]}, ot.ST_PARENTS),        # parent after child
    ({"parents": [-1, 0, 1, 2, 3], "dcap": 3}, ot.ST_DEPTH),
    ({"parents": [-1, 0], "size": 0}, ot.ST_SIZE),
    ({"parents": [-1, 0], "size": 65}, ot.ST_SIZE),
])
def test_validation_and_root_only_fallback(bad, code):
    par = bad["parents"] + [-1] * (64 - len(bad["parents"]))
    size = bad.get("size", len(bad["parents"]))
    r = ot.mask_positions(par, size, 50, 64, bad.get("dcap", 7))
    assert r["status"] == code
    assert mask_bits(r["tree_mask"], 3) == ["100", "000", "000"]
    assert r["positions"][0] == 50 and r["leaf_count"] == 1
    assert list(r["retrieve_indices"][0][:2]) == [0, -1]


def test_bad_logprobs_give_root_only():
    lp = np.full((1 + 2 * 2, 8), -1.0, np.float32)
    lp[3, 5] = 0.5                         # a positive log-prob
    tok, par, sc, T, st = ot.build_dynamic(lp, 4, 2, 2, 4, 64)
    assert st == ot.ST_LOGPROB and T == 1 and tok[0] == 4 and par[0] == -1
    lp[3, 5] = np.nan
    assert ot.build_dynamic(lp, 4, 2, 2, 4, 64)[4] == ot.ST_LOGPROB
    lp[3, 5] = -np.inf                     # zero probability is allowed
    assert ot.build_dynamic(lp, 4, 2, 2, 4, 64)[4] == ot.ST_OK


def test_config_trees_have_the_expected_sizes():
    sizes = {1: [11], 2: [61], 3: [49] * 2, 4: [61]}
    for cfg, exp in sizes.items():
        w = gen.make_workload(cfg, batch=len(exp), with_attention=False)
        r = ot.tree_build(w)
        assert list(r["tree_size"][:len(exp)]) == exp
        assert (r["status"] == 0).all()
