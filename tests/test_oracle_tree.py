"""Pins for the oracle's tree construction (CPU only)."""
import json
import os

import numpy as np
import pytest

from oracle import OracleError
from oracle import tree as T
from synth import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_hand_worked_select_and_flatten():
    g = _load("tree_select_flatten.json")
    t = T.build_one(np.array(g["cand_parent"]), np.array(g["cand_token"]),
                    np.array(g["cand_score"], np.float32), g["budget"],
                    np.array(g["ret_token"]), np.array(g["ret_parent"]),
                    g["ctx_len"], g["V"])
    e = g["expect"]
    assert t["n"] == e["n"]
    for key in ("parent", "token", "depth", "pos", "mask", "src"):
        assert list(t[key]) == e[key], key


def test_hand_worked_static_replace():
    g = _load("tree_static_replace.json")
    table = np.zeros((g["V"], g["k"]), np.int32)
    for t in range(g["V"]):
        table[t] = [(t + 1) % g["V"], (t + 2) % g["V"]]
    for row, vals in g["table_rows"].items():
        table[int(row)] = vals
    t = T.build_one(np.array(g["cand_parent"]), np.array(g["cand_token"]),
                    np.array(g["cand_score"], np.float32), g["budget"],
                    np.zeros(0, np.int32), np.zeros(0, np.int32), g["ctx_len"], g["V"],
                    static_replace=True, table=table, replace_thresh=g["thresh"])
    e = g["expect"]
    for key in ("token", "src", "parent", "depth"):
        assert list(t[key]) == e[key], key


def _random_cands(seed, C=40, V=1000):
    r = np.random.default_rng(seed)
    parent = [-1] + [int(r.integers(0, c)) for c in range(1, C)]
    score = [1.0]
    for c in range(1, C):
        score.append(score[parent[c]] * float(r.choice([0.5, 0.25, 0.9, 1.0, r.uniform(0, 1)])))
    token = r.integers(0, V, C)
    return np.array(parent), token.astype(np.int32), np.array(score, np.float64).astype(np.float32)


@pytest.mark.parametrize("seed", range(20))
def test_selection_is_top_budget_and_ancestor_closed(seed):
    parent, token, score = _random_cands(seed)
    budget = 1 + seed % 30
    kept = T.select_draft(score, budget)
    assert kept[0] == 0 and len(kept) == min(budget, len(score))
    ks = set(kept)
    # defining property of top-B with the (score desc, index asc) order
    for a in kept[1:]:
        for b in range(1, len(score)):
            if b not in ks:
                assert score[a] > score[b] or (score[a] == score[b] and a < b)
    # non-increasing scores along paths -> the kept set is closed under parents
    for c in kept[1:]:
        assert parent[c] in ks


@pytest.mark.parametrize("seed", range(20))
def test_mask_depth_pos_invariants(seed):
    parent, token, score = _random_cands(seed, C=64)
    r = np.random.default_rng(100 + seed)
    budget = int(r.integers(1, 50))
    R = int(r.integers(0, 64 - budget + 1))
    rp = np.array([int(r.integers(-1, i)) for i in range(R)], np.int32)
    rt = r.integers(0, 1000, R).astype(np.int32)
    ctx = int(r.integers(0, 5000))
    t = T.build_one(parent, token, score, budget, rt, rp, ctx, 1000)
    n = t["n"]
    assert n == min(budget, 64) + R
    for i in range(n):
        m = t["mask"][i]
        assert (m >> i) & 1 == 1
        assert m < (1 << (i + 1))  # only earlier nodes can be ancestors
        if i == 0:
            assert t["parent"][0] == -1 and m == 1 and t["depth"][0] == 0
        else:
            p = t["parent"][i]
            assert 0 <= p < i
            # recursive characterisation of ancestor-or-self
            assert m == t["mask"][p] | (1 << i)
            assert t["depth"][i] == t["depth"][p] + 1
        assert bin(m).count("1") == t["depth"][i] + 1
        assert t["pos"][i] == ctx + t["depth"][i]
    for i in range(n):
        expect_src = 0 if i == 0 else (1 if i < min(budget, 64) else 2)
        assert t["src"][i] == expect_src


def test_chain_positions_are_consecutive():
    C = 30
    parent = np.arange(-1, C - 1)
    score = (0.9 ** np.arange(C)).astype(np.float32)
    t = T.build_one(parent, np.arange(C), score, C, np.zeros(0), np.zeros(0), 777, 1000)
    assert t["pos"] == list(range(777, 777 + C))
    assert t["mask"] == [(1 << (i + 1)) - 1 for i in range(C)]


def test_star_tree():
    C = 20
    parent = np.array([-1] + [0] * (C - 1))
    score = np.array([1.0] + [0.5] * (C - 1), np.float32)
    t = T.build_one(parent, np.arange(C), score, C, np.zeros(0), np.zeros(0), 5, 100)
    assert t["mask"] == [1] + [1 | (1 << i) for i in range(1, C)]
    assert t["depth"] == [0] + [1] * (C - 1)


@pytest.mark.parametrize("budget,R", [(8, 52), (24, 36), (40, 20)])
def test_graft_stage_budgets_fill_60_slots(budget, R):
    # Graft page, section 2: 8+52, 24+36, 40+20 of 60 slots
    assert budget + R == 60
    r = W.rng(99, "stage-test")
    p, tk, s = W.eagle_candidates(r, 5000, 5, 10, 10, 7)
    assert len(p) == 411
    rp = np.array([-1] * R, np.int32)
    t = T.build_one(p, tk, s, budget, np.arange(R), rp, 100, 5000)
    assert t["n"] == 60
    assert sum(1 for x in t["src"] if x == 2) == R


def test_eagle_prune_bver63_closed():
    r = W.rng(98, "eagle-test")
    p, tk, s = W.eagle_candidates(r, 5000, 5, 10, 10, 7)
    t = T.build_one(p, tk, s, 63, np.zeros(0), np.zeros(0), 0, 5000)
    assert t["n"] == 63
    assert max(t["depth"]) <= 5


def test_errors():
    p = np.array([-1, 0, 1])
    s = np.array([1.0, 0.1, 0.5], np.float32)  # child outranks its parent
    with pytest.raises(OracleError):
        T.build_one(p, np.array([1, 2, 3]), s, 2, np.zeros(0), np.zeros(0), 0, 10)
    with pytest.raises(OracleError):
        T.build_one(np.array([-1, 0]), np.array([1, 10]), np.array([1, .5], np.float32), 2,
                    np.zeros(0), np.zeros(0), 0, 10)
    with pytest.raises(OracleError):
        T.build_one(np.array([-1, 1]), np.array([1, 2]), np.array([1, .5], np.float32), 2,
                    np.zeros(0), np.zeros(0), 0, 10)
    with pytest.raises(OracleError):
        C = 70
        T.build_one(np.arange(-1, C - 1), np.arange(C), (0.9 ** np.arange(C)).astype(np.float32),
                    C, np.zeros(0), np.zeros(0), 0, 100)


def test_static_replace_properties():
    r = W.rng(97, "replace-test")
    V, k = 3000, 8
    p, tk, s = W.eagle_candidates(r, V, 5, 10, 10, 7)
    table = W.zipf_table(W.rng(97, "table"), V, k)
    base = T.build_one(p, tk, s, 60, np.zeros(0), np.zeros(0), 0, V)
    t = T.build_one(p, tk, s, 60, np.zeros(0), np.zeros(0), 0, V,
                    static_replace=True, table=table, replace_thresh=0.05)
    assert t["parent"] == base["parent"] and t["n"] == 60
    low = [i for i in range(1, 60) if t["score"][i] < 0.05]
    assert low, "workload should exercise replacement"
    lowset = set(low)
    for i in range(1, 60):
        # descendants of low nodes are low (scores fall along paths)
        if t["parent"][i] in lowset:
            assert i in lowset
        if t["src"][i] == 3:
            assert i in lowset
            assert t["token"][i] in set(table[t["token"][t["parent"][i]]].tolist())
        else:
            assert t["token"][i] == base["token"][i]


def test_nan_scores_rank_last():
    """A NaN candidate score ranks below every number (ties among NaNs and
    between -0 and +0 go to the lower index)."""
    score = np.array([1.0, np.nan, 0.5, -0.0, np.nan, 0.0, 0.25, 0.5], np.float32)
    assert T.select_draft(score, 1) == [0]
    assert T.select_draft(score, 3) == [0, 2, 7]
    assert T.select_draft(score, 6) == [0, 2, 3, 5, 6, 7]
    assert T.select_draft(score, 7) == [0, 1, 2, 3, 5, 6, 7]
    assert T.select_draft(score, 8) == list(range(8))


def test_hand_worked_retrieval_anchor():
    """Retrieval hangs under the deepest kept node of the best path at the
    checkpoint depth (tests/golden/tree_anchor.json, worked by hand)."""
    g = _load("tree_anchor.json")
    cp = np.array(g["cand_parent"])
    cs = np.array(g["cand_score"], np.float32)
    for case in g["cases"]:
        a = T.retrieval_anchor(cp, cs, case["budget"], case["depth_c"])
        assert a == case["anchor"], case["name"]
        t = T.build_one(cp, np.array(g["cand_token"]), cs, case["budget"], np.array(case["ret_token"]),
                        np.array(case["ret_parent"]), g["ctx_len"], g["V"], anchor=a)
        e = case["expect"]
        assert t["n"] == e["n"], case["name"]
        for key in ("parent", "token", "depth", "pos", "mask", "src"):
            assert list(t[key]) == e[key], (case["name"], key)


@pytest.mark.parametrize("seed", range(6))
def test_retrieval_anchor_properties(seed):
    """On the drafter stand-in's candidates: the anchor is kept; it lies on
    the root path of the best candidate at the checkpoint depth and no
    deeper node of that path is kept; checkpoint 0 gives the root; at
    checkpoint 1 the best depth-1 candidate is always kept (every other
    candidate scores at most as high as its own depth-1 ancestor)."""
    r = np.random.default_rng(seed)
    par, tok, sc = W.eagle_candidates(r, 5000, 5, 10, 10, 7)
    dep = T.candidate_depths(par)
    for depth_c, budget in ((0, 8), (1, 24), (5, 40), (5, 12), (3, 6), (9, 60)):
        a = T.retrieval_anchor(par, sc, budget, depth_c)
        kept = set(T.select_draft(sc, budget))
        assert a in kept
        c_eff = min(depth_c, max(dep))
        if c_eff == 0:
            assert a == 0
            continue
        at_c = [c for c in range(1, len(par)) if dep[c] == c_eff]
        best = max(at_c, key=lambda c: (float(sc[c]), -c))
        path = T.ancestors_or_self(list(par), best)
        assert a in path
        assert all(v not in kept for v in path[:path.index(a)])
        if depth_c == 1:
            assert a == best
