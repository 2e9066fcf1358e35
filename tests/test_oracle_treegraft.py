"""Pins of the TreeGraft construction oracle (oracle/treegraft.py): a
hand-worked two-step example in which a mid step re-grafts at the root and
revives a child the small drafter ranked lower, against the same example
with a small second step; properties read off the output (small-step
frontiers are the previous step's best W; a mid step never re-expands a node
an earlier mid step had in its pool; growth only, by m children per chosen
node; the node count); and the result is a valid input of the global prune
(oracle.tree keeps an ancestor-closed set)."""
import numpy as np
import pytest

from oracle import treegraft as TG
from oracle import tree as OTree


def _example(mid_mask):
    # D = 2, W = 2, m = 2.  Step 0 from the root: children 1 (p 0.6, q 0.3)
    # and 2 (p 0.4, q 0.9).  Step 1's drafter outputs per frontier rank.
    tok = np.array([[[11, 12], [0, 0]], [[21, 22], [23, 24]]])
    p = np.array([[[0.6, 0.4], [0, 0]], [[0.5, 0.25], [0.75, 0.125]]], np.float32)
    q = np.array([1.0, 0.3, 0.9, 0.5, 0.5, 0.5, 0.5], np.float32)
    return TG.build(50, 2, 2, 2, mid_mask, tok, p, q)


def test_hand_worked_small_then_mid():
    # TreeGraft page, section 4: the mid step's pool is every node it has not
    # visited, {0, 1, 2}, ranked by its own path score r: r0 = 1, r2 = 0.9,
    # r1 = 0.3, so it grafts under the root (which keeps children 1 and 2)
    # and under node 2, which the small drafter ranked below node 1.
    parent, token, s = _example(0b10)
    assert parent == [-1, 0, 0, 0, 0, 2, 2]
    assert token == [50, 11, 12, 21, 22, 23, 24]
    assert s == [1.0, 0.6000000238418579, 0.4000000059604645, 0.5, 0.25,
                 float(np.float32(np.float32(0.4) * np.float32(0.75))),
                 float(np.float32(np.float32(0.4) * np.float32(0.125)))]


def test_hand_worked_small_then_small():
    # TreeGraft page, section 3: a small step's pool is the newest nodes
    # {1, 2} by stored score, so node 1 (0.6) comes first
    parent, token, s = _example(0b00)
    assert parent == [-1, 0, 0, 1, 1, 2, 2]
    assert token == [50, 11, 12, 21, 22, 23, 24]


def _random(r, D, W, m, mid_mask, V=1000):
    tok = r.integers(0, V, (D, W, m))
    p = np.sort(r.dirichlet(np.full(m, 0.3), (D, W)), axis=-1)[..., ::-1].astype(np.float32)
    q = r.random(TG.node_count(D, W, m, mid_mask)).astype(np.float32)
    return tok, p, q


@pytest.mark.parametrize("mid_mask", [0b00000, 0b00100, 0b01010, 0b11111, 0b00001])
def test_properties_read_off_the_output(mid_mask):
    r = np.random.default_rng(mid_mask + 3)
    D, W, m = 5, 10, 10
    tok, p, q = _random(r, D, W, m, mid_mask)
    parent, token, s = TG.build(7, D, W, m, mid_mask, tok, p, q)
    n = len(parent)
    assert n == TG.node_count(D, W, m, mid_mask)
    # creation step of every node, and each step's frontier (the parents of
    # the nodes it created, each chosen node with exactly m new children)
    step = [0] * n
    frontier = {}
    # nodes are created in blocks of m under consecutive frontier nodes
    sizes, newest, visited, cnt = [], 1, 0, 1
    for k in range(D):
        mid = (mid_mask >> k) & 1
        f = min(W, (cnt - visited) if mid else newest)
        if mid:
            visited = cnt
        sizes.append(f)
        newest = f * m
        cnt += newest
    base = 1
    for k in range(D):
        fr = []
        for j in range(sizes[k]):
            kids = list(range(base + j * m, base + (j + 1) * m))
            assert len({parent[c] for c in kids}) == 1
            fr.append(parent[kids[0]])
            for c in kids:
                step[c] = k + 1
        frontier[k] = fr
        base += sizes[k] * m
    assert base == n
    r_score = [1.0] * n
    for v in range(1, n):
        r_score[v] = float(np.float32(np.float32(r_score[parent[v]]) * q[v]))
    seen_by_mid = set()
    for k in range(D):
        if (mid_mask >> k) & 1:
            pool = [v for v in range(n) if step[v] <= k and v not in seen_by_mid]
            best = sorted(pool, key=lambda v: (-r_score[v], v))[:W]
            assert frontier[k] == best
            assert not (set(frontier[k]) & seen_by_mid)
            seen_by_mid |= set(pool)
        else:
            pool = [v for v in range(n) if step[v] == k]
            assert frontier[k] == sorted(pool, key=lambda v: (-s[v], v))[:W]
    # scores never grow along a path, so the global prune keeps a closed set
    t = OTree.build_one(parent, token, s, 63, [], [], 0, 1000)
    assert t["n"] == 63


def test_all_small_schedule_is_the_standard_construction_size():
    assert TG.node_count(5, 10, 10, 0) == 1 + 10 + 4 * 100   # 411, the EAGLE workloads' candidate count


def test_ties_go_to_the_lower_node_index():
    tok = np.array([[[11, 12]], [[21, 22]]])
    p = np.array([[[0.5, 0.5]], [[0.5, 0.5]]], np.float32)   # nodes 1 and 2 tie (s = r = 0.5)
    q = np.array([1.0, 0.5, 0.5, 0.5, 0.5], np.float32)
    for mask in (0b00, 0b10):  # small step: pool {1, 2}; mid step: pool {0, 1, 2}, root first
        parent, _, _ = TG.build(50, 2, 1, 2, mask, tok, p, q)
        assert parent[3:] == ([1, 1] if mask == 0 else [0, 0])
    tok2 = np.array([[[11, 12]], [[21, 22]], [[31, 32]]])
    p2 = np.array([[[0.5, 0.5]], [[0.5, 0.5]], [[0.5, 0.5]]], np.float32)
    q2 = np.ones(7, np.float32)
    # all r equal to 1: the second mid step's pool {3, 4} (0..2 were visited) -> node 3
    parent, _, _ = TG.build(50, 3, 1, 2, 0b110, tok2, p2, q2)
    assert parent[3:5] == [0, 0] and parent[5:] == [3, 3]
