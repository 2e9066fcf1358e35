"""Pins for the oracle's greedy acceptance (CPU only)."""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import OracleError
from oracle.accept import accept_batch, accept_one

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def brute(parent, token, argmax):
    """Enumerate every node's root path and check each edge on it."""
    n = len(parent)
    best, best_depth = 0, 0
    for i in range(n):
        path = []
        j = i
        while j >= 0:
            path.append(j)
            j = parent[j]
        path.reverse()
        ok = all(token[path[t + 1]] == argmax[path[t]] for t in range(len(path) - 1))
        if ok and len(path) - 1 > best_depth:
            best, best_depth = i, len(path) - 1
    path = []
    j = best
    while j >= 0:
        path.append(j)
        j = parent[j]
    return best_depth, path[::-1], argmax[best]


def test_golden_cases():
    with open(os.path.join(GOLD, "accept_small.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        a, path, bonus = accept_one(c["parent"], c["token"], c["argmax"])
        e = c["expect"]
        assert (a, path, bonus) == (e["acc_len"], e["path"], e["bonus"])


@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 6, 7])
def test_exhaustive_parent_arrays(N):
    r = np.random.default_rng(N)
    # every parent array with parent[i] < i
    for parents in itertools.product(*[range(i) for i in range(1, N)]):
        parent = [-1] + list(parents)
        for _ in range(3 if N == 7 else 6):
            token = r.integers(0, 3, N).tolist()
            argmax = r.integers(0, 3, N).tolist()
            assert accept_one(parent, token, argmax) == brute(parent, token, argmax)


@pytest.mark.parametrize("seed", range(200))
def test_random_trees_up_to_15(seed):
    r = np.random.default_rng(1000 + seed)
    N = int(r.integers(1, 16))
    parent = [-1] + [int(r.integers(0, i)) for i in range(1, N)]
    token = r.integers(0, 2, N).tolist()
    argmax = r.integers(0, 2, N).tolist()
    assert accept_one(parent, token, argmax) == brute(parent, token, argmax)


def _target(path_tokens):
    # a deterministic "target model": next token is a function of the prefix
    h = 1469598103934665603
    for t in path_tokens:
        h = ((h ^ t) * 1099511628211) & ((1 << 64) - 1)
    return h % 3


def _argmax_for(parent, token):
    out = []
    for i in range(len(parent)):
        path = []
        j = i
        while j >= 0:
            path.append(token[j])
            j = parent[j]
        out.append(_target(path[::-1]))
    return out


@pytest.mark.parametrize("seed", range(100))
def test_superset_tree_accepts_at_least_as_much(seed):
    # Graft page, section 3: a larger tree never shortens the accepted
    # prefix; the Graft tree (kept draft nodes + retrieved ones) contains
    # the pruned tree, so it accepts at least as much.
    r = np.random.default_rng(seed)
    n_small = int(r.integers(1, 12))
    parent = [-1] + [int(r.integers(0, i)) for i in range(1, n_small)]
    token = [0] + r.integers(0, 3, n_small - 1).tolist()
    a_small, _, _ = accept_one(parent, token, _argmax_for(parent, token))
    big_p, big_t = list(parent), list(token)
    for i in range(int(r.integers(0, 20))):
        big_p.append(int(r.integers(0, len(big_p))))
        big_t.append(int(r.integers(0, 3)))
    a_big, _, _ = accept_one(big_p, big_t, _argmax_for(big_p, big_t))
    assert a_big >= a_small


def test_prefix_survival_expectation():
    # BlockPilot page, section 8: with per-position acceptance p_j the
    # expected accepted length of a chain is sum_i prod_{j<=i} p_j.
    p = [0.9, 0.8, 0.7, 0.6, 0.5, 0.4]
    n = len(p) + 1
    parent = [-1] + list(range(n - 1))
    r = np.random.default_rng(123)
    trials = 20000
    lens = np.empty(trials)
    for t in range(trials):
        token = [0] + [1] * (n - 1)
        argmax = [1 if r.random() < p[j] else 2 for j in range(n - 1)] + [0]
        lens[t] = accept_one(parent, token, argmax)[0]
    expect = sum(np.prod(p[: i + 1]) for i in range(len(p)))
    sigma = lens.std() / np.sqrt(trials)
    assert abs(lens.mean() - expect) < 3 * sigma


def test_batch_layout_and_errors():
    parent = np.array([-1, 0, -1, -1, 0, 1], np.int32)
    token = np.array([0, 1, 9, 0, 2, 3], np.int32)
    argmax = np.array([1, 5, 9, 2, 3, 7], np.int32)
    # request 0 rows 0..1 (+1 padding), request 1 rows 3..5
    lens, paths, bonus = accept_batch([2, 3], [0, 3, 6], parent, token, argmax)
    assert lens == [1, 2] and paths == [[0, 1], [0, 1, 2]] and bonus == [5, 7]
    with pytest.raises(OracleError):
        accept_one([-1, 1], [0, 0], [0, 0])
