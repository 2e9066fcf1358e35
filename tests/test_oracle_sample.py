"""Pins of the sampling-acceptance oracle (oracle/sample.py).

* Gumbel-max draws match softmax(l / T) in frequency (chi-square over 10^5
  draws per temperature), reduce to the argmax as T -> 0, and break ties to
  the lower id.
* Losslessness, exactly: on small trees (duplicate siblings included) with
  given per-node target distributions, enumerating every joint draw with
  rational weights shows that the first emitted token has the root's
  distribution and, after a matched first token, the second has the matched
  child's distribution -- token-by-token sampling of the target.
* At the argmax draw the rule equals greedy acceptance (oracle.accept) on
  trees without duplicate siblings."""
import itertools
from fractions import Fraction

import numpy as np
import pytest

from oracle import OracleError
from oracle import accept as OAcc
from oracle import sample as OS


def gumbel(r, shape):
    u = r.random(shape)
    u = np.clip(u, 1e-300, 1.0 - 1e-16)
    return (-np.log(-np.log(u))).astype(np.float32)


@pytest.mark.parametrize("T", [0.5, 1.0, 2.0])
def test_gumbel_max_frequencies_follow_softmax(T):
    r = np.random.default_rng(int(T * 10))
    logits = np.array([1.0, 0.2, -0.5, 2.0, 0.0, -3.0], np.float32)
    n = 100_000
    ids = OS.sample_rows(np.tile(logits, (n, 1)), T, gumbel(r, (n, logits.size)))
    freq = np.bincount(ids, minlength=logits.size)
    p = np.exp(logits.astype(np.float64) / T)
    p /= p.sum()
    chi2 = float(np.sum((freq - n * p) ** 2 / (n * p)))
    assert chi2 < 30.0, (chi2, freq, n * p)  # 5 dof: P(chi2 > 30) < 2e-5


def test_temperature_scales_the_logits_not_the_noise():
    # at T = 2 a logit gap of 2 is a score gap of 1: with g = (0, 0.9) the
    # lower logit loses, with g = (0, 1.1) it wins
    l = np.array([[2.0, 0.0], [2.0, 0.0]], np.float32)
    g = np.array([[0.0, 0.9], [0.0, 1.1]], np.float32)
    assert OS.sample_rows(l, 2.0, g).tolist() == [0, 1]


def test_small_temperature_gives_the_argmax_and_ties_go_low():
    r = np.random.default_rng(3)
    l = r.standard_normal((200, 50)).astype(np.float32)
    assert np.array_equal(OS.sample_rows(l, 1e-4, gumbel(r, l.shape)), np.argmax(l, axis=1))
    assert OS.sample_rows(np.zeros((1, 7), np.float32), 1.0, np.zeros((1, 7), np.float32)).tolist() == [0]
    with pytest.raises(OracleError):
        OS.sample_rows(l, 0.0, gumbel(r, l.shape))


def _distribution_of_emissions(parent, token, dists, V):
    """Exact distribution of (first emitted token, second emitted token or
    None) over every joint draw, weights = product of the per-node
    probabilities."""
    n = len(parent)
    out = {}
    for draw in itertools.product(range(V), repeat=n):
        w = Fraction(1)
        for u in range(n):
            w *= dists[u][draw[u]]
        if w == 0:
            continue
        a, path, bonus = OS.accept_sampled_one(parent, token, draw)
        emitted = [token[i] for i in path[1:]] + [bonus]
        key = (emitted[0], emitted[1] if len(emitted) > 1 else None)
        out[key] = out.get(key, Fraction(0)) + w
    return out


@pytest.mark.parametrize("tree", [
    ([-1, 0, 0, 1, 2], [9, 0, 1, 2, 0]),          # two children at the root
    ([-1, 0, 0, 0, 1], [9, 1, 1, 2, 0]),          # duplicate siblings (token 1)
    ([-1, 0, 1, 2], [9, 2, 0, 1]),                # a chain
])
def test_emitted_tokens_follow_the_target_exactly(tree):
    parent, token = tree
    V = 3
    r = np.random.default_rng(len(parent))
    dists = []
    for _ in parent:
        w = r.integers(1, 6, V)
        dists.append([Fraction(int(x), int(w.sum())) for x in w])
    dist = _distribution_of_emissions(parent, token, dists, V)
    first = {}
    for (x1, _), w in dist.items():
        first[x1] = first.get(x1, Fraction(0)) + w
    for x in range(V):
        assert first.get(x, Fraction(0)) == dists[0][x]
    for x1 in range(V):
        kids = [c for c in range(1, len(parent)) if parent[c] == 0 and token[c] == x1]
        if not kids:
            continue
        c = kids[0]  # the lowest-index matching child carries the prefix x1
        for x2 in range(V):
            joint = dist.get((x1, x2), Fraction(0))
            assert joint == dists[0][x1] * dists[c][x2], (x1, x2)


def test_argmax_draws_give_greedy_acceptance():
    r = np.random.default_rng(11)
    for _ in range(300):
        n = int(r.integers(1, 15))
        parent = [-1] + [int(r.integers(0, i)) for i in range(1, n)]
        token = [0]
        for i in range(1, n):  # distinct tokens among siblings
            used = {token[j] for j in range(1, i) if parent[j] == parent[i]}
            token.append(min(set(range(20)) - used))
        am = r.integers(0, 4, n)
        assert OS.accept_sampled_one(parent, token, am) == OAcc.accept_one(parent, token, am)


def test_duplicate_siblings_only_the_first_counts():
    parent = [-1, 0, 0, 2]
    token = [5, 7, 7, 3]
    sample = [7, 1, 3, 0]  # node 2's subtree would go deeper
    assert OS.accept_sampled_one(parent, token, sample) == (1, [0, 1], 1)
    assert OAcc.accept_one(parent, token, sample)[0] == 2  # greedy takes the deeper one
