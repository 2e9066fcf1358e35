"""Pins for the oracle's retrieval template (CPU only).

The pages give the template's properties, not its node list (Graft page,
section 2, second step; section 5 depth/width sweep), so the exact shape is
parity-unpinned against the pages.  These tests pin the oracle against
(a) a brute-force enumeration of the stated rule and (b) the properties the
pages do state."""
from fractions import Fraction
from itertools import product

import pytest

from oracle.template import template


def brute_force_template(R, k, dmax):
    """Enumerate every rank path, score it as an exact rational, sort."""
    paths = []
    for d in range(1, dmax + 1):
        # prod (r+1) grows fast: only small ranks can reach the top R, but
        # enumerate exhaustively for small k/dmax
        for p in product(range(k), repeat=d):
            s = Fraction(1)
            for r in p:
                s *= Fraction(3, 4) / (r + 1)
            paths.append((-s, d, p))
    paths.sort()
    return [p for _, _, p in paths[:R]]


@pytest.mark.parametrize("R,k,dmax", [(10, 3, 4), (25, 4, 5), (40, 3, 6), (60, 5, 4), (1, 2, 1)])
def test_template_matches_brute_force(R, k, dmax):
    _, _, order = template(R, k, dmax)
    assert order == brute_force_template(R, k, dmax)


def bounded_enumeration(R, k, dmax, pmax):
    """All paths with prod(r+1) <= pmax (depth-first), sorted by the rule."""
    out = []

    def rec(p, prod_):
        if p:
            s = Fraction(1)
            for r in p:
                s *= Fraction(3, 4) / (r + 1)
            out.append((-s, len(p), tuple(p)))
        if len(p) == dmax:
            return
        for r in range(k):
            if prod_ * (r + 1) <= pmax:
                rec(p + [r], prod_ * (r + 1))

    rec([], 1)
    out.sort()
    return [p for _, _, p in out[:R]]


@pytest.mark.parametrize("R", [20, 36, 52])
def test_graft_sizes_match_bounded_enumeration(R):
    _, _, order = template(R, 8, 8)
    s_last = Fraction(1)
    for r in order[-1]:
        s_last *= Fraction(3, 4) / (r + 1)
    # any path scoring >= s_last has prod(r+1) <= 1/s_last
    pmax = int(1 / s_last) + 1
    assert order == bounded_enumeration(R, 8, 8, pmax)


def test_graft_template_properties():
    t20 = template(20, 8, 8)[2]
    t36 = template(36, 8, 8)[2]
    t52 = template(52, 8, 8)[2]
    # sizes: the slots pruning frees at stages 5 / 1 / 0 (Graft page, section 2)
    assert (len(t20), len(t36), len(t52)) == (20, 36, 52)
    # nested: a larger budget only adds nodes
    assert t20 == t36[:20] and t36 == t52[:36]
    for order in (t20, t36, t52):
        s = set(order)
        for p in order:
            assert len(p) <= 8
            if len(p) > 1:
                assert p[:-1] in s  # closed under parents -> a tree
                assert order.index(p[:-1]) < order.index(p)  # topological
    # depth 8 and width 8 at the largest budget (Graft page, section 5 optimum)
    assert max(len(p) for p in t52) == 8
    assert sum(1 for p in t52 if len(p) == 1) == 8
    # asymmetric: higher-ranked successors own larger subtrees and reach deeper
    sizes = [sum(1 for p in t52 if p[0] == r) for r in range(8)]
    depths = [max(len(p) for p in t52 if p[0] == r) for r in range(8)]
    assert sizes == sorted(sizes, reverse=True) and sizes[0] > sizes[1]
    assert depths == sorted(depths, reverse=True) and depths[0] == 8


def test_template_parent_rank_encoding():
    tp, tr, order = template(52, 8, 8)
    for t, p in enumerate(order):
        assert tr[t] == p[-1]
        if len(p) == 1:
            assert tp[t] == -1
        else:
            assert order[tp[t]] == p[:-1]
