"""The stage-adaptive retrieval template (oracle; test infrastructure only).

The Graft page (section 2, second step) fixes only properties of the
template: it is asymmetric -- successors of higher rank get more children
and reach deeper, forming a main continuation chain, while lower ranks keep
a few children for width (in the spirit of Token Recycling) -- and it fills
the slots pruning freed: 52, 36 or 20 of 60.  Section 5 of the same page
finds depth 8 and width about 8 best.

Reading used here (the exact shape is not printed on the pages, so the
template's shape is parity-unpinned against them; it is pinned against this
rule by brute force in the tests):
  nodes are rank paths (r1, ..., rd), 0 <= r < k, 1 <= d <= dmax = 8, each
  standing for "the r-th ranked successor of the previous token";
  score(path) = prod 0.75 / (r + 1);
  the template of size R is the R best paths ordered by score descending,
  then depth ascending, then the rank path lexicographically ascending.
A parent's score is strictly larger than its child's, so the R best paths
form a tree and the order is topological.

Scores are exact rationals (fractions.Fraction), so there is no rounding.
Output: tparent[t] = template index of the path without its last rank, or
-1 when that is the root; trank[t] = the last rank.
"""
from __future__ import annotations

import heapq
from fractions import Fraction

Q_NUM = Fraction(3, 4)


def path_score(path) -> Fraction:
    s = Fraction(1)
    for r in path:
        s *= Q_NUM / (r + 1)
    return s


def template(R: int, k: int, dmax: int = 8):
    """Best-first expansion from the root: a heap keyed by (-score, depth,
    path) pops paths in exactly the template order because every path's
    ancestors score strictly higher."""
    if R < 0 or k < 1 or dmax < 1:
        raise ValueError("bad template size")
    order: list[tuple] = []
    heap = [(-path_score((r,)), 1, (r,)) for r in range(k)]
    heapq.heapify(heap)
    while heap and len(order) < R:
        neg, dep, path = heapq.heappop(heap)
        order.append(path)
        if dep < dmax:
            for r in range(k):
                child = path + (r,)
                heapq.heappush(heap, (-path_score(child), dep + 1, child))
    if len(order) < R:
        raise ValueError("template larger than the k-ary tree of depth dmax")
    index = {p: t for t, p in enumerate(order)}
    tparent = [index[p[:-1]] if len(p) > 1 else -1 for p in order]
    trank = [p[-1] for p in order]
    return tparent, trank, order
