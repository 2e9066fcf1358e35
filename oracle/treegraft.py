"""TreeGraft's shared draft tree built by two drafters (oracle; test
infrastructure only).

TreeGraft page, section 3 (the standard single-drafter construction: at step
k the frontier F_k is the top-W of the candidate pool C_k by cumulative path
score s(v), the product of edge scores from the root, and every frontier node
gets its top-m children; the tree is finally pruned globally by s to the
verification budget) and section 4 ("Where": a mid-drafter step takes as its
pool every node the mid drafter has not yet visited, C_k = V(T_k) minus P_k,
rescoring them with its own distribution, while a small-drafter step keeps
C_k = N_k, the nodes the previous step created, with their stored scores; the
visited set grows by C_k after a mid step only.  "How": new children are
attached without overwriting anything; the global prune to Bver = 63 comes
last).  The drafters themselves and the schedule of mid steps ("When") are
out of scope and come in as inputs.  Readings:

* the drafter stand-in's output for step k is child tokens tok[k][j][c] and
  edge probabilities p[k][j][c] for the j-th best frontier node (c < m);
* the mid drafter's own score of node v is r(v), the product along the path
  of its edge probabilities q[v] (an input per node, by creation index,
  q[root] unused, r(root) = 1); a mid step ranks its pool by r, a small step
  by s;
* a child of frontier node f gets s = fl(s(f) * p) and r = fl(r(f) * q[child])
  (fp32 products); ties in ranking go to the lower node index;
* nodes are numbered in creation order (the root 0, then step by step, the
  j-th frontier node's children consecutively), which is topological.

The result is the candidate set of graft_build_tree (parent, token, score=s);
its prune to Bver is oracle.tree.
"""
from __future__ import annotations

import numpy as np

from . import OracleError
from .tree import score_rank_key


def node_count(D: int, W: int, m: int, mid_mask: int) -> int:
    """Nodes the construction creates (root included); depends on the sizes
    and the schedule only."""
    n, newest, visited = 1, 1, 0
    for k in range(D):
        pool = (n - visited) if (mid_mask >> k) & 1 else newest
        f = min(W, pool)
        if (mid_mask >> k) & 1:
            visited = n
        newest = f * m
        n += newest
    return n


def build(root_token: int, D: int, W: int, m: int, mid_mask: int, tok, p, q):
    """tok, p: [D][W][m]; q: [node_count] (q[0] unused).  Returns
    (parent, token, s) lists in creation order."""
    if D < 0 or W < 1 or m < 1:
        raise OracleError("bad sizes")
    tok = np.asarray(tok)
    p = np.asarray(p, np.float32)
    q = np.asarray(q, np.float32)
    parent, token = [-1], [int(root_token)]
    s, r = [np.float32(1.0)], [np.float32(1.0)]
    created = [0]       # step after which the node exists (root: 0)
    visited = [False]
    for k in range(D):
        mid = bool((mid_mask >> k) & 1)
        if mid:
            pool = [v for v in range(len(parent)) if not visited[v]]
            score = r
        else:
            pool = [v for v in range(len(parent)) if created[v] == k]
            score = s
        frontier = sorted(pool, key=lambda v: score_rank_key(score[v], v))[:W]
        if mid:
            for v in pool:
                visited[v] = True
        for j, f in enumerate(frontier):
            for c in range(m):
                idx = len(parent)
                if idx >= len(q):
                    raise OracleError("q shorter than the tree")
                parent.append(f)
                token.append(int(tok[k, j, c]))
                s.append(np.float32(s[f] * p[k, j, c]))
                r.append(np.float32(r[f] * q[idx]))
                created.append(k + 1)
                visited.append(False)
    return parent, token, [float(x) for x in s]
