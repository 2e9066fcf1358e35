"""Tree construction for one verify round (oracle; test infrastructure only).

* Draft selection.  The root (candidate 0) is always kept; of the other
  candidates the `budget - 1` with the highest cumulative score are kept.
  The cumulative score of a node is the product of the edge scores on its
  root path and the tree is pruned globally by it (TreeGraft page, section
  3, problem definition; section 4 "How": global prune to Bver).  Graft's
  stage budgets keep 8 / 24 / 40 draft nodes of 60 slots (Graft page,
  section 2, second step).  Ties in score go to the lower candidate index.
* Retrieved nodes are appended after the kept draft nodes, in template
  order; a template parent of -1 means the retrieval anchor (Graft page,
  section 2, second step: when pruning triggers at a checkpoint depth, the
  retrieval tree is expanded from the token generated up to that point and
  fills the slots pruning freed).  Reading (retrieval_anchor): the current
  best path at checkpoint depth c ends at the candidate of depth c with the
  highest cumulative score; the anchor is the deepest kept node on that
  path (all of it when the budget keeps it).  At checkpoint 0 the anchor is
  the root.
* Static replacement (Graft page, section 4, batched-serving paragraph):
  the per-request slot count stays fixed and low-confidence draft nodes are
  swapped for retrieved tokens.  Reading: a node whose score is below the
  threshold takes token table[token(parent)][j], j = its 0-based order among
  its low-score siblings; j >= k keeps the draft token.  The parent token
  is the final (possibly replaced) one.
* Flatten (Graft page, section 2, third step: the hybrid tree is flattened,
  tree positions and the mask are rebuilt): kept draft nodes in ascending
  candidate index, then retrieved nodes.  depth = number of edges to the
  root, pos = ctx_len + depth, mask bit j of node i set iff j is i or an
  ancestor of i.
"""
from __future__ import annotations

import numpy as np

from . import OracleError

SRC_ROOT, SRC_DRAFT, SRC_RETRIEVED, SRC_REPLACED = 0, 1, 2, 3
MAX_NODES = 64


def select_draft(score: np.ndarray, budget: int) -> list[int]:
    """Candidate indices kept: 0 plus the budget-1 best of the rest by
    (score descending, index ascending), returned in ascending order."""
    C = len(score)
    if C < 1 or budget < 1:
        raise OracleError("empty candidate set or budget")
    rest = sorted(range(1, C), key=lambda c: score_rank_key(score[c], c))
    return sorted([0] + rest[: budget - 1])


def score_rank_key(s, c: int):
    """Sort key of candidate c with score s: score descending, index
    ascending; a NaN score ranks below every number (the scores are products
    of probabilities, so NaN is not a valid score; its place is fixed so that
    a NaN never displaces a real candidate).  -0 and +0 tie."""
    s = float(s)
    return (1, 0.0, c) if s != s else (0, -s, c)


def candidate_depths(cand_parent) -> list[int]:
    """Depth of every candidate (parents precede their children)."""
    dep = []
    for c in range(len(cand_parent)):
        p = int(cand_parent[c])
        dep.append(0 if c == 0 else dep[p] + 1)
    return dep


def retrieval_anchor(cand_parent, cand_score, budget: int, depth_c: int) -> int:
    """Candidate under which the retrieved nodes of a tree pruned at
    checkpoint depth depth_c hang: the best candidate (score descending,
    index ascending) of depth min(depth_c, deepest candidate depth), or, if
    the budget does not keep it, its deepest kept ancestor."""
    C = len(cand_parent)
    for c in range(1, C):
        if not (0 <= int(cand_parent[c]) < c):
            raise OracleError("candidate parent must precede its child")
    if depth_c < 0:
        raise OracleError("checkpoint depth must be >= 0")
    dep = candidate_depths(cand_parent)
    c_eff = min(depth_c, max(dep))
    if c_eff == 0:
        return 0
    best = min((c for c in range(1, C) if dep[c] == c_eff), key=lambda c: score_rank_key(cand_score[c], c))
    kept = set(select_draft(cand_score, budget))
    v = best
    while v not in kept:
        v = int(cand_parent[v])
    return v


def ancestors_or_self(parent: list[int], i: int) -> list[int]:
    out = []
    j = i
    while j >= 0:
        out.append(j)
        j = parent[j]
    return out


def build_one(cand_parent, cand_token, cand_score, budget, ret_token, ret_parent,
              ctx_len: int, V: int, static_replace: bool = False, table=None,
              replace_thresh: float = 0.0, anchor: int = 0):
    """One request.  Retrieved nodes with template parent -1 hang under
    candidate `anchor` (0 = the root), which must be kept.  Returns dict of
    python lists: parent, token, depth, pos, mask (python int), src, score
    (draft score or None), cand (candidate index or -1)."""
    C = len(cand_parent)
    if C < 1 or int(cand_parent[0]) != -1:
        raise OracleError("candidate 0 must be the root")
    for c in range(1, C):
        if not (0 <= int(cand_parent[c]) < c):
            raise OracleError("candidate parent must precede its child")
    for c in range(C):
        if not (0 <= int(cand_token[c]) < V):
            raise OracleError("candidate token outside the vocabulary")
    kept = select_draft(cand_score, int(budget))
    newidx = {c: i for i, c in enumerate(kept)}
    parent, token, src, score, cand = [], [], [], [], []
    for c in kept:
        if c == 0:
            parent.append(-1)
            src.append(SRC_ROOT)
        else:
            pc = int(cand_parent[c])
            if pc not in newidx:
                raise OracleError("selection is not ancestor-closed")
            parent.append(newidx[pc])
            src.append(SRC_DRAFT)
        token.append(int(cand_token[c]))
        score.append(float(cand_score[c]))
        cand.append(c)
    nd = len(kept)
    if anchor not in newidx:
        raise OracleError("the retrieval anchor is not a kept candidate")
    R = len(ret_token)
    for r in range(R):
        tp = int(ret_parent[r])
        if tp >= r:
            raise OracleError("template parent must precede its child")
        if not (0 <= int(ret_token[r]) < V):
            raise OracleError("retrieved token outside the vocabulary")
        parent.append(newidx[anchor] if tp < 0 else nd + tp)
        token.append(int(ret_token[r]))
        src.append(SRC_RETRIEVED)
        score.append(None)
        cand.append(-1)
    n = len(parent)
    if n > MAX_NODES:
        raise OracleError("tree larger than 64 nodes")

    if static_replace:
        k = table.shape[1]
        low_rank: dict[int, int] = {}
        for i in range(1, n):
            if src[i] != SRC_DRAFT or not (score[i] < replace_thresh):
                continue
            p = parent[i]
            j = low_rank.get(p, 0)
            low_rank[p] = j + 1
            if j < k:
                t = int(table[token[p], j])
                if not (0 <= t < V):
                    raise OracleError("table entry outside the vocabulary")
                token[i] = t
                src[i] = SRC_REPLACED

    depth, mask = [], []
    for i in range(n):
        anc = ancestors_or_self(parent, i)
        depth.append(len(anc) - 1)
        m = 0
        for j in anc:
            m |= 1 << j
        mask.append(m)
    pos = [ctx_len + dd for dd in depth]
    return dict(parent=parent, token=token, depth=depth, pos=pos, mask=mask,
                src=src, score=score, cand=cand, n=n)


def build_batch(cand_parent, cand_token, cand_score, cand_off, budget,
                ret_token, ret_parent, ret_off, ctx_len, V, row_off,
                static_replace=False, table=None, replace_thresh=0.0, anchor=None):
    """All requests, written in the padded row layout: request b's node i
    sits at row row_off[b] + i.  Rows past n[b] hold parent=token=depth=
    pos=-1, mask=0, src=-1.  anchor[b]: request b's retrieval anchor
    (candidate index; None = every request's root)."""
    B = len(budget)
    rows = int(row_off[B])
    out = dict(parent=np.full(rows, -1, np.int32), token=np.full(rows, -1, np.int32),
               depth=np.full(rows, -1, np.int32), pos=np.full(rows, -1, np.int32),
               mask=np.zeros(rows, np.uint64), src=np.full(rows, -1, np.int8),
               n=np.zeros(B, np.int32))
    trees = []
    for b in range(B):
        c0, c1 = int(cand_off[b]), int(cand_off[b + 1])
        r0, r1 = int(ret_off[b]), int(ret_off[b + 1])
        t = build_one(cand_parent[c0:c1], cand_token[c0:c1], cand_score[c0:c1],
                      int(budget[b]), ret_token[r0:r1], ret_parent[r0:r1],
                      int(ctx_len[b]), V, static_replace, table, replace_thresh,
                      0 if anchor is None else int(anchor[b]))
        cap = int(row_off[b + 1]) - int(row_off[b])
        if t["n"] > cap:
            raise OracleError("tree larger than the request's row capacity")
        o = int(row_off[b])
        n = t["n"]
        out["parent"][o:o + n] = t["parent"]
        out["token"][o:o + n] = t["token"]
        out["depth"][o:o + n] = t["depth"]
        out["pos"][o:o + n] = t["pos"]
        out["mask"][o:o + n] = np.array(t["mask"], dtype=np.uint64)
        out["src"][o:o + n] = t["src"]
        out["n"][b] = n
        trees.append(t)
    out["trees"] = trees
    return out
