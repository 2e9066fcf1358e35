"""Successor table (oracle; test infrastructure only).

The table is a dense [V, k] int32 array kept in GPU memory: row t holds the
k successors of token t the target model ranked highest (Graft page,
section 2, second step, the "adjacency matrix").

* Update (Graft page, section 2, third step, and section 6, second level):
  after verification every verified position -- accepted or rejected --
  rewrites the row of its token with the target model's most likely
  successors at that position.  Reading: the whole row is overwritten with
  that position's top-k ids; when several positions carry the same token the
  one latest in (request, node) order wins.
* Retrieval (Graft page, section 2, second step): starting at the current
  token, the template is expanded by row lookups: template node t takes
  table[token of its template parent (the root token for -1)][rank_t].
"""
from __future__ import annotations

import numpy as np

from . import OracleError


def update(table: np.ndarray, n, row_off, token, topk) -> np.ndarray:
    """Returns an updated copy.  Node i of request b is row row_off[b] + i,
    for i < n[b]; rows are applied in (request, node) order."""
    V, k = table.shape
    out = table.copy()
    for b in range(len(n)):
        for i in range(int(n[b])):
            r = int(row_off[b]) + i
            t = int(token[r])
            row = np.asarray(topk[r][:k], dtype=np.int64)
            if not (0 <= t < V) or np.any(row < 0) or np.any(row >= V):
                raise OracleError("update token or successor id outside the vocabulary")
            out[t] = row
    return out


def retrieve(table: np.ndarray, root_token: int, tparent, trank) -> list[int]:
    V, k = table.shape
    if not (0 <= root_token < V):
        raise OracleError("root token outside the vocabulary")
    tok: list[int] = []
    for t in range(len(tparent)):
        p = int(tparent[t])
        if p >= t:
            raise OracleError("template parent must precede its child")
        src = root_token if p < 0 else tok[p]
        r = int(trank[t])
        if not (0 <= r < k):
            raise OracleError("template rank outside the table width")
        v = int(table[src, r])
        if not (0 <= v < V):
            raise OracleError("table entry outside the vocabulary")
        tok.append(v)
    return tok
