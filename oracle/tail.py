"""Graft-TAIL for block drafts (oracle; test infrastructure only).

Graft page, section 7 (an exploration on DFlash, whose diffusion drafter
writes a block of 16 tokens at once): the drafter's confidence correlates
with the target's acceptance, so the confident prefix of the block is kept
and its low-confidence tail is replaced by retrieval candidates from the
successor table, the verification budget staying the same.  The page gives
no thresholds or shapes; the plainest reading:

    K  = length of the longest prefix of the block whose confidences are all
         >= tau (the cut is at the first token below tau)
    kept: the root and block tokens 1..K, a chain
    tail: the R = L - K freed slots (budget 1 + L unchanged) hold the first R
          nodes of the retrieval template, expanded from the successor table
          at the deepest kept node -- the root when K = 0 -- and hung under it
          (the retrieval root at the deepest kept node rather than the tree
          root, since the kept prefix is a single path)

Because the template's first R nodes are the template of size R (its nodes
are generated best first), expanding the size-L template once and keeping a
prefix serves every K.  Flattened order: root, kept block tokens, retrieved
nodes in template order; depth, positions and mask as for every tree
(oracle.tree).
"""
from __future__ import annotations

import numpy as np

from . import OracleError
from .tree import MAX_NODES, SRC_DRAFT, SRC_RETRIEVED, SRC_ROOT, ancestors_or_self


def keep_length(conf, tau: float) -> int:
    """K: how many leading block tokens have confidence >= tau (fp32 compare;
    NaN counts as low)."""
    t = np.float32(tau)
    for i, c in enumerate(conf):
        if not (np.float32(c) >= t):
            return i
    return len(conf)


def retrieval_root(root_token: int, block_token, conf, tau: float) -> int:
    """Token of the deepest kept node: the root when K = 0."""
    K = keep_length(conf, tau)
    return int(root_token) if K == 0 else int(block_token[K - 1])


def build_one(root_token: int, block_token, conf, tau: float, ret_token, ret_parent, ctx_len: int, V: int):
    """One request.  ret_token / ret_parent: the size-L template expanded
    from retrieval_root(...) (oracle.table.retrieve).  Returns the tree as
    oracle.tree.build_one does (parent, token, depth, pos, mask, src, n)."""
    L = len(block_token)
    if len(conf) != L or len(ret_token) < L or len(ret_parent) < L:
        raise OracleError("block, confidences and template must cover L positions")
    if 1 + L > MAX_NODES:
        raise OracleError("tree larger than 64 nodes")
    for t in [root_token, *block_token]:
        if not (0 <= int(t) < V):
            raise OracleError("token outside the vocabulary")
    K = keep_length(conf, tau)
    parent = [-1] + list(range(K))
    token = [int(root_token)] + [int(t) for t in block_token[:K]]
    src = [SRC_ROOT] + [SRC_DRAFT] * K
    for r in range(L - K):
        tp = int(ret_parent[r])
        if tp >= r:
            raise OracleError("template parent must precede its child")
        if not (0 <= int(ret_token[r]) < V):
            raise OracleError("retrieved token outside the vocabulary")
        parent.append(K if tp < 0 else K + 1 + tp)
        token.append(int(ret_token[r]))
        src.append(SRC_RETRIEVED)
    n = len(parent)
    depth, mask = [], []
    for i in range(n):
        anc = ancestors_or_self(parent, i)
        depth.append(len(anc) - 1)
        m = 0
        for j in anc:
            m |= 1 << j
        mask.append(m)
    return dict(parent=parent, token=token, depth=depth, pos=[ctx_len + d for d in depth], mask=mask, src=src, n=n,
                keep=K)


def build_batch(root_token, block_token, conf, tau, ret_token, ret_parent, ret_off, ctx_len, V, row_off):
    """All requests in the padded row layout (rows past n: -1 / 0), with
    block_token / conf [B, L] and the per-request size-L template expansions
    at ret_off."""
    B = len(root_token)
    rows = int(row_off[B])
    out = dict(parent=np.full(rows, -1, np.int32), token=np.full(rows, -1, np.int32),
               depth=np.full(rows, -1, np.int32), pos=np.full(rows, -1, np.int32),
               mask=np.zeros(rows, np.uint64), src=np.full(rows, -1, np.int8), n=np.zeros(B, np.int32),
               keep=np.zeros(B, np.int32))
    for b in range(B):
        o0, o1 = int(ret_off[b]), int(ret_off[b + 1])
        t = build_one(int(root_token[b]), block_token[b], conf[b], tau, ret_token[o0:o1], ret_parent[o0:o1],
                      int(ctx_len[b]), V)
        r0 = int(row_off[b])
        if t["n"] > int(row_off[b + 1]) - r0:
            raise OracleError("tree larger than its rows")
        for key in ("parent", "token", "depth", "pos", "src"):
            out[key][r0:r0 + t["n"]] = t[key]
        out["mask"][r0:r0 + t["n"]] = np.array(t["mask"], dtype=np.uint64)
        out["n"][b] = t["n"]
        out["keep"][b] = t["keep"]
    return out
