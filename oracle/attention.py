"""Tree-masked GQA attention (oracle; test infrastructure only).

The flattened tree is verified in one parallel pass of the target model
using the rebuilt tree mask (Graft page, section 2, third step; TreeGraft
page, section 3 and section 7 item 1: tree attention lets one forward pass
verify the whole tree).  Query row (node i, head h) attends to every cached
context key 0 .. ctx-1 and to the tree key of every node j that is i or an
ancestor of i (bit j of mask[i]); tree node j's key/value sit at cache slot
ctx + j.  Grouped-query attention: head h reads key/value head h // (Hq/Hkv).

    o = sum_j softmax_j(scale * q . k_j) v_j     over the visible keys j

computed in fp64 as a two-pass softmax (max, then exp-sum) over the visible
keys in key order; bf16 inputs are upcast exactly.
"""
from __future__ import annotations

import numpy as np


def visible_keys(ctx: int, mask: int, n: int) -> np.ndarray:
    tree = [ctx + j for j in range(n) if (mask >> j) & 1]
    return np.concatenate([np.arange(ctx, dtype=np.int64), np.array(tree, dtype=np.int64)])


def attend_node(q: np.ndarray, K: np.ndarray, Vv: np.ndarray, ctx: int, mask: int, n: int,
                scale: float):
    """q: [Hq, d] fp64; K, Vv: [Hkv, >= ctx + n, d] fp64 for this request.
    Returns (o [Hq, d] fp64, lse [Hq] fp64, natural log)."""
    Hq = q.shape[0]
    Hkv = K.shape[0]
    G = Hq // Hkv
    keys = visible_keys(ctx, mask, n)
    o = np.empty_like(q)
    lse = np.empty(Hq)
    for h in range(Hq):
        kv = h // G
        s = (K[kv, keys] @ q[h]) * scale
        m = np.max(s)
        p = np.exp(s - m)
        z = np.sum(p)
        o[h] = (p @ Vv[kv, keys]) / z
        lse[h] = m + np.log(z)
    return o, lse


def tree_attention(q: np.ndarray, K_list, V_list, ctx_len, n, row_off, mask, scale: float,
                   nodes=None):
    """q: [rows, Hq, d] fp64 (padded row layout); K_list[b], V_list[b]:
    [Hkv, >= ctx_b + n_b, d] fp64.  `nodes` optionally restricts the work to
    a list of (b, i).  Returns dict {(b, i): (o, lse)}."""
    out = {}
    if nodes is None:
        nodes = [(b, i) for b in range(len(n)) for i in range(int(n[b]))]
    for b, i in nodes:
        r = int(row_off[b]) + i
        out[(b, i)] = attend_node(q[r], K_list[b], V_list[b], int(ctx_len[b]),
                                  int(mask[r]), int(n[b]), scale)
    return out
