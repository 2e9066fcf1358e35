"""KV compaction and round chaining (oracle; test infrastructure only).

The flattened tree is verified in one pass and only the accepted output is
kept; the next round drafts from the bonus token (Graft page, section 2,
third step).  The tree's keys and values sit at cache slots ctx .. ctx+n-1
in flattened order, the root (the previous round's bonus token) first.  The
plainest reading of "keep the accepted output": after a round the cache
holds, after the ctx context tokens, the accepted path root, p1, .., pa in
order, exactly what decoding those tokens one at a time would have written:

    slot ctx + t  <-  slot ctx + path[t]      for t = 0 .. a   (every layer,
                                                               KV head, K and V)
    ctx'  = ctx + a + 1                       (the root and a accepted drafts)
    root' = bonus

Rows are read from the cache as it was before the round's compaction; slots
past ctx + a are left as they are.
"""
from __future__ import annotations

import numpy as np

from . import OracleError


def compact_one(cache: np.ndarray, ctx: int, n: int, a: int, path) -> np.ndarray:
    """cache: [..., cap, d] rows of one request (any leading axes: layers,
    KV heads).  Returns the compacted copy."""
    cap = cache.shape[-2]
    if not 0 <= a <= 63:
        raise OracleError("accepted length outside [0, 63]")
    p = [int(x) for x in path[: a + 1]]
    if len(p) != a + 1 or p[0] != 0:
        raise OracleError("accepted path must start at the root")
    if any(p[t] <= p[t - 1] for t in range(1, a + 1)) or p[-1] >= n:
        raise OracleError("accepted path must climb through the tree's nodes")
    if ctx < 0 or ctx + n > cap:
        raise OracleError("tree does not fit the cache")
    out = cache.copy()
    for t in range(a + 1):
        out[..., ctx + t, :] = cache[..., ctx + p[t], :]
    return out


def compact_batch(kcache: np.ndarray, vcache: np.ndarray, ctx_len, n, acc_len, acc_path, bonus):
    """kcache, vcache: [layers, B, Hkv, cap, d]; acc_path: [B][>= a+1] node
    indices (root first).  Returns (kcache', vcache', ctx_next, root_next)."""
    k2, v2 = kcache.copy(), vcache.copy()
    B = len(ctx_len)
    ctx_next = np.zeros(B, np.int32)
    root_next = np.zeros(B, np.int32)
    for b in range(B):
        c, nb, a = int(ctx_len[b]), int(n[b]), int(acc_len[b])
        k2[:, b] = compact_one(kcache[:, b], c, nb, a, acc_path[b])
        v2[:, b] = compact_one(vcache[:, b], c, nb, a, acc_path[b])
        ctx_next[b] = c + a + 1
        root_next[b] = int(bonus[b])
    return k2, v2, ctx_next, root_next
