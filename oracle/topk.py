"""Per-row top-k and argmax over the vocabulary (oracle; test infrastructure
only).

Row t of the successor table holds the k successors the target model ranks
highest (Graft page, section 2, second step) and greedy acceptance compares
draft tokens with the target's most likely token (Graft page, section 2,
third step).  Both come from one per-row top-k of the fp32 logits.

Definition: sort the ids of a row by (value descending, id ascending) and
take the first k; argmax is the first.  Logits are ranked as given (fp32):
softmax is monotone, and ranking rounded probabilities could create ties the
logits do not have.  +0 and -0 compare equal (tie, lower id first).
"""
from __future__ import annotations

import numpy as np


def topk(logits: np.ndarray, k: int):
    """logits [M, V] fp32 -> (ids [M, k] int32, vals [M, k] fp32)."""
    x = np.asarray(logits, dtype=np.float32)
    M, V = x.shape
    if not (1 <= k <= V):
        raise ValueError("k outside [1, V]")
    ids = np.empty((M, k), np.int32)
    vals = np.empty((M, k), np.float32)
    for m in range(M):
        order = np.argsort(-x[m], kind="stable")[:k]
        ids[m] = order
        vals[m] = x[m, order]
    return ids, vals
