"""Sampling acceptance at temperature T > 0 (oracle; test infrastructure only).

Verification by rejection sampling keeps the target model's output
distribution unchanged (TreeGraft page, section 3 and its reading list,
item 1); the pages evaluate at T = 1 as well as T = 0 (Graft page, section
5).  They give no rule for a node with several children.  The plainest
lossless reading for a draft tree whose tokens are chosen, not sampled:

    at every node u draw y_u from the target's distribution softmax(l_u / T);
    the accepted path starts at the root and moves to the lowest-index child
    whose token is y_u; it stops at the first node where no child matches,
    and that node's draw is the bonus token.

Every emitted token is then distributed exactly as in sampling the target
one token at a time: the first is y_root ~ p_root whether or not it matches
a child, and after a match the next is drawn at that child, whose row is the
target's distribution after the matched prefix.  Later siblings with the
same token never count (choosing among duplicate subtrees by their outcomes
would bias the output).  As T -> 0 the draw is the argmax and the rule is
the greedy one (oracle.accept) on trees without duplicate siblings.

Draws use the Gumbel-max identity, y = argmax_t (l_t / T + g_t) with g_t
i.i.d. Gumbel(0, 1), the noise passed in as an input.  The perturbed score
is two fp32 operations, each rounded: s_t = fl(fl(l_t * fl(1/T)) + g_t);
ties go to the lower token id.  The ranking is taken in fp32 because the
GPU takes it in fp32.
"""
from __future__ import annotations

import numpy as np

from . import OracleError


def perturbed_scores(logits, temperature: float, gumbel) -> np.ndarray:
    """fl(fl(l * fl(1/T)) + g) in fp32."""
    if not temperature > 0:
        raise OracleError("temperature must be positive")
    inv = np.float32(1.0) / np.float32(temperature)
    x = np.asarray(logits, np.float32)
    g = np.asarray(gumbel, np.float32)
    return (x * inv).astype(np.float32) + g


def sample_rows(logits, temperature: float, gumbel) -> np.ndarray:
    """Per row: the index of the largest perturbed score, ties to the lowest
    index (NaN ranks below every number)."""
    s = perturbed_scores(logits, temperature, gumbel)
    s = np.where(np.isnan(s), -np.inf, s)
    out = np.empty(s.shape[0], np.int32)
    for r in range(s.shape[0]):
        out[r] = int(np.argmax(s[r]))  # numpy returns the first maximum
    return out


def accept_sampled_one(parent, token, sample):
    """sample[i]: the token drawn at node i.  Returns (a, path, bonus)."""
    n = len(parent)
    if n < 1 or int(parent[0]) != -1:
        raise OracleError("node 0 must be the root")
    for i in range(1, n):
        if not (0 <= int(parent[i]) < i):
            raise OracleError("parent must precede its child")
    path = [0]
    u = 0
    while True:
        nxt = -1
        for c in range(u + 1, n):  # children of u in index order
            if int(parent[c]) == u and int(token[c]) == int(sample[u]):
                nxt = c
                break
        if nxt < 0:
            return len(path) - 1, path, int(sample[u])
        path.append(nxt)
        u = nxt


def accept_sampled_batch(n, row_off, parent, token, sample):
    """Padded row layout; parents request-local.  Returns (acc_len [B],
    paths, bonus [B])."""
    lens, paths, bonus = [], [], []
    for b in range(len(n)):
        o = int(row_off[b])
        nb = int(n[b])
        a, p, x = accept_sampled_one(parent[o:o + nb], token[o:o + nb], sample[o:o + nb])
        lens.append(a)
        paths.append(p)
        bonus.append(x)
    return lens, paths, bonus
