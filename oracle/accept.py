"""Greedy acceptance on a verified tree (oracle; test infrastructure only).

Draft and retrieved nodes face the same verification rule, which keeps the
output identical to the target model decoding alone (Graft page, section 2,
third step).  At temperature 0 (TreeGraft page, section 5) the rule is
greedy: a node is accepted when its token is the target's most likely token
at its parent and its parent is accepted; the round keeps the deepest
accepted root path, stopping at the first rejection (TreeGraft page,
section 1).

    A = {root} U {i : token[i] == argmax[parent[i]] and parent[i] in A}
    best = the deepest node of A, ties to the lowest index
    accepted length a = depth(best)  (draft tokens accepted; the bonus token
                                      is not counted)
    path = root, ..., best            (node indices, root first)
    bonus = argmax[best]              (the target's own next token)
"""
from __future__ import annotations

from . import OracleError


def accept_one(parent, token, argmax):
    n = len(parent)
    if n < 1 or int(parent[0]) != -1:
        raise OracleError("node 0 must be the root")
    acc = [False] * n
    depth = [0] * n
    acc[0] = True
    for i in range(1, n):
        p = int(parent[i])
        if not (0 <= p < i):
            raise OracleError("parent must precede its child")
        depth[i] = depth[p] + 1
        acc[i] = acc[p] and int(token[i]) == int(argmax[p])
    best = 0
    for i in range(1, n):
        if acc[i] and depth[i] > depth[best]:
            best = i
    path = []
    j = best
    while j >= 0:
        path.append(j)
        j = int(parent[j])
    path.reverse()
    return depth[best], path, int(argmax[best])


def accept_batch(n, row_off, parent, token, argmax):
    """Padded row layout; parents are request-local indices.  Returns
    (acc_len [B], paths: list of lists, bonus [B])."""
    lens, paths, bonus = [], [], []
    for b in range(len(n)):
        o = int(row_off[b])
        nb = int(n[b])
        a, p, x = accept_one(parent[o:o + nb], token[o:o + nb], argmax[o:o + nb])
        lens.append(a)
        paths.append(p)
        bonus.append(x)
    return lens, paths, bonus
