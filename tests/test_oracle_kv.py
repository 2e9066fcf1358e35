"""Pins of the KV compaction oracle (oracle/kv.py) against what sequential
decoding would write, without using its formula: a stand-in model writes
each tree node's K/V row as a function of its token and its tree position
ctx + depth; decoding the accepted tokens one by one would write the same
function at slots ctx, ctx+1, ...  So after compaction (and over chained
rounds) the cache must read as the accepted tokens in order."""
import numpy as np
import pytest

from oracle import OracleError
from oracle import accept as OAcc
from oracle import kv as OKV

D = 8


def row(token, pos, layer, head, which):
    """Stand-in K/V row for `token` written at cache position `pos`."""
    base = np.array([token, pos, layer, head, which, token ^ pos, (token * 31 + pos) & 0xFFFF, 7], np.int64)
    return (base & 0xFFFF).astype(np.uint16)


def tree_rows(cache, b, ctx, parent, token, which):
    depth = [0] * len(parent)
    for i in range(1, len(parent)):
        depth[i] = depth[parent[i]] + 1
    L, _, H = cache.shape[:3]
    for i, t in enumerate(token):
        for l in range(L):
            for h in range(H):
                cache[l, b, h, ctx + i] = row(t, ctx + depth[i], l, h, which)


def random_tree(r, n, V):
    parent = [-1] + [int(r.integers(0, i)) for i in range(1, n)]
    token = [int(x) for x in r.integers(0, V, n)]
    return parent, token


def accepting_argmax(r, parent, token, V, keep):
    """argmax under which the nodes in `keep` (a root path) are accepted and
    their other children are not."""
    am = r.integers(0, V, len(parent))
    for i in keep[1:]:
        am[parent[i]] = token[i]
    return am


@pytest.mark.parametrize("seed", range(6))
def test_compaction_reads_like_sequential_decoding(seed):
    r = np.random.default_rng(seed)
    L, B, H, cap, V = 2, 3, 2, 120, 50
    kc = r.integers(0, 65536, (L, B, H, cap, D)).astype(np.uint16)
    vc = r.integers(0, 65536, (L, B, H, cap, D)).astype(np.uint16)
    ctx = [int(x) for x in r.integers(0, 40, B)]
    n, lens, paths, bonus, seqs = [], [], [], [], []
    for b in range(B):
        nb = int(r.integers(1, 64))
        parent, token = random_tree(r, nb, V)
        # a random deepest node's root path is made acceptable
        j = int(r.integers(0, nb))
        keep = []
        while j >= 0:
            keep.append(j)
            j = parent[j]
        keep.reverse()
        am = accepting_argmax(r, parent, token, V, keep)
        a, path, bo = OAcc.accept_one(parent, token, am)
        tree_rows(kc, b, ctx[b], parent, token, 0)
        tree_rows(vc, b, ctx[b], parent, token, 1)
        n.append(nb), lens.append(a), paths.append(path), bonus.append(bo)
        seqs.append([token[i] for i in path])
    before_k, before_v = kc.copy(), vc.copy()
    k2, v2, cn, rn = OKV.compact_batch(kc, vc, ctx, n, lens, paths, bonus)
    for b in range(B):
        a = lens[b]
        assert cn[b] == ctx[b] + a + 1 and rn[b] == bonus[b]
        for t, tok in enumerate(seqs[b]):
            for l in range(L):
                for h in range(H):
                    assert np.array_equal(k2[l, b, h, ctx[b] + t], row(tok, ctx[b] + t, l, h, 0))
                    assert np.array_equal(v2[l, b, h, ctx[b] + t], row(tok, ctx[b] + t, l, h, 1))
        # the context before the tree and the slots after the path stay
        assert np.array_equal(k2[:, b, :, :ctx[b]], before_k[:, b, :, :ctx[b]])
        assert np.array_equal(v2[:, b, :, ctx[b] + a + 1:], before_v[:, b, :, ctx[b] + a + 1:])


def test_root_only_acceptance_keeps_the_cache():
    r = np.random.default_rng(1)
    kc = r.integers(0, 65536, (1, 1, 2, 30, D)).astype(np.uint16)
    k2, v2, cn, rn = OKV.compact_batch(kc, kc, [5], [7], [0], [[0]], [42])
    assert np.array_equal(k2, kc) and np.array_equal(v2, kc)
    assert cn.tolist() == [6] and rn.tolist() == [42]


def test_chained_rounds_read_like_sequential_decoding():
    """Two rounds: the second tree sits after the first round's compacted
    path; the cache then holds both accepted sequences back to back."""
    r = np.random.default_rng(9)
    L, H, cap, V = 1, 2, 200, 40
    kc = np.zeros((L, 1, H, cap, D), np.uint16)
    vc = np.zeros_like(kc)
    ctx, decoded = 11, []
    for rnd in range(2):
        parent, token = random_tree(r, 30, V)
        keep = [0]
        for i in range(1, 30):  # follow the first child chain
            if parent[i] == keep[-1]:
                keep.append(i)
        am = accepting_argmax(r, parent, token, V, keep)
        a, path, bo = OAcc.accept_one(parent, token, am)
        tree_rows(kc, 0, ctx, parent, token, 0)
        tree_rows(vc, 0, ctx, parent, token, 1)
        kc, vc, cn, rn = OKV.compact_batch(kc, vc, [ctx], [30], [a], [path], [bo])
        decoded += [token[i] for i in path]
        ctx = int(cn[0])
    for s, tok in enumerate(decoded):
        for h in range(H):
            assert np.array_equal(kc[0, 0, h, 11 + s], row(tok, 11 + s, 0, h, 0))
    assert ctx == 11 + len(decoded)


@pytest.mark.parametrize("a,path,n,err", [
    (2, [1, 2, 3], 5, "root"),          # path does not start at the root
    (2, [0, 3, 2], 5, "climb"),         # not increasing
    (2, [0, 1, 5], 5, "climb"),         # node outside the tree
    (64, list(range(65)), 70, "63"),    # longer than a tree can be
])
def test_malformed_paths_are_rejected(a, path, n, err):
    kc = np.zeros((1, 1, 1, 100, D), np.uint16)
    with pytest.raises(OracleError, match=err):
        OKV.compact_batch(kc, kc, [3], [n], [a], [path], [0])


def test_tree_past_the_cache_is_rejected():
    kc = np.zeros((1, 1, 1, 20, D), np.uint16)
    with pytest.raises(OracleError, match="fit"):
        OKV.compact_batch(kc, kc, [15], [6], [1], [[0, 1]], [0])
