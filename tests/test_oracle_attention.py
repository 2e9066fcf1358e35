"""Pins for the oracle's tree attention (CPU only).

Independent references: torch's scaled_dot_product_attention on the CPU in
fp64 (a library routine the oracle does not call), in the special cases
where tree attention reduces to ordinary attention."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention as A
from oracle import tree as T


def _setup(seed, ctx, n, Hq, Hkv, d):
    r = np.random.default_rng(seed)
    q = r.standard_normal((n, Hq, d))
    K = r.standard_normal((Hkv, ctx + n, d))
    V = r.standard_normal((Hkv, ctx + n, d))
    return q, K, V


def _sdpa(q, K, V, scale, causal):
    # q [Hq, Lq, d], K/V [Hq, Lk, d]
    return F.scaled_dot_product_attention(torch.from_numpy(q)[None], torch.from_numpy(K)[None],
                                          torch.from_numpy(V)[None], is_causal=causal,
                                          scale=scale)[0].numpy()


@pytest.mark.parametrize("Hq,Hkv,ctx,n", [(4, 2, 37, 9), (8, 8, 0, 5), (6, 2, 100, 16), (5, 1, 64, 64)])
def test_chain_tree_equals_causal_attention(Hq, Hkv, ctx, n):
    d = 16
    q, K, V = _setup(Hq * 100 + n, ctx, n, Hq, Hkv, d)
    scale = 1 / np.sqrt(d)
    mask = [(1 << (i + 1)) - 1 for i in range(n)]
    out = A.tree_attention(q, [K], [V], [ctx], [n], [0, n], mask, scale)
    # causal attention over the whole sequence: context queries are filler
    G = Hq // Hkv
    L = ctx + n
    qfull = np.random.default_rng(7).standard_normal((Hq, L, d))
    qfull[:, ctx:] = q.transpose(1, 0, 2)
    Kr = np.repeat(K, G, axis=0)
    Vr = np.repeat(V, G, axis=0)
    ref = _sdpa(qfull, Kr, Vr, scale, causal=True)
    for i in range(n):
        o, _ = out[(0, i)]
        np.testing.assert_allclose(o, ref[:, ctx + i], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(4))
def test_row_equals_attention_over_context_plus_root_path(seed):
    Hq, Hkv, d, ctx, n = 4, 2, 8, 23, 30
    q, K, V = _setup(seed, ctx, n, Hq, Hkv, d)
    r = np.random.default_rng(50 + seed)
    parent = [-1] + [int(r.integers(0, i)) for i in range(1, n)]
    mask = []
    for i in range(n):
        m = 0
        for j in T.ancestors_or_self(parent, i):
            m |= 1 << j
        mask.append(m)
    scale = 0.3
    out = A.tree_attention(q, [K], [V], [ctx], [n], [0, n], mask, scale)
    G = Hq // Hkv
    for i in range(n):
        path = T.ancestors_or_self(parent, i)[::-1]
        idx = list(range(ctx)) + [ctx + j for j in path]
        Kp = np.repeat(K[:, idx], G, axis=0)
        Vp = np.repeat(V[:, idx], G, axis=0)
        ref = _sdpa(q[i][:, None, :], Kp, Vp, scale, causal=False)[:, 0]
        np.testing.assert_allclose(out[(0, i)][0], ref, rtol=1e-12, atol=1e-12)
        # log-sum-exp against a direct evaluation
        s = np.einsum("hd,hkd->hk", q[i], Kp) * scale
        np.testing.assert_allclose(out[(0, i)][1], np.log(np.exp(s).sum(-1)), rtol=1e-12)


def test_non_ancestors_do_not_change_a_row():
    Hq, Hkv, d, ctx = 2, 1, 8, 10
    n = 12
    q, K, V = _setup(3, ctx, n, Hq, Hkv, d)
    parent = [-1, 0, 1, 2, 0, 4, 1, 6, 6, 3, 9, 0]
    mask = []
    for i in range(n):
        m = 0
        for j in T.ancestors_or_self(parent, i):
            m |= 1 << j
        mask.append(m)
    full = A.tree_attention(q, [K], [V], [ctx], [n], [0, n], mask, 0.25)
    # drop the trailing nodes 10, 11 (not ancestors of 0..9): rows 0..9 bit-identical
    K2, V2 = K[:, :ctx + 10], V[:, :ctx + 10]
    part = A.tree_attention(q[:10], [K2], [V2], [ctx], [10], [0, 10], mask[:10], 0.25)
    for i in range(10):
        assert np.array_equal(full[(0, i)][0], part[(0, i)][0])


def test_star_tree_rows_see_context_root_and_self():
    Hq, Hkv, d, ctx, n = 3, 3, 4, 5, 6
    q, K, V = _setup(11, ctx, n, Hq, Hkv, d)
    mask = [1] + [1 | (1 << i) for i in range(1, n)]
    out = A.tree_attention(q, [K], [V], [ctx], [n], [0, n], mask, 0.5)
    for i in range(1, n):
        idx = list(range(ctx)) + [ctx, ctx + i]
        ref = _sdpa(q[i][:, None, :], K[:, idx], V[:, idx], 0.5, causal=False)[:, 0]
        np.testing.assert_allclose(out[(0, i)][0], ref, rtol=1e-12, atol=1e-12)
