"""The attention check discriminates at long context (CPU only).

The GPU attention tests compare each output row with the oracle through
tests/_attn_check.py.  Here, on the CPU alone, that check is shown to
  * accept what a correct split-K kernel returns: an emulation of one that
    rounds the softmax weights to bf16 before P.V, merges fp32 partials by
    their maxima and rounds the output to bf16;
  * reject outputs that are plausibly wrong: scaled by 0.95 or 1.05, zero,
    one key split dropped from the merge, splits merged without their max
    rescaling, the neighbouring KV head's values;
at 32K keys with the O(1)-output regime (synth/regimes.py) and at 64K keys
with plain N(0, 1) inputs, where the elementwise bound alone accepts a
scaled output.  The wrong outputs are made from the oracle's own output or
from the emulation; no kernel is involved.
"""
import numpy as np
import pytest

from oracle import attention as OA
from oracle import lmhead as OL
from oracle import tree as OTree
from synth import f32_to_bf16_bits
from synth import regimes

from _attn_check import ROW_REL, check_output, row_errors

D = 128
SPLIT = 1024


def _case(ctx, n, Hq, Hkv, seed, concentrated):
    r = np.random.default_rng(seed)
    cap = ctx + n
    q = f32_to_bf16_bits(r.standard_normal((n, Hq, D)).astype(np.float32))
    k = f32_to_bf16_bits(r.standard_normal((1, Hkv, cap, D)).astype(np.float32))
    v = f32_to_bf16_bits(r.standard_normal((1, Hkv, cap, D)).astype(np.float32))
    if concentrated:
        q, k, _ = regimes.concentrate(900 + seed, q, k, [ctx], [0, n], Hkv)
    par = [-1] + [int(r.integers(0, i)) for i in range(1, n)]
    mask = np.zeros(n, np.uint64)
    for i in range(n):
        m = 0
        for j in OTree.ancestors_or_self(par, i):
            m |= 1 << j
        mask[i] = m
    qf = OL.bf16_to_f64(q).reshape(q.shape)
    K = OL.bf16_to_f64(k[0]).reshape(Hkv, cap, D)
    V = OL.bf16_to_f64(v[0]).reshape(Hkv, cap, D)
    return qf, K, V, mask


def _bf16_round(x):
    from synth import bf16_bits_to_f32
    return bf16_bits_to_f32(f32_to_bf16_bits(np.asarray(x, np.float32))).astype(np.float64)


def _split_kernel(qf, K, V, ctx, mask, n, scale, mutate=None, kv_shift=0):
    """Emulates a split-K kernel's arithmetic per (row, head): fp32 scores,
    per-split max and exp-sum, weights rounded to bf16 for P.V, partials
    merged by their maxima, output rounded to bf16.  `mutate` plants one
    mistake in the merge; kv_shift reads the values of another KV head."""
    Hq = qf.shape[1]
    Hkv = K.shape[0]
    G = Hq // Hkv
    out = np.empty((n, Hq, D))
    for i in range(n):
        keys = OA.visible_keys(ctx, int(mask[i]), n)
        splits = [keys[(keys >= s) & (keys < s + SPLIT)] for s in range(0, ctx + n, SPLIT)]
        splits = [s for s in splits if len(s)]
        for h in range(Hq):
            kv = h // G
            parts = []
            for sk in splits:
                x = (K[kv, sk] @ qf[i, h]).astype(np.float32).astype(np.float64) * scale
                m = x.max()
                p = np.exp(x - m).astype(np.float32).astype(np.float64)
                l = p.sum()
                o = _bf16_round(p) @ V[(kv + kv_shift) % Hkv, sk]
                parts.append((m, l, o))
            if mutate == "drop_heaviest":
                w = [l * np.exp(m) for m, l, _ in parts]
                parts.pop(int(np.argmax(w)))
            M = max(m for m, _, _ in parts)
            if mutate == "no_rescale":
                num = sum(o for _, _, o in parts)
                den = sum(l for _, l, _ in parts)
            else:
                num = sum(np.exp(m - M) * o for m, _, o in parts)
                den = sum(np.exp(m - M) * l for m, l, _ in parts)
            out[i, h] = _bf16_round(num / den)
    return out


def _oracle(qf, K, V, ctx, mask, n, scale):
    ref = OA.tree_attention(qf, [K], [V], [ctx], [n], [0, n], mask, scale)
    return np.stack([ref[(0, i)][0] for i in range(n)])


@pytest.fixture(scope="module")
def concentrated_32k():
    ctx, n, Hq, Hkv = 32768, 6, 4, 2
    qf, K, V, mask = _case(ctx, n, Hq, Hkv, seed=3, concentrated=True)
    scale = 1 / np.sqrt(D)
    ref = _oracle(qf, K, V, ctx, mask, n, scale)
    return qf, K, V, mask, ctx, n, scale, ref


def test_regime_outputs_are_order_one(concentrated_32k):
    *_, ref = concentrated_32k
    mags = np.abs(ref).max(axis=-1)
    assert np.median(mags) > 0.3, np.median(mags)
    # and the plain regime's are not: the reason for the regime
    qf, K, V, mask = _case(32768, 2, 2, 1, seed=4, concentrated=False)
    plain = _oracle(qf, K, V, 32768, mask, 2, 1 / np.sqrt(D))
    assert np.abs(plain).max() < 0.08


def test_correct_split_kernel_passes(concentrated_32k):
    qf, K, V, mask, ctx, n, scale, ref = concentrated_32k
    got = _split_kernel(qf, K, V, ctx, mask, n, scale)
    elem_ok, row_ok, _, ratio = row_errors(got, ref)
    assert elem_ok and row_ok, ratio
    assert ratio < ROW_REL / 2, ratio  # the bound keeps a margin over the roundings


@pytest.mark.parametrize("mistake", ["scale_0.95", "scale_1.05", "zeros", "drop_heaviest", "no_rescale",
                                     "other_kv_head"])
def test_plausible_mistakes_are_rejected(concentrated_32k, mistake):
    qf, K, V, mask, ctx, n, scale, ref = concentrated_32k
    if mistake == "scale_0.95":
        bad = _bf16_round(0.95 * ref)
    elif mistake == "scale_1.05":
        bad = _bf16_round(1.05 * ref)
    elif mistake == "zeros":
        bad = np.zeros_like(ref)
    elif mistake == "other_kv_head":
        bad = _split_kernel(qf, K, V, ctx, mask, n, scale, kv_shift=1)
    else:
        bad = _split_kernel(qf, K, V, ctx, mask, n, scale, mutate=mistake)
    # every row is wrong in the first three; at least one in the others
    per_row = [check_output(bad[i], ref[i]) for i in range(n)]
    assert not all(per_row)
    if mistake in ("scale_0.95", "scale_1.05", "zeros"):
        assert not any(per_row)


def test_plain_inputs_at_64k_keys():
    """N(0, 1) inputs at 64K keys: the elementwise bound alone accepts a
    0.95-scaled output; the row-scaled bound rejects it and accepts the
    emulated kernel."""
    ctx, n = 65536, 3
    qf, K, V, mask = _case(ctx, n, 2, 1, seed=5, concentrated=False)
    scale = 1 / np.sqrt(D)
    ref = _oracle(qf, K, V, ctx, mask, n, scale)
    bad = _bf16_round(0.95 * ref)
    elem_ok, row_ok, _, _ = row_errors(bad, ref)
    assert elem_ok and not row_ok
    got = _split_kernel(qf, K, V, ctx, mask, n, scale)
    elem_ok, row_ok, _, ratio = row_errors(got, ref)
    assert elem_ok and row_ok, ratio
