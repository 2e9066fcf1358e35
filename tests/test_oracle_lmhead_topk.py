"""Pins for the oracle's lm-head and top-k (CPU only)."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import lmhead as LM
from oracle import topk as TK
from synth import bf16_bits_to_f32, f32_to_bf16_bits
from synth import workloads as W


def test_bf16_roundtrip_and_rne():
    x = np.array([1.0, 1.00390625, 1.005859375, -2.5, 0.0, -0.0, 3.0e38], np.float32)
    b = f32_to_bf16_bits(x)
    # 1 + 2^-8 is a tie between 1 and 1+2^-7: even mantissa (1.0) wins;
    # 1 + 1.5*2^-8 rounds up to 1 + 2^-7
    assert bf16_bits_to_f32(b).tolist()[:4] == [1.0, 1.0, 1.0078125, -2.5]
    assert b[5] == 0x8000


def test_lmhead_brute_force_exact_rationals():
    r = np.random.default_rng(0)
    M, H, V = 3, 16, 5
    h = f32_to_bf16_bits(r.standard_normal((M, H)).astype(np.float32))
    w = f32_to_bf16_bits((0.02 * r.standard_normal((V, H))).astype(np.float32))
    out = LM.logits(h, w)
    hf = bf16_bits_to_f32(h)
    wf = bf16_bits_to_f32(w)
    for m in range(M):
        for v in range(V):
            exact = sum(Fraction(float(hf[m, j])) * Fraction(float(wf[v, j])) for j in range(H))
            ref = np.float32(float(exact))
            # one rounding to fp32 of the exact sum (fp64 accumulation may
            # differ from exact rounding by at most one fp32 ulp)
            assert abs(out[m, v] - ref) <= np.spacing(np.abs(ref)) + 1e-30


def test_lmhead_one_hot_rows_pick_weight_columns():
    r = np.random.default_rng(1)
    H, V = 32, 7
    w = f32_to_bf16_bits(r.standard_normal((V, H)).astype(np.float32))
    h = np.zeros((H, H), np.float32)
    np.fill_diagonal(h, 1.0)
    out = LM.logits(f32_to_bf16_bits(h), w)
    assert np.array_equal(out, bf16_bits_to_f32(w).T)


def test_planted_peak_raises_logit_by_boost():
    wl = W.WORKLOADS[1]
    w = W.make_lm_weights(wl)
    parent = np.array([-1, 0, 0, 1], np.int32)
    token = np.array([3, 10, 20, 30], np.int32)
    hid, planted = W.plant_hidden(wl, lambda ids: w[ids], parent, token,
                                  np.array([4]), np.array([0, 4]), p_plant=1.0)
    lg = LM.logits(hid, w)
    z = W.rng(1, "hidden").standard_normal((4, wl.H), dtype=np.float32)
    base = LM.logits(f32_to_bf16_bits(z), w)
    for m in range(4):
        t = planted[m]
        assert t >= 0
        # +6 up to the bf16 rounding of the hidden state
        assert abs((lg[m, t] - base[m, t]) - 6.0) < 0.15
    # nodes with children plant one of their children's tokens
    assert planted[0] in (10, 20) and planted[1] == 30


def brute_topk(row, k):
    ids = list(range(len(row)))
    out = []
    for _ in range(k):
        best = None
        for i in ids:
            if best is None or row[i] > row[best] or (row[i] == row[best] and i < best):
                best = i
        out.append(best)
        ids.remove(best)
    return out


@pytest.mark.parametrize("seed", range(10))
def test_topk_brute_force(seed):
    r = np.random.default_rng(seed)
    V = 50
    x = r.integers(-5, 5, (6, V)).astype(np.float32)  # many ties
    x[0, 3] = -0.0
    x[0, 4] = 0.0
    k = 1 + seed % 10
    ids, vals = TK.topk(x, k)
    for m in range(6):
        b = brute_topk(x[m].tolist(), k)
        assert ids[m].tolist() == b
        assert vals[m].tolist() == [float(x[m, i]) for i in b]


def test_topk_special_cases():
    x = np.zeros((2, 20), np.float32)
    x[1, 0] = -0.0
    x[1, 1] = 0.0
    ids, _ = TK.topk(x, 5)
    assert ids[0].tolist() == [0, 1, 2, 3, 4]
    assert ids[1].tolist() == [0, 1, 2, 3, 4]  # -0 and +0 tie: lower id first
    y = np.random.default_rng(3).standard_normal((4, 1000)).astype(np.float32)
    y[2, 777] = 100.0
    ids, vals = TK.topk(y, 8)
    assert ids[2, 0] == 777 and vals[2, 0] == 100.0
    assert np.all(np.diff(vals, axis=1) <= 0)


def test_topk_nan_ranks_below_every_number():
    """A NaN logit ranks after every number, -inf included; NaNs tie with
    each other (lower id first).  Checked against the same order written out
    as repeated extraction of the best remaining entry."""
    r = np.random.default_rng(7)
    x = r.integers(-3, 3, (4, 23)).astype(np.float32)
    x[0, [0, 5, 9]] = np.nan
    x[1, :] = np.nan
    x[1, [4, 17]] = [-np.inf, 2.0]
    x[2, [3, 4]] = [np.inf, np.nan]
    for m in range(4):
        remaining = list(range(x.shape[1]))
        order = []
        while remaining:
            def beats(a, b):
                va, vb = x[m, a], x[m, b]
                if np.isnan(vb) and not np.isnan(va):
                    return True
                if np.isnan(va):
                    return np.isnan(vb) and a < b
                return va > vb or (va == vb and a < b)
            best = remaining[0]
            for c in remaining[1:]:
                if beats(c, best):
                    best = c
            order.append(best)
            remaining.remove(best)
        ids, vals = TK.topk(x[m:m + 1], 12)
        assert ids[0].tolist() == order[:12]
        assert np.array_equal(vals[0], x[m, order[:12]], equal_nan=True)
