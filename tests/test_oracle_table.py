"""Pins for the oracle's successor-table update and retrieval (CPU only)."""
import numpy as np
import pytest

from oracle import OracleError
from oracle import table as TB
from oracle.template import template


def _rand_rows(r, n, k, V):
    return np.stack([r.choice(V, size=k, replace=False) for _ in range(n)]).astype(np.int32)


@pytest.mark.parametrize("seed", range(5))
def test_update_rows_equal_last_fed_topk(seed):
    r = np.random.default_rng(seed)
    V, k, B, N = 300, 8, 3, 20
    table = _rand_rows(r, V, k, V)
    token = r.integers(0, 40, B * N).astype(np.int32)  # many repeats
    topk = _rand_rows(r, B * N, k, V)
    n = np.array([20, 13, 0], np.int32)
    row_off = np.array([0, 20, 40, 60], np.int32)
    out = TB.update(table, n, row_off, token, topk)
    # independent statement: for every token, the last verified row carrying it
    last = {}
    for b in range(B):
        for i in range(int(n[b])):
            last[int(token[row_off[b] + i])] = row_off[b] + i
    for t in range(V):
        if t in last:
            assert np.array_equal(out[t], topk[last[t]])
        else:
            assert np.array_equal(out[t], table[t])  # untouched rows unchanged
    # idempotent
    assert np.array_equal(TB.update(out, n, row_off, token, topk), out)


def test_update_last_writer_hand_example():
    table = np.zeros((10, 2), np.int32)
    token = np.array([3, 5, 3], np.int32)
    topk = np.array([[1, 2], [4, 6], [7, 8]], np.int32)
    out = TB.update(table, np.array([2, 1]), np.array([0, 2, 3]), token, topk)
    assert out[3].tolist() == [7, 8] and out[5].tolist() == [4, 6]
    assert out[0].tolist() == [0, 0]


def test_retrieve_closed_form_shift_table():
    # table[t][r] = (t + r + 1) mod V  =>  a rank path (r1..rd) from root x
    # lands on (x + sum(r_i + 1)) mod V
    V, k = 97, 8
    table = np.array([[(t + r + 1) % V for r in range(k)] for t in range(V)], np.int32)
    tp, tr, order = template(52, k, 8)
    for root in (0, 5, 96):
        tok = TB.retrieve(table, root, tp, tr)
        for t, p in enumerate(order):
            assert tok[t] == (root + sum(r + 1 for r in p)) % V


def test_retrieve_chain_follows_rank0():
    V, k = 50, 3
    r = np.random.default_rng(1)
    table = _rand_rows(r, V, k, V)
    tp = [-1, 0, 1, 2]
    tr = [0, 0, 0, 0]
    tok = TB.retrieve(table, 7, tp, tr)
    x = 7
    for t in range(4):
        x = int(table[x, 0])
        assert tok[t] == x


def test_errors():
    table = np.zeros((10, 2), np.int32)
    with pytest.raises(OracleError):
        TB.update(table, [1], [0, 1], np.array([10]), np.array([[0, 1]]))
    with pytest.raises(OracleError):
        TB.update(table, [1], [0, 1], np.array([1]), np.array([[0, 10]]))
    bad = table.copy()
    bad[0, 0] = 11
    with pytest.raises(OracleError):
        TB.retrieve(bad, 0, [-1], [0])
    with pytest.raises(OracleError):
        TB.retrieve(table, 10, [-1], [0])
