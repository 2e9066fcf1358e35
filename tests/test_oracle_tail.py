"""Pins of the Graft-TAIL oracle (oracle/tail.py): a hand-worked example,
the budget invariant, the two ends of the cut (K = 0 is a retrieval-only
Graft tree built by the separately pinned oracle.tree; K = L is the plain
chain), independence from confidences after the cut, the retrieved subtree's
shape, and the fp32 threshold compare."""
import numpy as np
import pytest

from oracle import OracleError
from oracle import table as OTab
from oracle import tail as OTail
from oracle import tree as OTree
from oracle.template import template


def test_hand_worked_example():
    # Graft page, section 7 (Graft-TAIL), read as in oracle/tail.py: block
    # 11 12 13 14 with confidences 0.9 0.8 0.3 0.95 and tau = 0.5 keeps 11 12
    # (the cut is at 13); the two freed slots take the template's first two
    # nodes (rank 0 under the retrieval root, then rank 0 under that node),
    # expanded from 12: table[12][0] = 20, table[20][0] = 30.
    V, k = 40, 2
    table = np.zeros((V, k), np.int32)
    table[12] = [20, 21]
    table[20] = [30, 31]
    tp, tr, _ = template(4, k, 8)
    assert tp[:2] == [-1, 0] and tr[:2] == [0, 0]
    root_r = OTail.retrieval_root(5, [11, 12, 13, 14], [0.9, 0.8, 0.3, 0.95], 0.5)
    assert root_r == 12
    ret = OTab.retrieve(table, root_r, tp, tr)
    t = OTail.build_one(5, [11, 12, 13, 14], [0.9, 0.8, 0.3, 0.95], 0.5, ret, tp, 100, V)
    assert t["keep"] == 2 and t["n"] == 5
    assert t["parent"] == [-1, 0, 1, 2, 3]
    assert t["token"] == [5, 11, 12, 20, 30]
    assert t["depth"] == [0, 1, 2, 3, 4]
    assert t["pos"] == [100, 101, 102, 103, 104]
    assert t["mask"] == [1, 3, 7, 15, 31]
    assert t["src"] == [OTree.SRC_ROOT, OTree.SRC_DRAFT, OTree.SRC_DRAFT, OTree.SRC_RETRIEVED, OTree.SRC_RETRIEVED]


def _case(r, L, V, k):
    table = np.stack([r.choice(V, k, replace=False) for _ in range(V)]).astype(np.int32)
    block = [int(x) for x in r.integers(0, V, L)]
    conf = [float(np.float32(x)) for x in r.random(L)]
    root = int(r.integers(0, V))
    tp, tr, _ = template(L, k, 8)
    return table, block, conf, root, tp, tr


@pytest.mark.parametrize("seed", range(20))
def test_budget_is_fixed_and_retrieval_hangs_under_the_deepest_kept_node(seed):
    r = np.random.default_rng(seed)
    L, V, k = 16, 300, 8
    table, block, conf, root, tp, tr = _case(r, L, V, k)
    tau = float(r.random())
    root_r = OTail.retrieval_root(root, block, conf, tau)
    t = OTail.build_one(root, block, conf, tau, OTab.retrieve(table, root_r, tp, tr), tp, 7, V)
    K = t["keep"]
    assert t["n"] == 1 + L
    assert all(c >= np.float32(tau) for c in conf[:K]) and (K == L or not conf[K] >= np.float32(tau))
    assert t["parent"][:K + 1] == [-1] + list(range(K))
    tdepth = [0] * L
    for i in range(L):
        tdepth[i] = 1 if tp[i] < 0 else tdepth[tp[i]] + 1
    assert t["depth"][K + 1:] == [K + d for d in tdepth[:L - K]]
    if K < L:
        assert t["token"][K + 1] == int(table[t["token"][K], tr[0]])


def test_no_confident_token_is_a_retrieval_only_graft_tree():
    r = np.random.default_rng(5)
    L, V, k = 16, 300, 8
    table, block, conf, root, tp, tr = _case(r, L, V, k)
    conf[0] = 0.01
    ret = OTab.retrieve(table, root, tp, tr)
    t = OTail.build_one(root, block, conf, 0.5, ret, tp, 3, V)
    ref = OTree.build_one([-1], [root], [1.0], 1, ret, tp, 3, V)
    for key in ("parent", "token", "depth", "pos", "mask", "src"):
        assert t[key] == ref[key], key


def test_all_confident_is_the_plain_chain():
    L, V = 16, 300
    block = list(range(100, 116))
    t = OTail.build_one(7, block, [1.0] * L, 0.5, [0] * L, [-1] * L, 0, V)
    assert t["keep"] == L and t["parent"] == [-1] + list(range(L)) and t["token"] == [7] + block
    assert t["depth"] == list(range(L + 1)) and t["mask"] == [(1 << (i + 1)) - 1 for i in range(L + 1)]


def test_confidences_after_the_cut_do_not_matter():
    r = np.random.default_rng(8)
    L, V, k = 16, 300, 8
    table, block, conf, root, tp, tr = _case(r, L, V, k)
    conf[5] = 0.0
    a = OTail.build_one(root, block, conf, 0.5, OTab.retrieve(table, block[4] if OTail.keep_length(conf, 0.5) == 5
                                                              else root, tp, tr), tp, 0, V)
    conf2 = conf[:6] + [1.0] * (L - 6)
    b = OTail.build_one(root, block, conf2, 0.5, OTab.retrieve(table, OTail.retrieval_root(root, block, conf2, 0.5),
                                                               tp, tr), tp, 0, V)
    assert OTail.keep_length(conf2, 0.5) == OTail.keep_length(conf, 0.5) <= 5
    assert a == b


def test_threshold_compare_is_fp32_and_nan_is_low():
    t = np.float32(0.3)
    assert OTail.keep_length([float(t), 0.9], 0.3) == 2          # equal to tau is kept
    assert OTail.keep_length([float(np.nextafter(t, 0)), 0.9], 0.3) == 0
    assert OTail.keep_length([0.9, float("nan"), 0.9], 0.3) == 1


def test_malformed_inputs_are_rejected():
    with pytest.raises(OracleError):
        OTail.build_one(1, [2, 3], [0.9], 0.5, [0, 0], [-1, 0], 0, 10)
    with pytest.raises(OracleError):
        OTail.build_one(1, [2, 30], [0.9, 0.9], 0.5, [0, 0], [-1, 0], 0, 10)
