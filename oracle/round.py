"""One round composed from the oracle's steps (test infrastructure only).

Order within a round (Graft page, section 2; section 6, second level):
the previous round's verified positions update the successor table, the
current token's retrieval tree is read from the updated table, the hybrid
tree is built and flattened, the target verifies it (tree attention, then
the lm-head), every position's top-k is taken, and the deepest greedily
accepted path is kept.  The next round's update reads this round's tokens
and top-k; chaining (next_round_inputs) then compacts the accepted path's
K/V, advances the context and makes the bonus token the next root.

The inputs object only needs the attributes named below (numpy arrays);
hidden states are passed in because the synthetic target model plants them
on the built tree.
"""
from __future__ import annotations

import numpy as np

from . import accept as _accept
from . import attention as _attention
from . import kv as _kv
from . import lmhead as _lmhead
from . import table as _table
from . import tail as _tail
from . import treegraft as _treegraft
from . import template as _template
from . import topk as _topk
from . import tree as _tree


def tree_stage(ri, dmax: int = 8):
    """Update + retrieve + build.  Returns dict(table, tparent, trank,
    tmpl_off, ret_token, tree)."""
    table = _table.update(ri.table, ri.prev_n, ri.prev_row_off, ri.prev_token, ri.prev_topk)
    if getattr(ri.wl, "tail", False):
        return _tail_tree_stage(ri, table, dmax)
    cand_parent, cand_token, cand_score, cand_off = ri.cand_parent, ri.cand_token, ri.cand_score, ri.cand_off
    if getattr(ri, "tg_tok", None) is not None:
        cand_parent, cand_token, cand_score, cand_off = treegraft_candidates(ri)
    # Graft's checkpoints: a tree pruned at checkpoint depth c retrieves from
    # the deepest kept node of the best path at depth c (the root at c = 0)
    stage = getattr(ri, "stage", None)
    anchor = np.zeros(ri.B, np.int32)
    if stage is not None:
        for b in range(ri.B):
            c0, c1 = int(cand_off[b]), int(cand_off[b + 1])
            if int(stage[b]) > 0:
                anchor[b] = _tree.retrieval_anchor(cand_parent[c0:c1], cand_score[c0:c1], int(ri.budget[b]),
                                                   int(stage[b]))
    tp_all, tr_all, rt_all, off = [], [], [], [0]
    for b in range(ri.B):
        tp, tr, _ = _template.template(int(ri.n_ret[b]), ri.k, dmax)
        root = int(cand_token[int(cand_off[b]) + int(anchor[b])]) if anchor[b] else int(ri.root_token[b])
        rt = _table.retrieve(table, root, tp, tr)
        tp_all += tp
        tr_all += tr
        rt_all += rt
        off.append(off[-1] + len(tp))
    tparent = np.array(tp_all, np.int32)
    trank = np.array(tr_all, np.int32)
    ret_token = np.array(rt_all, np.int32)
    tmpl_off = np.array(off, np.int32)
    wl = ri.wl
    tree = _tree.build_batch(cand_parent, cand_token, cand_score, cand_off,
                             ri.budget, ret_token, tparent, tmpl_off, ri.ctx_len, ri.V,
                             ri.row_off, static_replace=wl.static_replace, table=table,
                             replace_thresh=wl.replace_thresh, anchor=anchor)
    return dict(table=table, tparent=tparent, trank=trank, tmpl_off=tmpl_off,
                ret_token=ret_token, tree=tree, anchor=anchor)


def treegraft_candidates(ri):
    """TreeGraft workloads: each request's candidates built by the shared-tree
    construction (oracle.treegraft) from its drafter outputs and schedule,
    with the current root token.  Returns (parent, token, score, cand_off)."""
    wl = ri.wl
    par, tok, sc, off = [], [], [], [0]
    for b in range(ri.B):
        n = _treegraft.node_count(wl.D, wl.Wf, wl.m, int(ri.tg_mask[b]))
        p, t, s = _treegraft.build(int(ri.root_token[b]), wl.D, wl.Wf, wl.m, int(ri.tg_mask[b]), ri.tg_tok[b],
                                   ri.tg_prob[b], ri.tg_q[b][:n])
        par += p
        tok += t
        sc += s
        off.append(off[-1] + n)
    return (np.array(par, np.int32), np.array(tok, np.int32), np.array(sc, np.float32), np.array(off, np.int32))


def _tail_tree_stage(ri, table, dmax: int):
    """Graft-TAIL workloads: candidates are the root and a block of L tokens
    (cand_score = confidences); retrieval runs from each request's deepest
    kept node with the size-L template (oracle.tail)."""
    L = ri.N - 1
    tau = ri.wl.replace_thresh
    tp, tr, _ = _template.template(L, ri.k, dmax)
    roots, blocks, confs, rets, rroots = [], [], [], [], []
    for b in range(ri.B):
        o = int(ri.cand_off[b])
        roots.append(int(ri.cand_token[o]))
        blocks.append(np.asarray(ri.cand_token[o + 1:o + 1 + L], np.int32))
        confs.append(np.asarray(ri.cand_score[o + 1:o + 1 + L], np.float32))
        rroots.append(_tail.retrieval_root(roots[-1], blocks[-1], confs[-1], tau))
        rets += _table.retrieve(table, rroots[-1], tp, tr)
    tparent = np.tile(np.array(tp, np.int32), ri.B)
    trank = np.tile(np.array(tr, np.int32), ri.B)
    tmpl_off = (np.arange(ri.B + 1) * L).astype(np.int32)
    ret_token = np.array(rets, np.int32)
    tree = _tail.build_batch(roots, blocks, confs, tau, ret_token, tparent, tmpl_off, ri.ctx_len, ri.V, ri.row_off)
    return dict(table=table, tparent=tparent, trank=trank, tmpl_off=tmpl_off, ret_token=ret_token, tree=tree,
                retrieval_root=np.array(rroots, np.int32))


def kv_f64(ri, b: int):
    """Request b's K and V caches as fp64 [Hkv, ctx_b + N, d]."""
    L = int(ri.ctx_len[b]) + ri.N
    K = _lmhead.bf16_to_f64(ri.kcache[b, :, :L]).reshape(ri.wl.Hkv, L, ri.wl.d)
    V = _lmhead.bf16_to_f64(ri.vcache[b, :, :L]).reshape(ri.wl.Hkv, L, ri.wl.d)
    return K, V


def verify_stage(ri, tree, hidden_bits, w_bits, attention_nodes=None):
    """Tree attention (one layer), lm-head, top-k, acceptance."""
    q = _lmhead.bf16_to_f64(ri.q).reshape(ri.q.shape)
    Ks, Vs = [], []
    for b in range(ri.B):
        K, V = kv_f64(ri, b)
        Ks.append(K)
        Vs.append(V)
    att = _attention.tree_attention(q, Ks, Vs, ri.ctx_len, tree["n"], ri.row_off,
                                    tree["mask"], ri.scale, nodes=attention_nodes)
    logits = _lmhead.logits(hidden_bits, w_bits)
    ids, vals = _topk.topk(logits, ri.k)
    lens, paths, bonus = _accept.accept_batch(tree["n"], ri.row_off, tree["parent"],
                                              tree["token"], ids[:, 0])
    return dict(attention=att, logits=logits, topk_id=ids, topk_val=vals,
                acc_len=lens, acc_path=paths, bonus=bonus)


def next_round_inputs(ri, ts, topk_id, acc_len, acc_path, bonus):
    """The inputs of the round after `ri` (Graft page, section 2, third
    step: only the accepted output is kept; the table update reads every
    verified position): the updated table, this round's tree tokens and
    top-k ids as the update list, the accepted path's K/V compacted to the
    front of the tree slots, ctx + a + 1, and the bonus token as the root --
    of retrieval and of the drafter stand-in's candidates alike (their
    candidate 0).  Returns a new inputs object; `ri` is not modified."""
    nxt = type(ri)(**dict(ri.__dict__))
    tree = ts["tree"]
    B = ri.B
    kc, vc, ctx_next, root_next = _kv.compact_batch(ri.kcache[None], ri.vcache[None], ri.ctx_len, tree["n"],
                                                    acc_len, acc_path, bonus)
    nxt.kcache, nxt.vcache = kc[0], vc[0]
    nxt.ctx_len = ctx_next.astype(np.int32)
    nxt.root_token = root_next.astype(np.int32)
    if ri.cand_token is not None:
        cand_token = np.array(ri.cand_token, np.int32).copy()
        for b in range(B):
            cand_token[int(ri.cand_off[b])] = int(bonus[b])
        nxt.cand_token = cand_token
    nxt.table = ts["table"]
    nxt.prev_n = np.array(tree["n"], np.int32)
    nxt.prev_row_off = np.array(ri.row_off, np.int32)
    nxt.prev_token = np.array(tree["token"], np.int32)
    nxt.prev_topk = np.array(topk_id, np.int32)
    return nxt
