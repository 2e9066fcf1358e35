"""Python binding of the C ABI (include/graft.h): same names, torch tensors in.

Argument marshalling only -- every step runs in libgraft's HIP kernels.
Device tensors must be contiguous and on the current GPU; work is enqueued
on `stream` (default: torch's current stream) and nothing synchronises,
except the table checkpoint calls, which wait for their stream.
"""
from __future__ import annotations

import os

import numpy as np
import torch

from . import _native as N
from ._native import call

_DT = {
    "i32": (torch.int32,),
    "i64": (torch.int64,),
    "u64": (torch.int64, getattr(torch, "uint64", torch.int64)),
    "f32": (torch.float32,),
    "bf16": (torch.bfloat16,),
    "i8": (torch.int8,),
}


def _p(t, kind: str, name: str):
    """Device pointer of `t` (or None), after dtype/layout checks."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name}: expected a CUDA/HIP tensor")
    if t.dtype not in _DT[kind]:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {_DT[kind]}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return t.data_ptr()


def _s(stream):
    return (stream if stream is not None else torch.cuda.current_stream()).cuda_stream


def graft_table_update_retrieve(table, upd_n, upd_row_off, upd_rows, upd_token, upd_topk,
                                root_token, tmpl_parent, tmpl_rank, tmpl_off, tmpl_rows,
                                ret_token, err=None, stream=None):
    V, k = table.shape
    B_upd = 0 if upd_n is None else upd_n.numel()
    B = 0 if root_token is None else root_token.numel()
    return call("graft_table_update_retrieve", _p(table, "i32", "table"), V, k, B_upd,
                _p(upd_n, "i32", "upd_n"), _p(upd_row_off, "i32", "upd_row_off"), int(upd_rows),
                _p(upd_token, "i32", "upd_token"), _p(upd_topk, "i32", "upd_topk"), B,
                _p(root_token, "i32", "root_token"), _p(tmpl_parent, "i32", "tmpl_parent"),
                _p(tmpl_rank, "i32", "tmpl_rank"), _p(tmpl_off, "i32", "tmpl_off"), int(tmpl_rows),
                _p(ret_token, "i32", "ret_token"), _p(err, "i32", "err"), _s(stream))


def graft_table_save(path, table, stream=None):
    """Writes the [V, k] int32 successor table (device) to `path`; waits for
    the stream."""
    V, k = table.shape
    return call("graft_table_save", os.fsencode(path), int(V), int(k), _p(table, "i32", "table"), _s(stream))


def graft_table_load(path, table, stream=None):
    """Reads a table file into `table` (device, [V, k] int32, overwritten
    only when the file checks out); waits for the stream."""
    V, k = table.shape
    return call("graft_table_load", os.fsencode(path), int(V), int(k), _p(table, "i32", "table"), _s(stream))


def graft_build_tree(mode, cand_parent, cand_token, cand_score, cand_off, max_cand, budget,
                     ret_token, ret_parent, ret_off, table, V, k, replace_thresh, ctx_len, row_off,
                     n_out, parent, token, depth, pos, mask, src, err=None, stream=None, ret_anchor=None):
    B = budget.numel()
    return call("graft_build_tree", B, int(mode), _p(cand_parent, "i32", "cand_parent"),
                _p(cand_token, "i32", "cand_token"), _p(cand_score, "f32", "cand_score"),
                _p(cand_off, "i32", "cand_off"), int(max_cand), _p(budget, "i32", "budget"),
                _p(ret_token, "i32", "ret_token"), _p(ret_parent, "i32", "ret_parent"),
                _p(ret_off, "i32", "ret_off"), _p(ret_anchor, "i32", "ret_anchor"),
                _p(table, "i32", "table"), int(V), int(k),
                float(replace_thresh), _p(ctx_len, "i32", "ctx_len"), _p(row_off, "i32", "row_off"),
                _p(n_out, "i32", "n_out"), _p(parent, "i32", "parent"), _p(token, "i32", "token"),
                _p(depth, "i32", "depth"), _p(pos, "i32", "pos"), _p(mask, "u64", "mask"),
                _p(src, "i8", "src"), _p(err, "i32", "err"), _s(stream))


def graft_prune_anchor(cand_parent, cand_token, cand_score, cand_off, max_cand, budget, stage, anchor,
                       anchor_token, err=None, stream=None):
    """Per request: the candidate a tree pruned at checkpoint depth stage[b]
    hangs its retrieved nodes under, and that candidate's token."""
    B = budget.numel()
    return call("graft_prune_anchor", B, _p(cand_parent, "i32", "cand_parent"), _p(cand_token, "i32", "cand_token"),
                _p(cand_score, "f32", "cand_score"), _p(cand_off, "i32", "cand_off"), int(max_cand),
                _p(budget, "i32", "budget"), _p(stage, "i32", "stage"), _p(anchor, "i32", "anchor"),
                _p(anchor_token, "i32", "anchor_token"), _p(err, "i32", "err"), _s(stream))


def graft_tree_attention_workspace_bytes(B, Hq, Hkv, d, max_ctx, max_n):
    return int(N.lib().graft_tree_attention_workspace_bytes(B, Hq, Hkv, d, max_ctx, max_n))


def graft_tree_attention(Hq, Hkv, d, scale, q, kcache, vcache, kv_off, kv_head_stride, ctx_len,
                         max_ctx, n, max_n, row_off, mask, out, lse=None, ws=None, err=None,
                         stream=None):
    B = ctx_len.numel()
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    return call("graft_tree_attention", B, Hq, Hkv, d, float(scale), _p(q, "bf16", "q"),
                _p(kcache, "bf16", "kcache"), _p(vcache, "bf16", "vcache"), _p(kv_off, "i64", "kv_off"),
                int(kv_head_stride), _p(ctx_len, "i32", "ctx_len"), int(max_ctx), _p(n, "i32", "n"),
                int(max_n), _p(row_off, "i32", "row_off"), _p(mask, "u64", "mask"), _p(out, "bf16", "out"),
                _p(lse, "f32", "lse"), None if ws is None else ws.data_ptr(), ws_bytes,
                _p(err, "i32", "err"), _s(stream))


def graft_lmhead_topk_workspace_bytes(M, V, k):
    return int(N.lib().graft_lmhead_topk_workspace_bytes(M, V, k))


def graft_lmhead_topk(M, H, V, k, hidden, w, logits, topk_id=None, topk_val=None, ws=None,
                      stream=None, w_layout=N.W_ROWMAJOR):
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    return call("graft_lmhead_topk", int(M), int(H), int(V), int(k), _p(hidden, "bf16", "hidden"),
                _p(w, "bf16", "w"), int(w_layout), _p(logits, "f32", "logits"), _p(topk_id, "i32", "topk_id"),
                _p(topk_val, "f32", "topk_val"), None if ws is None else ws.data_ptr(), ws_bytes,
                _s(stream))


def graft_lmhead_topk_noalloc_bytes(M, k):
    return int(N.lib().graft_lmhead_topk_noalloc_bytes(int(M), int(k)))


def graft_lmhead_topk_noalloc(M, H, V, k, hidden, w_packed, topk_id, topk_val=None, stream=None):
    """Fused packed lm-head + top-k with the library's built-in scratch (no
    workspace argument; the call allocates nothing)."""
    return call("graft_lmhead_topk_noalloc", int(M), int(H), int(V), int(k), _p(hidden, "bf16", "hidden"),
                _p(w_packed, "bf16", "w_packed"), _p(topk_id, "i32", "topk_id"), _p(topk_val, "f32", "topk_val"),
                _s(stream))


def graft_lmhead_pack_bytes(V, H):
    return int(N.lib().graft_lmhead_pack_bytes(V, H))


def graft_lmhead_pack(V, H, w, w_packed, stream=None):
    """Rewrite the row-major lm-head weight w [V, H] into the packed layout
    (w_packed: bf16 device tensor of graft_lmhead_pack_bytes(V, H) bytes)."""
    need = graft_lmhead_pack_bytes(V, H)
    if w_packed.numel() * w_packed.element_size() < need:
        raise ValueError(f"w_packed holds {w_packed.numel() * w_packed.element_size()} bytes < {need}")
    return call("graft_lmhead_pack", int(V), int(H), _p(w, "bf16", "w"), _p(w_packed, "bf16", "w_packed"),
                _s(stream))


def graft_accept(n, row_off, parent, token, topk_id, k, acc_len, acc_path, bonus, err=None,
                 stream=None):
    B = n.numel()
    return call("graft_accept", B, _p(n, "i32", "n"), _p(row_off, "i32", "row_off"),
                _p(parent, "i32", "parent"), _p(token, "i32", "token"), _p(topk_id, "i32", "topk_id"),
                int(k), _p(acc_len, "i32", "acc_len"), _p(acc_path, "i32", "acc_path"),
                _p(bonus, "i32", "bonus"), _p(err, "i32", "err"), _s(stream))


def graft_lmhead_sample_workspace_bytes(M, V, k):
    return int(N.lib().graft_lmhead_sample_workspace_bytes(int(M), int(V), int(k)))


def graft_lmhead_topk_sample(M, H, V, k, temperature, hidden, w_packed, gumbel, topk_id, topk_val, sample_id, ws,
                             stream=None):
    """Fused packed lm-head: per-row top-k and one Gumbel-max draw at
    `temperature` (noise `gumbel` fp32 [M, V])."""
    return call("graft_lmhead_topk_sample", int(M), int(H), int(V), int(k), float(temperature),
                _p(hidden, "bf16", "hidden"), _p(w_packed, "bf16", "w_packed"), _p(gumbel, "f32", "gumbel"),
                _p(topk_id, "i32", "topk_id"), _p(topk_val, "f32", "topk_val"), _p(sample_id, "i32", "sample_id"),
                None if ws is None else ws.data_ptr(), 0 if ws is None else ws.numel() * ws.element_size(),
                _s(stream))


def graft_sample_rows(temperature, logits, gumbel, sample_id, stream=None):
    M, V = logits.shape
    return call("graft_sample_rows", int(M), int(V), float(temperature), _p(logits, "f32", "logits"),
                _p(gumbel, "f32", "gumbel"), _p(sample_id, "i32", "sample_id"), _s(stream))


def graft_accept_sampled(n, row_off, parent, token, sample_id, acc_len, acc_path, bonus, err=None, stream=None):
    B = n.numel()
    return call("graft_accept_sampled", B, _p(n, "i32", "n"), _p(row_off, "i32", "row_off"),
                _p(parent, "i32", "parent"), _p(token, "i32", "token"), _p(sample_id, "i32", "sample_id"),
                _p(acc_len, "i32", "acc_len"), _p(acc_path, "i32", "acc_path"), _p(bonus, "i32", "bonus"),
                _p(err, "i32", "err"), _s(stream))


def graft_treegraft_node_count(D, W, m, mid_mask):
    return int(N.lib().graft_treegraft_node_count(int(D), int(W), int(m), int(mid_mask)))


def graft_treegraft_build(D, W, m, mid_mask, root_token, tok, prob, q, cand_off, cand_parent, cand_token, cand_score,
                          err=None, stream=None):
    """TreeGraft's shared tree per request (see include/graft.h)."""
    B = root_token.numel()
    return call("graft_treegraft_build", int(B), int(D), int(W), int(m), _p(mid_mask, "i32", "mid_mask"),
                _p(root_token, "i32", "root_token"), _p(tok, "i32", "tok"), _p(prob, "f32", "prob"),
                _p(q, "f32", "q"), _p(cand_off, "i32", "cand_off"), _p(cand_parent, "i32", "cand_parent"),
                _p(cand_token, "i32", "cand_token"), _p(cand_score, "f32", "cand_score"), _p(err, "i32", "err"),
                _s(stream))


def graft_tail_cut(root_token, block_token, block_conf, tau, keep_len, retrieval_root, stream=None):
    """Graft-TAIL: per request the kept prefix length of a block draft and
    the retrieval root (token of the deepest kept node)."""
    B, L = block_token.shape
    return call("graft_tail_cut", int(B), int(L), _p(root_token, "i32", "root_token"),
                _p(block_token, "i32", "block_token"), _p(block_conf, "f32", "block_conf"), float(tau),
                _p(keep_len, "i32", "keep_len"), _p(retrieval_root, "i32", "retrieval_root"), _s(stream))


def graft_kv_compact(Hkv, d, kcache, vcache, kv_off, kv_head_stride, ctx_len, n, acc_len, acc_path, bonus,
                     ctx_next, root_next, n_layers=1, layer_stride=0, err=None, stream=None):
    """Moves each request's accepted path K/V to slots ctx..ctx+a (every
    layer and KV head), writes ctx_next = ctx + a + 1 and root_next = bonus.
    kcache / vcache: bf16 caches addressed as in graft_tree_attention, plus
    `layer` * layer_stride elements."""
    B = ctx_len.numel()
    return call("graft_kv_compact", B, int(Hkv), int(d), int(n_layers), _p(kcache, "bf16", "kcache"),
                _p(vcache, "bf16", "vcache"), int(layer_stride), _p(kv_off, "i64", "kv_off"), int(kv_head_stride),
                _p(ctx_len, "i32", "ctx_len"), _p(n, "i32", "n"), _p(acc_len, "i32", "acc_len"),
                _p(acc_path, "i32", "acc_path"), _p(bonus, "i32", "bonus"), _p(ctx_next, "i32", "ctx_next"),
                _p(root_next, "i32", "root_next"), _p(err, "i32", "err"), _s(stream))


def graft_make_template(R, k, dmax=8):
    """Host helper: (tmpl_parent, tmpl_rank) int32 numpy arrays of length R."""
    tp = np.zeros(max(R, 1), np.int32)
    tr = np.zeros(max(R, 1), np.int32)
    call("graft_make_template", int(R), int(k), int(dmax), tp.ctypes.data, tr.ctypes.data)
    return tp[:R], tr[:R]


def graft_stage_budget(stage):
    d = np.zeros(1, np.int32)
    r = np.zeros(1, np.int32)
    call("graft_stage_budget", int(stage), d.ctypes.data, r.ctypes.data)
    return int(d[0]), int(r[0])
