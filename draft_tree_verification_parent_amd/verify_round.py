"""One round of tree speculative decoding driven through libgraft.

Order on one HIP stream (Graft page, arXiv:2605.20104 write-up, section 2;
section 6, second level):
  0. graft_prune_anchor          -- (trees pruned past checkpoint 0) the
                                    retrieval anchor inside the draft tree;
  1. graft_table_update_retrieve -- the previous round's verified positions
     rewrite their table rows, then the retrieval template is expanded from
     the current root token (or the anchor's);
  2. graft_build_tree            -- select, append retrieved nodes, flatten,
                                    depth / positions / mask;
  3. graft_tree_attention        -- one tree-masked attention layer;
  4. graft_lmhead_topk           -- logits and their per-row top-k, fused
                                    (logits never written) or, with
                                    fused=False, as two calls that
                                    materialise the logits;
  5. graft_accept                -- deepest accepted path and bonus token;
  6. graft_kv_compact            -- (chain=True) the accepted path's K/V to
                                    the front of the tree slots, the context
                                    advances, the bonus becomes the root.
The next round's update reads this round's tree tokens and top-k ids.

Device memory comes from torch; every computation runs in libgraft.
"""
from __future__ import annotations

import numpy as np
import torch

from . import api
from ._native import TREE_PRUNE, TREE_STATIC_REPLACE, TREE_TAIL, W_PACKED, W_ROWMAJOR

STEPS_FUSED = ("update_retrieve", "build_tree", "tree_attention", "lmhead_topk", "accept")
STEPS_SPLIT = ("update_retrieve", "build_tree", "tree_attention", "lmhead", "topk", "accept")
# temperature T > 0: one Gumbel-max draw per row, first-match acceptance
STEPS_FUSED_T = ("update_retrieve", "build_tree", "tree_attention", "lmhead_topk_sample", "accept_sampled")
STEPS_SPLIT_T = ("update_retrieve", "build_tree", "tree_attention", "lmhead", "topk", "sample", "accept_sampled")


def _i32(x, dev):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(dev)


def _bf16(bits, dev):
    a = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(a).to(dev).view(torch.bfloat16)


class VerifyRound:
    def __init__(self, ri, w_bits=None, device="cuda", dmax: int = 8, fused: bool = True,
                 packed: bool = True, chain: bool = False, temperature: float = 0.0):
        """fused: lm-head and top-k in one pass (logits never stored);
        packed: the lm-head weight is packed once here (when H % 128 == 0)
        and the fused pass reads the packed copy;
        chain: every round ends with KV compaction and the next round
        starts from its context and root (the cache needs headroom: see
        synth make_round_inputs(extra_slots=...));
        temperature > 0: acceptance by one draw per node (set_gumbel gives
        each round's noise) instead of the argmax."""
        dev = torch.device(device)
        self.fused = fused
        self.chain = chain
        self.temperature = float(temperature)
        if self.temperature > 0:
            base = STEPS_FUSED_T if fused else STEPS_SPLIT_T
        else:
            base = STEPS_FUSED if fused else STEPS_SPLIT
        self.tail = bool(getattr(ri.wl, "tail", False))
        stage = getattr(ri, "stage", None)
        # trees pruned past checkpoint 0 retrieve from an anchor inside the draft tree
        self.anchored = stage is not None and bool(np.any(np.asarray(stage) > 0))
        pre = ("tail_cut",) if self.tail else (("treegraft",) if getattr(ri, "tg_tok", None) is not None else ())
        if self.anchored:
            pre = pre + ("prune_anchor",)
        self.steps = pre + base + (("kv_compact",) if chain else ())
        wl = ri.wl
        self.ri, self.wl, self.dev = ri, wl, dev
        B, N, k, V = ri.B, ri.N, ri.k, ri.V
        self.B, self.N, self.k, self.V = B, N, k, V
        self.rows = int(ri.row_off[-1])

        # retrieval templates from the library's host helper
        tp, tr, off = [], [], [0]
        for b in range(B):
            p, r = api.graft_make_template(int(ri.n_ret[b]), k, dmax)
            tp.append(p)
            tr.append(r)
            off.append(off[-1] + len(p))
        self.tmpl_rows = off[-1]
        self.tmpl_parent = _i32(np.concatenate(tp) if self.tmpl_rows else np.zeros(1), dev)
        self.tmpl_rank = _i32(np.concatenate(tr) if self.tmpl_rows else np.zeros(1), dev)
        self.tmpl_off = _i32(off, dev)

        self.table = _i32(ri.table, dev)
        self.treegraft = getattr(ri, "tg_tok", None) is not None
        if self.treegraft:
            # TreeGraft: the candidates are built on the device every round
            # (graft_treegraft_build) from the drafter stand-ins' outputs
            counts = [api.graft_treegraft_node_count(wl.D, wl.Wf, wl.m, int(mk)) for mk in ri.tg_mask]
            cand_off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
            self.tg_mask = _i32(ri.tg_mask, dev)
            self.tg_tok = _i32(ri.tg_tok, dev)
            self.tg_prob = torch.from_numpy(np.ascontiguousarray(ri.tg_prob, np.float32)).to(dev)
            self.tg_q = torch.from_numpy(np.concatenate([ri.tg_q[b][:counts[b]] for b in range(B)])
                                         .astype(np.float32)).to(dev)
            self.cand_parent = torch.empty(int(cand_off[-1]), dtype=torch.int32, device=dev)
            self.cand_token = torch.empty(int(cand_off[-1]), dtype=torch.int32, device=dev)
            self.cand_score = torch.empty(int(cand_off[-1]), dtype=torch.float32, device=dev)
        else:
            cand_off = np.asarray(ri.cand_off, np.int32)
            self.cand_parent = _i32(ri.cand_parent, dev)
            self.cand_token = _i32(ri.cand_token, dev)
            self.cand_score = torch.from_numpy(np.ascontiguousarray(ri.cand_score, np.float32)).to(dev)
        self.cand_off_h = cand_off
        self.cand_off = _i32(cand_off, dev)
        self.max_cand = int(np.max(np.diff(cand_off)))
        self.budget = _i32(ri.budget, dev)
        if self.anchored:
            self.stage = _i32(stage, dev)
            self.anchor = torch.empty(B, dtype=torch.int32, device=dev)
            self.anchor_token = torch.empty(B, dtype=torch.int32, device=dev)
        self.ctx_len = _i32(ri.ctx_len, dev)
        # chained rounds plan attention for the largest context the cache
        # can still hold a tree after
        self.max_ctx = int(ri.kv_cap - ri.N) if chain else int(np.max(ri.ctx_len))
        self.row_off = _i32(ri.row_off, dev)
        self.root_token = _i32(ri.root_token, dev)
        self.mode = TREE_TAIL if self.tail else (TREE_STATIC_REPLACE if wl.static_replace else TREE_PRUNE)
        if self.tail:
            # Graft-TAIL: the block after each root and its confidences, and
            # the cut's outputs (kept length, retrieval root)
            L = N - 1
            idx = np.asarray(ri.cand_off[:-1], np.int64)[:, None] + 1 + np.arange(L)[None, :]
            self.block_token = _i32(np.asarray(ri.cand_token)[idx], dev)
            self.block_conf = torch.from_numpy(np.ascontiguousarray(np.asarray(ri.cand_score)[idx], np.float32)).to(dev)
            self.tail_keep = torch.empty(B, dtype=torch.int32, device=dev)
            self.tail_root = torch.empty(B, dtype=torch.int32, device=dev)

        # the update list of the first round: the synthetic previous round
        self.upd = dict(n=_i32(ri.prev_n, dev), row_off=_i32(ri.prev_row_off, dev),
                        token=_i32(ri.prev_token, dev), topk=_i32(ri.prev_topk, dev),
                        rows=int(ri.prev_row_off[-1]))

        rows = self.rows
        z = lambda *s, dt=torch.int32: torch.empty(*s, dtype=dt, device=dev)  # noqa: E731
        self.ret_token = z(max(self.tmpl_rows, 1))
        self.n_out = z(B)
        self.parent = z(rows)
        self.token = z(rows)
        self.depth = z(rows)
        self.pos = z(rows)
        self.mask = z(rows, dt=torch.int64)
        self.src = z(rows, dt=torch.int8)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)

        self.q = _bf16(ri.q.reshape(rows, wl.Hq, wl.d), dev)
        self.kcache = _bf16(ri.kcache.reshape(-1), dev)
        self.vcache = _bf16(ri.vcache.reshape(-1), dev)
        self.kv_off = torch.from_numpy(np.ascontiguousarray(ri.kv_off, np.int64)).to(dev)
        self.attn_out = torch.empty(rows, wl.Hq, wl.d, dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty(rows, wl.Hq, dtype=torch.float32, device=dev)
        wsb = api.graft_tree_attention_workspace_bytes(B, wl.Hq, wl.Hkv, wl.d, self.max_ctx, N)
        self.attn_ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)

        self.w = _bf16(w_bits, dev) if w_bits is not None else None
        self.w_packed = None
        if self.w is not None and packed and wl.H % 128 == 0:
            nb = api.graft_lmhead_pack_bytes(V, wl.H)
            self.w_packed = torch.empty(nb // 2, dtype=torch.bfloat16, device=dev)
            api.graft_lmhead_pack(V, wl.H, self.w, self.w_packed)
        self.hidden = None
        self.logits = None if fused else torch.empty(rows, V, dtype=torch.float32, device=dev)
        self.topk_id = z(rows, k)
        self.topk_val = torch.empty(rows, k, dtype=torch.float32, device=dev)
        tkb = api.graft_lmhead_topk_workspace_bytes(rows, V, k)
        self.topk_ws = torch.empty(max(tkb, 1), dtype=torch.uint8, device=dev)

        self.sample_id = z(rows)
        self.gumbel = None
        self.sample_ws = None
        if self.temperature > 0 and fused:
            if self.w_packed is None:
                raise ValueError("sampling with the fused lm-head needs the packed weight (H % 128 == 0)")
            self.sample_ws = torch.empty(api.graft_lmhead_sample_workspace_bytes(rows, V, k), dtype=torch.uint8,
                                         device=dev)
        self.acc_len = z(B)
        self.acc_path = z(B, 64)
        self.bonus = z(B)
        self.graph = None
        self.graph_rounds = 0
        if chain:
            # the next round's context and root are written to the other
            # buffer of each pair (compaction reads the current one in every
            # workgroup); the pairs swap after each round
            self.ctx_alt = z(B)
            self.root_alt = z(B)
            self.cand_root_idx = torch.from_numpy(np.asarray(self.cand_off_h[:-1], np.int64)).to(dev)

    def set_hidden(self, hidden_bits):
        self.hidden = _bf16(hidden_bits.reshape(self.rows, self.wl.H), self.dev)

    def set_gumbel(self, noise):
        """This round's Gumbel(0, 1) noise, fp32 [rows, V] (temperature > 0).
        Copied into one fixed buffer, so captured graphs see new noise."""
        x = torch.from_numpy(np.ascontiguousarray(noise, np.float32).reshape(self.rows, self.V))
        if self.gumbel is None:
            self.gumbel = x.to(self.dev)
        else:
            self.gumbel.copy_(x)

    def chain_update(self):
        """Make the next round's update read this round's verified nodes."""
        self.upd = dict(n=self.n_out, row_off=self.row_off, token=self.token, topk=self.topk_id,
                        rows=self.rows)

    # individual steps -------------------------------------------------
    def step_treegraft(self):
        wl = self.wl
        api.graft_treegraft_build(wl.D, wl.Wf, wl.m, self.tg_mask, self.root_token, self.tg_tok, self.tg_prob,
                                  self.tg_q, self.cand_off, self.cand_parent, self.cand_token, self.cand_score,
                                  self.err)

    def step_tail_cut(self):
        api.graft_tail_cut(self.root_token, self.block_token, self.block_conf, self.wl.replace_thresh,
                           self.tail_keep, self.tail_root)

    def step_prune_anchor(self):
        api.graft_prune_anchor(self.cand_parent, self.cand_token, self.cand_score, self.cand_off, self.max_cand,
                               self.budget, self.stage, self.anchor, self.anchor_token, self.err)

    def step_update_retrieve(self):
        u = self.upd
        # Graft-TAIL: the deepest kept node; checkpoint pruning: the anchor
        root = self.tail_root if self.tail else (self.anchor_token if self.anchored else self.root_token)
        api.graft_table_update_retrieve(self.table, u["n"], u["row_off"], u["rows"], u["token"],
                                        u["topk"], root, self.tmpl_parent, self.tmpl_rank,
                                        self.tmpl_off, self.tmpl_rows, self.ret_token, self.err)

    def step_build_tree(self):
        api.graft_build_tree(self.mode, self.cand_parent, self.cand_token, self.cand_score,
                             self.cand_off, self.max_cand, self.budget, self.ret_token,
                             self.tmpl_parent, self.tmpl_off if self.tmpl_rows else None,
                             self.table, self.V, self.k, self.wl.replace_thresh, self.ctx_len,
                             self.row_off, self.n_out, self.parent, self.token, self.depth,
                             self.pos, self.mask, self.src, self.err,
                             ret_anchor=self.anchor if self.anchored else None)

    def step_tree_attention(self):
        wl = self.wl
        api.graft_tree_attention(wl.Hq, wl.Hkv, wl.d, self.ri.scale, self.q, self.kcache, self.vcache,
                                 self.kv_off, self.ri.kv_head_stride, self.ctx_len, self.max_ctx,
                                 self.n_out, self.N, self.row_off, self.mask, self.attn_out, self.lse,
                                 self.attn_ws, self.err)

    def step_lmhead(self):
        api.graft_lmhead_topk(self.rows, self.wl.H, self.V, 0, self.hidden, self.w, self.logits)

    def step_lmhead_topk(self):
        if self.w_packed is not None:
            api.graft_lmhead_topk(self.rows, self.wl.H, self.V, self.k, self.hidden, self.w_packed, None,
                                  self.topk_id, self.topk_val, self.topk_ws, w_layout=W_PACKED)
        else:
            api.graft_lmhead_topk(self.rows, self.wl.H, self.V, self.k, self.hidden, self.w, None,
                                  self.topk_id, self.topk_val, self.topk_ws, w_layout=W_ROWMAJOR)

    def step_topk(self):
        api.graft_lmhead_topk(self.rows, self.wl.H, self.V, self.k, None, None, self.logits,
                              self.topk_id, self.topk_val, self.topk_ws)

    def step_lmhead_topk_sample(self):
        api.graft_lmhead_topk_sample(self.rows, self.wl.H, self.V, self.k, self.temperature, self.hidden,
                                     self.w_packed, self.gumbel, self.topk_id, self.topk_val, self.sample_id,
                                     self.sample_ws)

    def step_sample(self):
        api.graft_sample_rows(self.temperature, self.logits, self.gumbel, self.sample_id)

    def step_accept_sampled(self):
        api.graft_accept_sampled(self.n_out, self.row_off, self.parent, self.token, self.sample_id,
                                 self.acc_len, self.acc_path, self.bonus, self.err)

    def step_kv_compact(self):
        wl = self.wl
        api.graft_kv_compact(wl.Hkv, wl.d, self.kcache, self.vcache, self.kv_off, self.ri.kv_head_stride,
                             self.ctx_len, self.n_out, self.acc_len, self.acc_path, self.bonus,
                             self.ctx_alt, self.root_alt, err=self.err)
        # drafter stand-in: the next round's candidates hang off the new root
        self.cand_token.index_copy_(0, self.cand_root_idx, self.root_alt)
        self.ctx_len, self.ctx_alt = self.ctx_alt, self.ctx_len
        self.root_token, self.root_alt = self.root_alt, self.root_token
        self.chain_update()

    def step_accept(self):
        api.graft_accept(self.n_out, self.row_off, self.parent, self.token, self.topk_id, self.k,
                         self.acc_len, self.acc_path, self.bonus, self.err)

    def build_only(self):
        """Enqueue the round's steps up to and including the tree build (for a
        first look at the tree, e.g. to plant the synthetic target on it)."""
        for name in self.steps:
            getattr(self, "step_" + name)()
            if name == "build_tree":
                return

    def run(self, events=None):
        """Enqueue one round.  `events`, if given, is a dict step -> list that
        receives (start, end) torch.cuda.Event pairs recorded on the stream."""
        for name in self.steps:
            fn = getattr(self, "step_" + name)
            if events is None:
                fn()
            else:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                events.setdefault(name, []).append((e0, e1))

    def capture(self, rounds: int = 1):
        """Record `rounds` consecutive rounds as one HIP graph with the update
        pointers as they stand (call chain_update() first for steady-state
        rounds: every round then reads the previous round's outputs from the
        same buffers, so rounds chain inside the graph as they do across
        replays).  Nothing runs during capture; replay() issues the rounds.
        The rounds have no memset nodes and no host synchronisation, so they
        replay as recorded."""
        if rounds < 1:
            raise ValueError("rounds must be >= 1")
        if self.chain and rounds % 2:
            # each chained round swaps the context / root buffers; an odd
            # count would start every replay from the stale pair
            raise ValueError("chained rounds are captured in even numbers")
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for _ in range(rounds):
                self.run()
        self.graph = g
        self.graph_rounds = rounds
        return g

    def replay(self):
        """Issue the captured rounds (graph_rounds of them)."""
        self.graph.replay()

    def tree_host(self):
        """Built tree copied to the host (synchronises)."""
        return dict(n=self.n_out.cpu().numpy(), parent=self.parent.cpu().numpy(),
                    token=self.token.cpu().numpy(), depth=self.depth.cpu().numpy(),
                    pos=self.pos.cpu().numpy(), mask=self.mask.cpu().numpy().view(np.uint64),
                    src=self.src.cpu().numpy())
