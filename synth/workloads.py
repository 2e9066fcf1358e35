"""The five synthetic verify-round workloads and their seeded generators.

Every tensor is drawn from numpy's PCG64 seeded with
``SeedSequence(20261202 + cfg)`` and a per-tensor spawn key (the CRC32 of
the tensor's name), so each tensor can be regenerated on its own.

Workload shapes follow the model families the pages evaluate on
(Llama-3.1-8B, Qwen3-8B, Qwen3-14B; Graft page, section 4; TreeGraft page,
section 5) and the tree settings they state: Graft's 60-slot budget split
8/52, 24/36, 40/20 by pruning stage (Graft page, section 2), TreeGraft's
D=5, W=10, m=10, Bver=63 (TreeGraft page, section 5), and Graft's batched
static tree (Graft page, section 4, serving paragraph).

The draft candidates come from a stand-in for an EAGLE-style drafter
(TreeGraft page, section 3): the drafter itself needs trained weights and
is outside the verify round, so its per-edge probabilities are drawn from
Dirichlet(0.3) instead of computed.
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass

import numpy as np

from .bf16 import bf16_bits_to_f32, f32_to_bf16_bits

SEED_BASE = 20261202
W_BLOCK_ROWS = 4096  # lm-head weight rows drawn per independent child stream


def rng(cfg: int, name: str) -> np.random.Generator:
    ss = np.random.SeedSequence(SEED_BASE + cfg, spawn_key=(zlib.crc32(name.encode()),))
    return np.random.Generator(np.random.PCG64(ss))


@dataclass(frozen=True)
class Workload:
    cfg: int
    name: str
    B: int            # requests
    Hq: int           # query heads
    Hkv: int          # key/value heads
    d: int            # head dim
    H: int            # hidden size (lm-head K)
    V: int            # vocabulary (lm-head N, successor-table rows)
    k: int            # successor-table width = top-k width
    ctx_lo: int       # per-request context length, uniform in [ctx_lo, ctx_hi]
    ctx_hi: int
    tree: str         # 'random' (small random parent array) | 'eagle' (drafter stand-in)
    n_nodes: int      # verify slots per request, root included
    draft_budget: int  # draft nodes kept, root included
    n_retrieved: int  # retrieved nodes appended under the root
    static_replace: bool = False
    replace_thresh: float = 0.05
    ctx_tokens: bool = False  # draw a token context with repeated 8-gram spans
    D: int = 5        # drafter depth
    Wf: int = 10      # drafter frontier width
    m: int = 10       # children per frontier node
    tail: bool = False  # Graft-TAIL on a block draft of n_nodes - 1 tokens
    mid_mask: int = -1  # >= 0: TreeGraft shared tree built on the device (bit k: step k by the mid drafter)
    stages: tuple = ()  # per-request pruning checkpoint (0, 1, 5; -1 = none), cycled over the batch; sets
    #                     the draft budget and retrieved count per request (Graft's 60-slot split)

    def with_ctx(self, lo: int, hi: int | None = None) -> "Workload":
        d = dict(self.__dict__)
        d["ctx_lo"] = lo
        d["ctx_hi"] = lo if hi is None else hi
        return Workload(**d)

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    1: Workload(1, "tiny: 4q/2kv heads d64, ctx 256, 15-node random tree, lm-head 256x1024",
                B=1, Hq=4, Hkv=2, d=64, H=256, V=1024, k=8, ctx_lo=256, ctx_hi=256,
                tree="random", n_nodes=15, draft_budget=15, n_retrieved=0),
    2: Workload(2, "Llama-3.1-8B-shaped, batch 1: 32q/8kv d128, ctx 4096, 60 slots = 8 draft + 52 retrieved, "
                   "lm-head 4096x128256, table 128256x8",
                B=1, Hq=32, Hkv=8, d=128, H=4096, V=128256, k=8, ctx_lo=4096, ctx_hi=4096,
                tree="eagle", n_nodes=60, draft_budget=8, n_retrieved=52),
    3: Workload(3, "Qwen3-8B-shaped, batch 1: 32q/8kv d128, ctx 32768, EAGLE tree pruned to Bver=63, "
                   "lm-head 4096x151936, table 151936x10",
                B=1, Hq=32, Hkv=8, d=128, H=4096, V=151936, k=10, ctx_lo=32768, ctx_hi=32768,
                tree="eagle", n_nodes=63, draft_budget=63, n_retrieved=0),
    4: Workload(4, "Qwen3-14B-shaped long context: 40q/8kv d128, ctx 65536, 60 slots = 24 draft + 36 retrieved "
                   "(pruned at checkpoint 1), lm-head 5120x151936, table 151936x8 warmed from a repetitive context",
                B=1, Hq=40, Hkv=8, d=128, H=5120, V=151936, k=8, ctx_lo=65536, ctx_hi=65536,
                tree="eagle", n_nodes=60, draft_budget=24, n_retrieved=36, ctx_tokens=True, stages=(1,)),
    5: Workload(5, "batched static tree: 16 requests, Qwen3-8B shapes, ctx U[4096,16384], 60-slot trees with "
                   "score<0.05 nodes replaced from a shared 151936x8 table",
                B=16, Hq=32, Hkv=8, d=128, H=4096, V=151936, k=8, ctx_lo=4096, ctx_hi=16384,
                tree="eagle", n_nodes=60, draft_budget=60, n_retrieved=0,
                static_replace=True, replace_thresh=0.05),
    6: Workload(6, "Graft-TAIL on DFlash-style block drafts: 4 requests, Qwen3-8B shapes, ctx 4096, 16-token blocks "
                   "cut at confidence < 0.5, tails from a shared 151936x8 table",
                B=4, Hq=32, Hkv=8, d=128, H=4096, V=151936, k=8, ctx_lo=4096, ctx_hi=4096,
                tree="block", n_nodes=17, draft_budget=17, n_retrieved=16, tail=True, replace_thresh=0.5),
    7: Workload(7, "TreeGraft shared tree: Qwen3-8B shapes, batch 1, ctx 32768, D=5 W=10 m=10 with the mid "
                   "drafter at step 2, pruned to Bver=63, lm-head 4096x151936, table 151936x10",
                B=1, Hq=32, Hkv=8, d=128, H=4096, V=151936, k=10, ctx_lo=32768, ctx_hi=32768,
                tree="treegraft", n_nodes=63, draft_budget=63, n_retrieved=0, mid_mask=0b00100),
    8: Workload(8, "Graft stage-adaptive batch: 4 requests, Qwen3-8B shapes, ctx U[4096,8192], 60 slots pruned at "
                   "checkpoints 5, 1, 0 and not at all (40+20, 24+36, 8+52, 60+0), table 151936x8",
                B=4, Hq=32, Hkv=8, d=128, H=4096, V=151936, k=8, ctx_lo=4096, ctx_hi=8192,
                tree="eagle", n_nodes=60, draft_budget=40, n_retrieved=20, stages=(5, 1, 0, -1)),
}

# Graft's split of 60 verify slots by pruning checkpoint (Graft page, section
# 2, second step): checkpoint depth -> (draft nodes with the root, retrieved)
STAGE_SLOTS = {-1: (60, 0), 0: (8, 52), 1: (24, 36), 5: (40, 20)}


# ----------------------------------------------------------------------------
# drafter stand-ins
# ----------------------------------------------------------------------------

def _distinct_tokens(r: np.random.Generator, V: int, n: int) -> np.ndarray:
    if n > V:
        raise ValueError("more siblings than vocabulary entries")
    out: list[int] = []
    seen: set[int] = set()
    while len(out) < n:
        for t in r.integers(0, V, size=2 * n):
            t = int(t)
            if t not in seen:
                seen.add(t)
                out.append(t)
                if len(out) == n:
                    break
    return np.array(out, dtype=np.int32)


def eagle_candidates(r: np.random.Generator, V: int, D: int, Wf: int, m: int, root_token: int):
    """Candidate pool of a dynamic draft tree: the root is expanded into m
    children, then D-1 times the Wf best newest nodes (by cumulative score)
    each get m children.  Edge probabilities ~ Dirichlet(0.3), sorted
    descending; scores are kept in fp64 while drawing and returned as fp32.
    Candidate indices are topological (a parent precedes its children)."""
    parent = [-1]
    token = [root_token]
    score = [1.0]
    newest = [0]
    for step in range(D):
        if step == 0:
            frontier = [0]
        else:
            frontier = sorted(newest, key=lambda c: (-score[c], c))[:Wf]
        newest = []
        for f in frontier:
            p = np.sort(r.dirichlet(np.full(m, 0.3)))[::-1]
            toks = _distinct_tokens(r, V, m)
            for j in range(m):
                parent.append(f)
                token.append(int(toks[j]))
                score.append(score[f] * float(p[j]))
                newest.append(len(parent) - 1)
    return (np.array(parent, np.int32), np.array(token, np.int32),
            np.array(score, np.float64).astype(np.float32))


def block_draft(r: np.random.Generator, V: int, L: int, root_token: int):
    """A stand-in for a block (diffusion) drafter: the root and L chained
    tokens (Zipf over the vocabulary) with per-token confidences that decay
    along the block, conf_i = prod_{j<=i} b_j, b_j ~ Beta(8, 1) -- the score
    Graft-TAIL cuts on."""
    cdf = _zipf_cdf(V)
    tokens = np.concatenate([[root_token], zipf_ids(r, cdf, L)]).astype(np.int32)
    conf = np.cumprod(r.beta(8.0, 1.0, L)).astype(np.float32)
    parent = np.arange(-1, L, dtype=np.int32)
    score = np.concatenate([[1.0], conf]).astype(np.float32)
    return parent, tokens, score


def treegraft_drafter_outputs(r: np.random.Generator, V: int, D: int, Wf: int, m: int, n_nodes: int):
    """Stand-ins for TreeGraft's two drafters: for step k and frontier rank j,
    m distinct child tokens with edge probabilities Dirichlet(0.3) sorted
    descending (tok, prob [D][Wf][m]); and the mid drafter's probability of
    the edge into every node, by creation index (q [n_nodes], U(0.05, 1))."""
    tok = np.stack([np.stack([_distinct_tokens(r, V, m) for _ in range(Wf)]) for _ in range(D)]).astype(np.int32)
    prob = np.sort(r.dirichlet(np.full(m, 0.3), (D, Wf)), axis=-1)[..., ::-1].astype(np.float32).copy()
    q = r.uniform(0.05, 1.0, n_nodes).astype(np.float32)
    return tok, prob, q


def random_tree(r: np.random.Generator, V: int, N: int, root_token: int,
                max_depth: int = 4, max_children: int = 3):
    """Small random parent array: node i hangs under a uniformly chosen
    earlier node of depth < max_depth with fewer than max_children children.
    Scores are products of uniform(0.05, 1) edge factors."""
    parent = [-1]
    depth = [0]
    nchild = [0]
    token = [root_token]
    score = [1.0]
    kids: dict[int, set[int]] = {0: set()}
    for i in range(1, N):
        ok = [j for j in range(i) if depth[j] < max_depth and nchild[j] < max_children]
        p = ok[int(r.integers(0, len(ok)))]
        t = int(r.integers(0, V))
        while t in kids[p]:
            t = int(r.integers(0, V))
        kids[p].add(t)
        kids[i] = set()
        parent.append(p)
        depth.append(depth[p] + 1)
        nchild.append(0)
        nchild[p] += 1
        token.append(t)
        score.append(score[p] * float(r.uniform(0.05, 1.0)))
    return (np.array(parent, np.int32), np.array(token, np.int32),
            np.array(score, np.float64).astype(np.float32))


# ----------------------------------------------------------------------------
# successor-table initialisation (stand-in for the pages' warm-up)
# ----------------------------------------------------------------------------

def _zipf_cdf(V: int, s: float = 1.1) -> np.ndarray:
    w = np.arange(1, V + 1, dtype=np.float64) ** (-s)
    c = np.cumsum(w)
    return c / c[-1]


def zipf_ids(r: np.random.Generator, cdf: np.ndarray, size) -> np.ndarray:
    u = r.random(size)
    return np.minimum(np.searchsorted(cdf, u, side="right"), len(cdf) - 1).astype(np.int32)


def zipf_table(r: np.random.Generator, V: int, k: int, s: float = 1.1) -> np.ndarray:
    """[V, k] int32: every row holds k distinct ids drawn from Zipf(s) over
    ranks 1..V (id = rank - 1), repeats rejected, in draw order."""
    cdf = _zipf_cdf(V, s)
    M = 4 * k
    cand = zipf_ids(r, cdf, (V, M))
    order = np.argsort(cand, axis=1, kind="stable")
    sc = np.take_along_axis(cand, order, 1)
    dup_s = np.zeros(sc.shape, bool)
    dup_s[:, 1:] = sc[:, 1:] == sc[:, :-1]
    dup = np.empty_like(dup_s)
    np.put_along_axis(dup, order, dup_s, 1)
    first = ~dup
    cnt = np.cumsum(first, axis=1)
    table = np.empty((V, k), np.int32)
    short = cnt[:, -1] < k
    okrows = np.nonzero(~short)[0]
    sel = first[okrows] & (cnt[okrows] <= k)
    table[okrows] = cand[okrows][sel].reshape(-1, k)
    for v in np.nonzero(short)[0]:
        row: list[int] = []
        while len(row) < k:
            t = int(zipf_ids(r, cdf, 1)[0])
            if t not in row:
                row.append(t)
        table[v] = row
    return table


def context_tokens(r: np.random.Generator, L: int, V: int, span: int = 8, p_copy: float = 0.3):
    """Token context built from `span`-token spans: with probability p_copy a
    span repeats the tokens at a uniformly chosen earlier offset, otherwise
    it is fresh Zipf(1.1) tokens."""
    cdf = _zipf_cdf(V)
    out = np.empty(L, np.int32)
    t = 0
    while t < L:
        n = min(span, L - t)
        if t >= span and r.random() < p_copy:
            o = int(r.integers(0, t - span + 1))
            out[t:t + n] = out[o:o + n]
        else:
            out[t:t + n] = zipf_ids(r, cdf, n)
        t += n
    return out


def warm_table_from_context(table: np.ndarray, ctx: np.ndarray) -> np.ndarray:
    """Stand-in warm-up: walk the context left to right and move each
    observed successor to the front of its predecessor's row (distinct,
    truncated to the row width)."""
    table = table.copy()
    k = table.shape[1]
    for a, b in zip(ctx[:-1].tolist(), ctx[1:].tolist()):
        row = table[a].tolist()
        if b in row:
            row.remove(b)
        table[a] = ([b] + row)[:k]
    return table


# ----------------------------------------------------------------------------
# one round's inputs
# ----------------------------------------------------------------------------

class RoundInputs:
    """Host arrays for one verify round (all numpy)."""

    def __init__(self, **kw):
        self.__dict__.update(kw)


def _normal_bf16(r: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = r.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_bf16_bits(x)


def make_round_inputs(wl: Workload, kv: bool = True, extra_slots: int = 0) -> RoundInputs:
    """extra_slots: cache slots per (request, KV head) beyond ctx_hi + N, for
    chained rounds whose context grows."""
    cfg = wl.cfg
    B, N, k, V = wl.B, wl.n_nodes, wl.k, wl.V
    rc = rng(cfg, "ctx_len")
    if wl.ctx_lo == wl.ctx_hi:
        ctx_len = np.full(B, wl.ctx_lo, np.int32)
    else:
        ctx_len = rc.integers(wl.ctx_lo, wl.ctx_hi + 1, size=B).astype(np.int32)

    table = zipf_table(rng(cfg, "table"), V, k)
    ctx_tok = None
    if wl.ctx_tokens:
        ctx_tok = context_tokens(rng(cfg, "context"), int(ctx_len[0]), V)
        table = warm_table_from_context(table, ctx_tok)

    cp, ct, cs, coff, roots, tg_out = [], [], [], [0], [], []
    for b in range(B):
        rb = rng(cfg, f"draft/{b}")
        root = int(ctx_tok[-1]) if ctx_tok is not None else int(rb.integers(0, V))
        if wl.tree == "treegraft":
            # drafter outputs only: the candidate tree is what the method builds
            tg_out.append(treegraft_drafter_outputs(rb, V, wl.D, wl.Wf, wl.m, 1 + wl.D * wl.Wf * wl.m))
            roots.append(root)
            continue
        elif wl.tree == "random":
            p, t, s = random_tree(rb, V, N, root)
        elif wl.tree == "block":
            p, t, s = block_draft(rb, V, N - 1, root)
        else:
            p, t, s = eagle_candidates(rb, V, wl.D, wl.Wf, wl.m, root)
        cp.append(p); ct.append(t); cs.append(s)
        coff.append(coff[-1] + len(p))
        roots.append(root)

    # previous round's verified nodes: tokens (Zipf, so repeats occur) and
    # their k distinct successor ids
    rp = rng(cfg, "prev_round")
    cdf = _zipf_cdf(V)
    prev_n = np.full(B, N, np.int32)
    prev_row_off = (np.arange(B + 1) * N).astype(np.int32)
    prev_token = zipf_ids(rp, cdf, B * N)
    prev_topk = np.empty((B * N, k), np.int32)
    for i in range(B * N):
        prev_topk[i] = _distinct_tokens(rp, V, k)

    ri = RoundInputs(
        wl=wl, B=B, N=N, k=k, V=V,
        ctx_len=ctx_len, ctx_tokens=ctx_tok,
        cand_parent=np.concatenate(cp) if cp else None, cand_token=np.concatenate(ct) if ct else None,
        cand_score=np.concatenate(cs) if cs else None, cand_off=np.array(coff, np.int32) if cp else None,
        root_token=np.array(roots, np.int32),
        budget=np.full(B, wl.draft_budget, np.int32),
        n_ret=np.full(B, wl.n_retrieved, np.int32),
        stage=None,
        row_off=(np.arange(B + 1) * N).astype(np.int32),
        table=table,
        prev_n=prev_n, prev_row_off=prev_row_off, prev_token=prev_token, prev_topk=prev_topk,
        scale=float(1.0 / np.sqrt(wl.d)),
    )
    if wl.stages:  # per-request checkpoint: budget and retrieved count from Graft's split
        ri.stage = np.array([wl.stages[b % len(wl.stages)] for b in range(B)], np.int32)
        ri.budget = np.array([STAGE_SLOTS[int(s)][0] for s in ri.stage], np.int32)
        ri.n_ret = np.array([STAGE_SLOTS[int(s)][1] for s in ri.stage], np.int32)
    if tg_out:  # TreeGraft: per request tok [D][W][m], prob [D][W][m], q [1 + D*W*m]
        ri.tg_mask = np.full(B, wl.mid_mask, np.int32)
        ri.tg_tok = np.stack([o[0] for o in tg_out])
        ri.tg_prob = np.stack([o[1] for o in tg_out])
        ri.tg_q = np.stack([o[2] for o in tg_out])
    if kv:
        make_qkv(ri, extra_slots)
    return ri


def make_qkv(ri: RoundInputs, extra_slots: int = 0) -> None:
    """Q [B*N, Hq, d] and K/V caches laid out [B][Hkv][cap][d] with
    cap = ctx_hi + N + extra_slots; request b's tree keys sit at slots
    ctx_b .. ctx_b+N-1.  Slots past ctx_b + N are zero."""
    wl = ri.wl
    cfg = wl.cfg
    B, N = ri.B, ri.N
    cap = wl.ctx_hi + N + extra_slots
    ri.kv_cap = cap
    ri.kv_head_stride = cap * wl.d
    ri.kv_off = (np.arange(B, dtype=np.int64) * wl.Hkv * cap * wl.d)
    ri.q = _normal_bf16(rng(cfg, "q"), (B * N, wl.Hq, wl.d))
    kc = np.zeros((B, wl.Hkv, cap, wl.d), np.uint16)
    vc = np.zeros((B, wl.Hkv, cap, wl.d), np.uint16)
    for b in range(B):
        L = int(ri.ctx_len[b]) + N
        kc[b, :, :L] = _normal_bf16(rng(cfg, f"k/{b}"), (wl.Hkv, L, wl.d))
        vc[b, :, :L] = _normal_bf16(rng(cfg, f"v/{b}"), (wl.Hkv, L, wl.d))
    ri.kcache = kc
    ri.vcache = vc


def gumbel_noise(cfg: int, name: str, shape) -> np.ndarray:
    """Seeded i.i.d. Gumbel(0, 1) noise, fp32: -log(-log(u)) of uniforms
    drawn in fp64 (the random input of sampling at temperature T > 0)."""
    u = rng(cfg, f"gumbel/{name}").random(shape)
    u = np.clip(u, 1e-300, 1.0 - 1e-16)
    return (-np.log(-np.log(u))).astype(np.float32)


# ----------------------------------------------------------------------------
# lm-head weights and planted hidden states
# ----------------------------------------------------------------------------

def _w_block(wl: Workload, blk: int) -> np.ndarray:
    r0 = blk * W_BLOCK_ROWS
    r1 = min(wl.V, r0 + W_BLOCK_ROWS)
    return _normal_bf16(rng(wl.cfg, f"w/{blk}"), (r1 - r0, wl.H), std=0.02)


def make_lm_weights(wl: Workload) -> np.ndarray:
    """lm-head weight [V, H] bf16 bits, N(0, 0.02), drawn in blocks of
    4096 rows so any row can be regenerated alone."""
    nb = (wl.V + W_BLOCK_ROWS - 1) // W_BLOCK_ROWS
    return np.concatenate([_w_block(wl, b) for b in range(nb)], axis=0)


def make_weight_rows(wl: Workload, rows) -> np.ndarray:
    """The selected rows of make_lm_weights(wl), without drawing the rest."""
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((len(rows), wl.H), np.uint16)
    for blk in np.unique(rows // W_BLOCK_ROWS):
        sel = np.nonzero(rows // W_BLOCK_ROWS == blk)[0]
        wb = _w_block(wl, int(blk))
        out[sel] = wb[rows[sel] - blk * W_BLOCK_ROWS]
    return out


def plant_hidden(wl: Workload, weight_rows, parent: np.ndarray, token: np.ndarray,
                 n: np.ndarray, row_off: np.ndarray, p_plant: float = 0.7,
                 boost: float = 6.0):
    """Hidden states [rows, H] bf16 for the verified tree nodes.

    Every row is N(0,1).  With probability p_plant a node gets a planted
    peak: a target token t (the token of a uniformly chosen child when the
    node has children, else a uniform token) and hidden += c * W[t] with
    c = boost / |W[t]|^2, which raises that row's logit at t by `boost`
    (up to the bf16 rounding of the hidden state).  `weight_rows(ids)`
    returns the bf16 rows of W for the given ids.

    Returns (hidden_bits, planted_token) with planted_token = -1 where no
    peak was planted."""
    r = rng(wl.cfg, "hidden")
    rows = int(row_off[-1])
    z = r.standard_normal((rows, wl.H), dtype=np.float32).astype(np.float64)
    planted = np.full(rows, -1, np.int64)
    B = len(n)
    for b in range(B):
        o = int(row_off[b])
        nb = int(n[b])
        kids: dict[int, list[int]] = {}
        for i in range(1, nb):
            kids.setdefault(int(parent[o + i]), []).append(i)
        for i in range(nb):
            if r.random() < p_plant:
                ch = kids.get(i)
                if ch:
                    planted[o + i] = int(token[o + ch[int(r.integers(0, len(ch)))]])
                else:
                    planted[o + i] = int(r.integers(0, wl.V))
    sel = np.nonzero(planted >= 0)[0]
    if len(sel):
        wr = bf16_bits_to_f32(weight_rows(planted[sel])).astype(np.float64)
        c = boost / np.sum(wr * wr, axis=1)
        z[sel] += c[:, None] * wr
    return f32_to_bf16_bits(z.astype(np.float32)), planted
