"""Input regimes for checking attention outputs at long context.

With Q, K, V ~ N(0, 1) and scale 1/sqrt(d) the softmax over L keys is
nearly flat, so each output element is an average of about L values and its
magnitude falls like 1/sqrt(L) (about 0.006 at 64K keys).  A check whose
absolute tolerance is larger than that cannot tell a correct output from a
scaled or partial one.  The regime here keeps the outputs of order one at
any context length by shaping the inputs only:

  * every query row of KV head h of request b gets a shared direction u
    (a random unit vector): q = (z - (z . u) u) + a u, z its N(0, 1) draw;
  * n_hot context keys of that head, spread over the whole context (one per
    equal share, so they land in different key splits of a split-K kernel),
    become k = z' + c_j u with c_j evenly spaced in [c_lo, c_hi] in a random
    order.

A hot key then scores about a c_j / sqrt(d) (about 13 to 18 at d = 128 with
the defaults) against a bulk that sums to about log L + 0.6, so a few hot
keys in different splits carry most of the softmax mass and each output row
is a weighted mix of their values: the split weights must be right for the
output to be right.  No attention arithmetic is done here; only inputs are
drawn and placed.
"""
from __future__ import annotations

import numpy as np

from .bf16 import bf16_bits_to_f32, f32_to_bf16_bits
from .workloads import rng


def concentrate(cfg: int, q_bits: np.ndarray, k_bits: np.ndarray, ctx_len, row_off, Hkv: int,
                n_hot: int = 8, a: float = 4.0, c_lo: float = 36.0, c_hi: float = 50.0):
    """q_bits [rows, Hq, d] and k_bits [B, Hkv, cap, d] (bf16 bits, the
    layouts of make_round_inputs) -> new (q_bits, k_bits, hot) where hot[b][h]
    lists the hot key slots.  Request b's query rows are
    row_off[b] .. row_off[b+1]-1; its hot keys sit in [0, ctx_len[b])."""
    q = bf16_bits_to_f32(q_bits).astype(np.float64)
    kk = k_bits.copy()
    rows, Hq, d = q.shape
    G = Hq // Hkv
    B = len(ctx_len)
    hot = []
    for b in range(B):
        hb = []
        ctx = int(ctx_len[b])
        r0, r1 = int(row_off[b]), int(row_off[b + 1])
        for h in range(Hkv):
            r = rng(cfg, f"concentrate/{b}/{h}")
            u = r.standard_normal(d)
            u /= np.linalg.norm(u)
            blk = q[r0:r1, h * G:(h + 1) * G]          # [rows_b, G, d]
            blk -= (blk @ u)[..., None] * u
            blk += a * u
            slots = []
            if ctx >= n_hot:
                c = np.linspace(c_lo, c_hi, n_hot)[r.permutation(n_hot)]
                for j in range(n_hot):
                    s = int((j + r.uniform(0.2, 0.8)) * ctx / n_hot)
                    z = bf16_bits_to_f32(kk[b, h, s]).astype(np.float64)
                    kk[b, h, s] = f32_to_bf16_bits((z + c[j] * u).astype(np.float32))
                    slots.append(s)
            hb.append(slots)
        hot.append(hb)
    return f32_to_bf16_bits(q.astype(np.float32)), kk, hot
