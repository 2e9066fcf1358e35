"""lm-head logits (oracle; test infrastructure only).

The verification pass ends in the target model's next-token distribution at
every tree position; the table update and the acceptance test both read it
(Graft page, section 2, third step).  Here that is the lm-head product

    logits[m, v] = sum_h hidden[m, h] * W[v, h]

with bf16 hidden states and weights upcast exactly to fp64, accumulated in
fp64 and rounded once to fp32.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def logits(hidden_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """hidden [M, H], W [Vs, H] (bf16 bit patterns) -> fp32 [M, Vs]."""
    h = bf16_to_f64(hidden_bits)
    w = bf16_to_f64(w_bits)
    return (h @ w.T).astype(np.float32)
