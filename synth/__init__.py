"""Seeded synthetic inputs for one round of tree speculative decoding.

This package only draws random numbers and shapes them into the input
tensors of a verify round (candidate trees from a stand-in drafter,
Q/K/V, hidden states, lm-head weights, a Zipf-initialised successor
table, the previous round's verified nodes).  It holds none of the
round's own arithmetic: no tree selection, no masks, no attention, no
top-k, no acceptance, no table update.  Both the oracle tests and the
GPU path consume exactly the bytes produced here.
"""
from .bf16 import f32_to_bf16_bits, bf16_bits_to_f32  # noqa: F401
from .workloads import WORKLOADS, Workload, RoundInputs, make_round_inputs, \
    make_lm_weights, make_weight_rows, plant_hidden  # noqa: F401
