"""Shared set-up for the GPU round tests: seeded inputs, the oracle's tree
stage, planted hidden states (planted on the oracle's tree), and one GPU
round through the C ABI."""
from __future__ import annotations

import functools
import sys

import numpy as np

from oracle import round as OR
from synth import workloads as W

# |gpu - ref| <= ATOL + RTOL * |ref| for floating-point outputs
ATOL, RTOL = 2e-2, 1e-2


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=1)
def prepared(cfg: int):
    wl = W.WORKLOADS[cfg]
    say(f"[inputs] cfg {cfg}: {wl.name}")
    ri = W.make_round_inputs(wl)
    w = W.make_lm_weights(wl)
    ts = OR.tree_stage(ri)
    tree = ts["tree"]
    hidden, planted = W.plant_hidden(wl, lambda ids: w[ids], tree["parent"], tree["token"],
                                     tree["n"], ri.row_off)
    return wl, ri, w, ts, hidden


def run_gpu_round(cfg: int, fused: bool = False):
    import torch

    from draft_tree_verification_parent_amd.verify_round import VerifyRound
    wl, ri, w, ts, hidden = prepared(cfg)
    say(f"[gpu] cfg {cfg}: one round through libgraft ({'fused' if fused else 'split'} lm-head/top-k)")
    vr = VerifyRound(ri, w, fused=fused)
    vr.set_hidden(hidden)
    vr.run()
    torch.cuda.synchronize()
    say(f"[gpu] cfg {cfg}: round done")
    return wl, ri, w, ts, hidden, vr


def bf16_tensor_to_f64(t):
    import torch
    return t.float().cpu().numpy().astype(np.float64)


def within_tol(got, ref):
    err = np.abs(got - ref)
    bound = ATOL + RTOL * np.abs(ref)
    return bool(np.all(err <= bound)), float(err.max()) if err.size else 0.0
