"""Benchmark: one verify round of tree speculative decoding on one MI355X.

A step is one whole round through libgraft on one HIP stream (table update
+ retrieval, tree build, one tree-attention layer, lm-head, top-k,
acceptance).  The headline workload is the batched static-tree round: 16
requests with Qwen3-8B shapes (32 q / 8 kv heads, d 128, per-request
context uniform in [4096, 16384]), each a 60-slot tree whose draft nodes of
cumulative score < 0.05 are replaced from a shared 151936 x 8 successor
table; lm-head 4096 x 151936 over the 960 tree rows.  The Llama-3.1-8B
batch-1 round (context 4096, 8 draft + 52 retrieved nodes, lm-head
4096 x 128256) is measured after it and reported under "batch1_llama8b".

Inputs are seeded synthetic data resident in HBM before timing; each round's
table update reads the previous round's verified nodes, as in decoding.
Consecutive rounds are captured once as a HIP graph (up to 8 chained rounds
per graph) and replayed for the throughput figure; one round per graph is
timed beside it, and the same rounds issued eagerly give the per-step times
(HIP events on the stream the kernels run on).

Prints one JSON line: verified tree tokens/s (B*N per round / round time),
round latency, per-step times, the dominant kernel's roofline fraction
(the batched lm-head against the dense bf16 MFMA peak; the batch-1 lm-head
against HBM), and the oracle timed on host cores.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--cfg 5] [--cfg2 2]
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import resource
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0  # dense bf16
METRIC = "verify-round latency (µs) & verified tree tokens/s; % MFMA / HBM roofline"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "lmhead_traffic.json")
LMHEAD_SRCS = [os.path.join(ROOT, "draft_tree_verification_parent_amd", "csrc", n)
               for n in ("lmhead.hip", "topk.hip", "topk_list.h")]
CPU_SAMPLE_REQUESTS = 2  # requests of a batched workload the oracle is timed on


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def lmhead_source_hash():
    """SHA-256 (first 16 hex digits) of the sources of one graft_lmhead_topk
    call's kernels: the lm-head kernels, the top-k merge and their shared
    key lists, read in that order."""
    h = hashlib.sha256()
    for path in LMHEAD_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload_key):
    """HBM bytes per lm-head launch from the committed rocprofv3 counter
    summary, or None when it is missing or the kernel changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(workload_key)
    if not e or e.get("kernel_source_sha256_16") != lmhead_source_hash():
        return None
    return e.get("bytes_per_launch")


def cpu_baseline(ri, w, hidden_tree_fn, budget_s=15.0):
    """The oracle, as it stands, on the host.  Batch-1 workloads: whole
    rounds until about budget_s seconds have run.  Batched workloads: one
    round of the first CPU_SAMPLE_REQUESTS requests (the tree stage for the
    whole batch, then attention, lm-head, top-k and acceptance for those
    requests' rows); the oracle's cost is per request, so the sample's
    tokens/s is the batch's.  `cores` is the CPU time the run used divided
    by its wall time: the cores it kept busy on average."""
    from threadpoolctl import threadpool_info

    from oracle import accept as OAcc
    from oracle import attention as OA
    from oracle import lmhead as OL
    from oracle import round as OR
    from oracle import topk as OT

    def cpu_s():
        u = resource.getrusage(resource.RUSAGE_SELF)
        return u.ru_utime + u.ru_stime

    c0 = cpu_s()
    t0 = time.perf_counter()
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    if ri.B == 1:
        rounds = 0
        while True:
            ts = OR.tree_stage(ri)
            hidden = hidden_tree_fn(ts["tree"])
            OR.verify_stage(ri, ts["tree"], hidden, w)
            rounds += 1
            el = time.perf_counter() - t0
            if el >= budget_s or el / rounds * (rounds + 1) > 2.5 * budget_s:
                break
        tokens = ri.B * ri.N * rounds
        what = f"{rounds} whole round(s) of the workload (same inputs)"
    else:
        nb = min(CPU_SAMPLE_REQUESTS, ri.B)
        rounds = 0
        while True:
            ts = OR.tree_stage(ri)
            tree = ts["tree"]
            hidden = hidden_tree_fn(tree)
            q = OL.bf16_to_f64(ri.q).reshape(ri.q.shape)
            Ks, Vs = [None] * ri.B, [None] * ri.B
            for b in range(nb):
                Ks[b], Vs[b] = OR.kv_f64(ri, b)
            nodes = [(b, i) for b in range(nb) for i in range(int(tree["n"][b]))]
            OA.tree_attention(q, Ks, Vs, ri.ctx_len, tree["n"], ri.row_off, tree["mask"], ri.scale, nodes=nodes)
            r1 = int(ri.row_off[nb])
            logits = OL.logits(hidden[:r1], w)
            ids, _ = OT.topk(logits, ri.k)
            OAcc.accept_batch(tree["n"][:nb], ri.row_off[:nb + 1], tree["parent"][:r1], tree["token"][:r1],
                              ids[:, 0])
            rounds += 1
            el = time.perf_counter() - t0
            if el >= budget_s or el / rounds * (rounds + 1) > 2.5 * budget_s:
                break
        tokens = ri.N * nb * rounds
        what = (f"{rounds} round(s) of {nb} of the {ri.B} requests ({ri.N * nb} of {ri.B * ri.N} tree rows each: "
                f"the tree stage for the whole batch, then attention, lm-head, top-k and acceptance for those "
                f"rows), scaled per request")
    busy = (cpu_s() - c0) / el
    return dict(value=tokens / el, unit="verified tree tokens/s", cores=round(busy, 1), kind="oracle",
                sample=f"{what}, {el:.1f} s wall; {busy:.1f} cores busy on average (numpy/BLAS thread pool "
                       f"of {threads}, host nproc={os.cpu_count()})")


def graph_us(fn, calls):
    """Device time per call of `calls` back-to-back calls captured in one
    HIP graph (kernel time, not host launch time)."""
    import torch
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / calls


def measure(cfg, steps, warmup, with_cpu, extras):
    """Times `steps` rounds of workload cfg.  Returns the report dict and,
    for the CPU baseline, what it needs."""
    import torch

    from draft_tree_verification_parent_amd import api
    from draft_tree_verification_parent_amd.verify_round import VerifyRound
    from synth import workloads as W

    wl = W.WORKLOADS[cfg]
    log(f"[bench] cfg {cfg}: generating inputs: {wl.name}")
    ri = W.make_round_inputs(wl)
    w = W.make_lm_weights(wl)
    vr = VerifyRound(ri, w)

    # the synthetic target model plants its hidden states on the built tree
    def plant(tree):
        return W.plant_hidden(wl, lambda ids: w[ids], tree["parent"], tree["token"], tree["n"],
                              ri.row_off)[0]

    vr.build_only()
    torch.cuda.synchronize()
    tree0 = vr.tree_host()
    vr.set_hidden(plant(tree0))
    vr.table.copy_(torch.from_numpy(ri.table).cuda())

    log(f"[bench] cfg {cfg}: warmup {warmup} rounds")
    for _ in range(warmup):
        vr.run()
        vr.chain_update()
    torch.cuda.synchronize()
    if vr.err.item() != 0:
        raise SystemExit(f"device error flag {vr.err.item()}")

    # Throughput: consecutive rounds captured once as a HIP graph (the steady
    # state: every round reads the previous round's outputs from the same
    # buffers, inside the graph as across replays) and replayed, so host
    # launch overhead stays out of the rounds.  G rounds per graph, G the
    # largest of 8, 4, 2, 1 dividing the step count, so exactly `steps`
    # rounds are timed; each graph launch costs a fixed device-side gap,
    # which G spreads over G rounds.
    per_graph = next(g for g in (8, 4, 2, 1) if steps % g == 0)

    def timed_replays(rounds_per_graph):
        vr.capture(rounds_per_graph)
        for _ in range(max(1, warmup // rounds_per_graph)):
            vr.replay()
        torch.cuda.synchronize()
        log(f"[bench] cfg {cfg}: timing {steps} graph-replayed rounds, {rounds_per_graph} per graph")
        t0 = time.perf_counter()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(steps // rounds_per_graph):
            vr.replay()
        g1.record()
        torch.cuda.synchronize()
        wall_s = time.perf_counter() - t0
        if vr.err.item() != 0:
            raise SystemExit(f"device error flag {vr.err.item()}")
        return g0.elapsed_time(g1), wall_s

    # one round per graph first: the GPU's clocks settle while it runs
    total_ms_1, wall_1 = timed_replays(1)
    total_ms, wall = timed_replays(per_graph) if per_graph > 1 else (total_ms_1, wall_1)

    # Per-step durations (and the lm-head roofline) from the same rounds
    # issued eagerly, with HIP events on the stream the kernels run on.
    log(f"[bench] cfg {cfg}: timing {steps} eager rounds, per step")
    events = {}
    rounds = []
    torch.cuda.synchronize()
    for _ in range(steps):
        r0 = torch.cuda.Event(enable_timing=True)
        r1 = torch.cuda.Event(enable_timing=True)
        r0.record()
        vr.run(events)
        r1.record()
        rounds.append((r0, r1))
    torch.cuda.synchronize()
    round_us = np.array([a.elapsed_time(b) * 1e3 for a, b in rounds])
    step_us = {k: float(np.mean([a.elapsed_time(b) * 1e3 for a, b in v])) for k, v in events.items()}
    if vr.err.item() != 0:
        raise SystemExit(f"device error flag {vr.err.item()}")

    tokens = ri.B * ri.N
    M, H, V = vr.rows, wl.H, wl.V
    # fused lm-head + top-k: W once, hidden once, k (id, value) pairs per row out
    lm_bytes = V * H * 2 + M * H * 2 + M * ri.k * 8
    lm_flops = 2.0 * M * H * V
    lm_s = step_us["lmhead_topk"] * 1e-6
    wide = M > 64
    kk = 8 if ri.k <= 8 else 16
    # the merge takes one wavefront per row when the lm-head leaves at most 64 lists per row (four or more 256-row
    # m tiles)
    merge = "topk_merge_wave_kernel" if M > 3 * 256 else "topk_merge_kernel"
    kern = (f"lmhead_big_kernel<{kk}> + {merge}<{kk}> (one graft_lmhead_topk call, packed weights, "
            f"{M} rows, 256 x 256 tiles)" if M > 128 else
            f"lmhead_wide_kernel + topk_merge_kernel<{kk}> (one graft_lmhead_topk call, packed weights, {M} rows)"
            if wide else
            f"lmhead_packed_kernel<true,{8 if ri.k <= 8 else 16},8> + topk_merge_kernel<{8 if ri.k <= 8 else 16}> "
            f"(one graft_lmhead_topk call, packed weights)")
    traffic = measured_traffic(f"cfg{cfg}")
    if wide:  # 960 rows: a dense contraction at about 950 flop per weight byte
        tfs = lm_flops / lm_s / 1e12
        roofline = {"bound": "mfma", "achieved": round(tfs, 1), "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                    "frac": round(tfs / MFMA_BF16_PEAK_TFS, 4), "traffic": traffic, "kernel": kern,
                    "algorithmic_flops_per_launch": lm_flops, "algorithmic_bytes_per_launch": lm_bytes,
                    "hbm_frac": round(lm_bytes / lm_s / 1e9 / HBM_PEAK_GBS, 4)}
    else:  # tens of rows: a weight stream at about 60 flop per byte
        gbs = lm_bytes / lm_s / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": kern,
                    "algorithmic_bytes_per_launch": lm_bytes,
                    "mfma_frac": round(lm_flops / lm_s / 1e12 / MFMA_BF16_PEAK_TFS, 4)}

    att_keys = int(np.sum(ri.ctx_len)) + tokens
    att_bytes = 2 * att_keys * wl.Hkv * wl.d * 2 + 2 * tokens * wl.Hq * wl.d * 2
    att_flops = 4.0 * wl.Hq * wl.d * ri.N * float(np.sum(ri.ctx_len.astype(np.float64) + ri.N))
    att_us = step_us["tree_attention"]
    kernels = {"tree_attention": {"us": round(att_us, 2),
                                  "algorithmic_bytes": att_bytes, "algorithmic_flops": att_flops,
                                  "hbm_frac": round(att_bytes / (att_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                                  "mfma_frac": round(att_flops / (att_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFS, 4)}}

    # Tree attention warm: back-to-back calls on the same inputs, so the KV
    # is served from the 256 MB Infinity Cache when it fits there.  In the
    # round it is cold: the lm-head's weight stream evicts it between calls.
    att_warm = graph_us(vr.step_tree_attention, steps)
    kernels["tree_attention"].update({
        "us_warm": round(att_warm, 2),
        "note": "us: in the round (cold caches: the lm-head's weight stream evicts the KV between calls); "
                "us_warm: back-to-back calls"})

    if extras:
        # KV compaction (round chaining) on this round's accepted paths: the
        # accepted rows move within the tree slots; the context is not
        # advanced here (the next context goes to a scratch buffer), so every
        # call moves the same rows.  Algorithmic bytes: each moved K and V
        # row read once and written once.
        ctx_s = torch.empty_like(vr.ctx_len)
        root_s = torch.empty_like(vr.root_token)
        acc_len_h = vr.acc_len.cpu().numpy()
        acc_path_h = vr.acc_path.cpu().numpy()
        moved = sum(int(np.sum(acc_path_h[b, 1:acc_len_h[b] + 1] != np.arange(1, acc_len_h[b] + 1)))
                    for b in range(ri.B))
        kv_bytes = moved * wl.Hkv * wl.d * 2 * 2 * 2

        def compact():
            api.graft_kv_compact(wl.Hkv, wl.d, vr.kcache, vr.vcache, vr.kv_off, ri.kv_head_stride, vr.ctx_len,
                                 vr.n_out, vr.acc_len, vr.acc_path, vr.bonus, ctx_s, root_s, err=vr.err)
        kv_us = graph_us(compact, steps)
        kernels["kv_compact"] = {"us": round(kv_us, 2), "rows_moved": moved, "bytes": kv_bytes,
                                 "note": "round chaining step, timed on its own (not in the round)"}

        # Sampling at T = 1 (graft_lmhead_topk_sample: top-k plus one
        # Gumbel-max draw per row in the same pass over W; the noise is an
        # input, 4 B per logit), timed on its own beside the greedy pass.
        noise = torch.from_numpy(W.gumbel_noise(cfg, "bench", (M, V))).to(vr.dev)
        sws = torch.empty(api.graft_lmhead_sample_workspace_bytes(M, V, ri.k), dtype=torch.uint8, device=vr.dev)
        s_id = torch.empty(M, ri.k, dtype=torch.int32, device=vr.dev)
        s_val = torch.empty(M, ri.k, dtype=torch.float32, device=vr.dev)
        s_draw = torch.empty(M, dtype=torch.int32, device=vr.dev)

        def sample_pass():
            api.graft_lmhead_topk_sample(M, H, V, ri.k, 1.0, vr.hidden, vr.w_packed, noise, s_id, s_val, s_draw,
                                         sws)
        s_us = graph_us(sample_pass, steps)
        g_us = graph_us(vr.step_lmhead_topk, steps)
        s_bytes = lm_bytes + M * V * 4
        kernels["lmhead_topk_sample_T1"] = {
            "us": round(s_us, 2), "greedy_us_same_timing": round(g_us, 2), "bytes": s_bytes,
            "hbm_frac": round(s_bytes / (s_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "note": "temperature 1: top-k and one draw per row in one pass; timed on its own (not in the round)"}
        del noise, sws

    rep = {
        "value": round(tokens * steps / (total_ms / 1e3), 1),
        "ms_per_step": round(total_ms / steps, 4),
        "config": {"workload": wl.name, "requests": ri.B, "tree_nodes": ri.N, "lm_head_rows": M,
                   "context": int(ri.ctx_len[0]) if ri.B == 1 else [int(x) for x in ri.ctx_len],
                   "attention_layers": 1, "parallelism": "none (1 GPU)"},
        "launch": f"HIP graph of {per_graph} chained rounds, replayed {steps // per_graph} times",
        "one_round_per_graph": {"value": round(tokens * steps / (total_ms_1 / 1e3), 1),
                                "ms_per_step": round(total_ms_1 / steps, 4)},
        "round_us_eager": {"mean": round(float(round_us.mean()), 2), "median": round(float(np.median(round_us)), 2),
                           "p90": round(float(np.percentile(round_us, 90)), 2)},
        "step_us": {k: round(v, 2) for k, v in step_us.items()},
        "roofline": roofline,
        "kernels": kernels,
        "accepted_len_last_round": vr.acc_len.cpu().numpy().tolist()[:16],
        "wall_s_timed": round(wall, 3),
    }
    cpu = None
    if with_cpu:
        log(f"[bench] cfg {cfg}: timing the oracle on the host (cpu_baseline)")
        del vr
        gc.collect()
        torch.cuda.empty_cache()
        cpu = cpu_baseline(ri, w, plant)
    return rep, cpu


def topk_probe(M=960, V=151936, reps=8):
    """The top-k on materialised logits (A5 off the round's path): one
    graft_lmhead_topk call with the logits given, on seeded N(0, 1) fp32
    logits of the batched workload's shape, cold: a read of 1 GiB of other
    memory (no writes, so no dirty lines to write back) before every call.
    A plain reduction over the same logits (torch.amax, row maxima) timed
    the same way is the streaming reference."""
    import torch
    from draft_tree_verification_parent_amd import api

    g = torch.Generator(device="cuda").manual_seed(5)
    logits = torch.randn(M, V, device="cuda", generator=g)
    evict = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    out = {"workload": f"top-k of {M} x {V} fp32 logits, cold", "bytes": M * V * 4}
    for k in (8, 16):
        ids = torch.empty(M, k, dtype=torch.int32, device="cuda")
        vals = torch.empty(M, k, dtype=torch.float32, device="cuda")
        ws = torch.empty(max(api.graft_lmhead_topk_workspace_bytes(M, V, k), 16), dtype=torch.uint8, device="cuda")

        def timed(fn):
            best = float("inf")
            for _ in range(reps):
                torch.amax(evict)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                torch.cuda.synchronize()
                best = min(best, e0.elapsed_time(e1) * 1e3)
            return best

        us = timed(lambda: api.graft_lmhead_topk(M, 0, V, k, None, None, logits, ids, vals, ws))
        ref = torch.topk(logits, k, dim=1)
        out[f"k{k}"] = {"us": round(us, 1), "GB/s": round(M * V * 4 / us / 1e3, 1),
                        "hbm_frac": round(M * V * 4 / us / 1e3 / HBM_PEAK_GBS, 4),
                        "values_match_torch_topk": bool(torch.equal(vals, ref.values))}
    ref_us = timed(lambda: torch.amax(logits, dim=1))
    out["torch_amax_us"] = round(ref_us, 1)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=48)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--cfg", type=int, default=5, help="headline workload (5 = 16 requests, the largest)")
    ap.add_argument("--cfg2", type=int, default=2, help="second workload reported beside it (0 = none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--topk-probe", action="store_true",
                    help="only time the top-k of materialised logits (960 x 151936 fp32, cold)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark measures one GPU only: the verify round runs as "
                                   "one process on one GPU and no multi-GPU path is implemented",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)

    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n * 4, "launches": 5}))
        return

    if args.topk_probe:
        print(json.dumps(topk_probe()))
        return

    head, cpu = measure(args.cfg, args.steps, args.warmup, not args.no_cpu_baseline, extras=False)
    gc.collect()
    torch.cuda.empty_cache()
    second = None
    if args.cfg2:
        second, _ = measure(args.cfg2, args.steps, args.warmup, False, extras=True)

    out = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "verified tree tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; random-init lm-head weights and KV)",
        "config": head["config"],
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
    }
    for k in ("launch", "one_round_per_graph", "round_us_eager", "step_us", "kernels", "accepted_len_last_round",
              "wall_s_timed"):
        out[k] = head[k]
    if second is not None:
        out["batch1_llama8b" if args.cfg2 == 2 else f"cfg{args.cfg2}"] = second
    print(json.dumps(out))


if __name__ == "__main__":
    main()
