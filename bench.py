#!/usr/bin/env python3
"""Benchmark of the DSA decode step (indexer + top-k + sparse MLA attention) on one MI355X.

Workload (default): decode_128k, one query row over a 131072-position cache, 64 fp8 indexer heads of width
64, top-k 2048, 128 bf16 attention heads over a 512-wide latent.  Inputs are seeded synthetic data already
resident in HBM; the timed loop rotates through enough distinct input copies that the 256 MiB Infinity
Cache cannot serve one step's bytes to a later step.

Prints one JSON line.  `value` = query rows completed per second of wall time (torch.cuda.synchronize()
on both sides of exactly --steps steps).  `roofline` = the indexer kernel (the dominant one) against the
8 TB/s HBM peak: algorithmic bytes per launch over its mean launch time, from HIP events on its stream.
`cpu_baseline` = the fp64 CPU oracle timed on this host over a bounded sample of the same workload.

`--crossover` instead times the sparse step against dense attention over every visible position
(dsa_dense_mla_attn) for one query row at a range of context lengths, one JSON line per length: the short-context
fallback's break-even on this GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP8_MFMA_PEAK_TFLOPS = 5000.0  # dense OCP fp8 MFMA, MI355X
METRIC = "DSA decode queries/s @T=128K, k=2048 (indexer+topk+attn); % HBM roofline"
METRIC_PREFILL = "DSA chunked-prefill query rows/s (indexer+topk+attn); indexer % fp8 MFMA peak"
PMC_FILE = os.path.join(ROOT, "profiles", "indexer_decode_128k_pmc.json")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("indexer.hip", "common.h"):
        with open(os.path.join(ROOT, "long_context_sparse_indexer_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per indexer launch from the committed counter run, if it was taken on the current kernel."""
    try:
        with open(PMC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def crossover(lengths, rows: int, steps: int) -> int:
    """Sparse step vs dense attention, one JSON line per context length (graph replay, rotated inputs)."""
    import numpy as np
    import torch

    import long_context_sparse_indexer_amd as dsa
    from long_context_sparse_indexer_amd import cost
    import synth
    from synth.device import upload

    dev = torch.device("cuda:0")
    names = ["q_idx", "q_idx_scale", "head_w", "k_idx_pool", "k_idx_scale", "q", "kv_pool"]
    for n in lengths:
        prob = synth.make_problem(synth.get("decode_128k", lengths=[n] * rows, seed=7))
        base = upload(prob, dev)
        P = dsa.make_problem(**base.fields)
        L = dsa.make_layout(base.row_seq, base.row_len, base.page_table)
        sparse_bytes = cost.decode_row_bytes(n, prob.k, prob.H_I, prob.d_I, prob.H, prob.d_c)
        touched = rows * max(sparse_bytes, n * prob.d_c * 2)
        copies = max(2, min(32, int(np.ceil(3 * 256e6 / touched))))
        sets = [{m: getattr(base, m) for m in names}] + [{m: getattr(base, m).clone() for m in names}
                                                         for _ in range(copies - 1)]
        idx = torch.empty((prob.R, prob.k), dtype=torch.int32, device=dev)
        out = torch.empty((prob.R, prob.H, prob.d_c), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((prob.R, prob.H), dtype=torch.float32, device=dev)
        ws_bytes = max(dsa.dsa_workspace_bytes(P, dsa.DSA_OP_STEP), dsa.dsa_workspace_bytes(P, dsa.DSA_OP_DENSE))
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

        def sparse(s, st):
            dsa.dsa_decode_step(P, L, s["q_idx"], s["q_idx_scale"], s["head_w"], s["k_idx_pool"], s["k_idx_scale"],
                                s["q"], s["kv_pool"], idx, out, lse, ws, st)

        def dense(s, st):
            dsa.dsa_dense_mla_attn(P, L, s["q"], s["kv_pool"], out, lse, ws, st)

        res = {}
        for mode, fn in (("sparse", sparse), ("dense", dense)):
            for s in sets:
                fn(s, torch.cuda.current_stream().cuda_stream)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for s in sets:
                    fn(s, torch.cuda.current_stream().cuda_stream)
            reps = max(1, steps // copies)
            for _ in range(2):
                g.replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(reps):
                g.replay()
            torch.cuda.synchronize()
            res[mode] = (time.perf_counter() - t0) * 1e6 / (reps * copies)
        print(json.dumps({"crossover": True, "context": n, "rows": rows, "k": prob.k,
                          "sparse_us": round(res["sparse"], 2), "dense_us": round(res["dense"], 2),
                          "faster": "dense" if res["dense"] < res["sparse"] else "sparse",
                          "input_copies": copies}), flush=True)
        del base, sets, ws
        torch.cuda.empty_cache()
    return 0


def append_sweep(steps: int) -> int:
    """Indexer-key append (bf16 latent rows x W_KI -> e4m3 codes + scale), one JSON line per (tokens, d_I): graph
    replay of one call on the same inputs, which the preceding kernels of a layer would have left in cache."""
    import numpy as np
    import torch

    import long_context_sparse_indexer_amd as dsa
    import synth
    from synth.device import upload

    dev = torch.device("cuda:0")
    for d_I in (128, 64):
        for rows in (1, 64, 4096):
            prob = synth.make_problem(synth.get("prefill_chunk", cache_len=8192, rows=rows, H=16, d_I=d_I, seed=9))
            app = synth.append_inputs(prob, 9)
            d = upload(prob, dev)
            P = dsa.make_problem(**d.fields)
            L = dsa.make_layout(d.row_seq, d.row_len, d.page_table)
            pos = torch.from_numpy(app["positions"]).to(dev)
            c = torch.from_numpy(app["c"].view(np.int16)).to(dev)
            w = torch.from_numpy(app["w"].view(np.int16)).to(dev)
            pool, scale = d.k_idx_pool.clone(), d.k_idx_scale.clone()

            def call():
                dsa.dsa_indexer_key_append(P, L, pos, c, w, pool, scale, torch.cuda.current_stream().cuda_stream)
            call()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(10):
                    call()
            reps = max(1, steps // 10)
            g.replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(reps):
                g.replay()
            torch.cuda.synchronize()
            us = (time.perf_counter() - t0) * 1e6 / (reps * 10)
            flops = 2.0 * rows * prob.d_c * d_I
            print(json.dumps({"append": True, "tokens": rows, "d_c": prob.d_c, "d_I": d_I, "us_per_call": round(us, 2),
                              "tokens_per_s": round(rows / us * 1e6, 1),
                              "fp64_tflops": round(flops / us * 1e-6, 3), "fp64_peak_tflops": 78.6}), flush=True)
            del d, pool, scale
            torch.cuda.empty_cache()
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="decode_128k",
                    choices=["decode_128k", "batched_paged", "decode_1m", "prefill_chunk", "decode_128k_di128",
                             "decode_128k_fp8kv", "prefill_chunk_di128", "batched_paged_fp8kv"])
    ap.add_argument("--copies", type=int, default=0, help="distinct input copies to rotate (0 = auto)")
    ap.add_argument("--phase-iters", type=int, default=400)
    ap.add_argument("--graph", dest="graph", action="store_true", default=True,
                    help="replay the step loop from a captured HIP graph (default)")
    ap.add_argument("--no-graph", dest="graph", action="store_false", help="launch every step from the host")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--crossover", action="store_true",
                    help="time the sparse step against dense attention over context lengths, then exit")
    ap.add_argument("--crossover-rows", type=int, default=1)
    ap.add_argument("--append", action="store_true",
                    help="time the indexer-key append for 1, 64 and 4096 tokens at d_I = 128 and 64, then exit")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the run, copy a buffer of this many MiB 4 times (reference dispatches for byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (see the sharding design); "
              "run with --gpus 1", file=sys.stderr)
        return 2
    if args.crossover:
        return crossover([2048, 4096, 8192, 16384, 32768, 65536, 131072], args.crossover_rows, min(args.steps, 400))
    if args.append:
        return append_sweep(min(args.steps, 1000))

    import numpy as np
    import torch

    import long_context_sparse_indexer_amd as dsa
    from long_context_sparse_indexer_amd import cost
    import synth
    from synth.device import upload

    torch.cuda.init()
    dev = torch.device("cuda:0")
    cfg = synth.get(args.workload)
    t0 = time.perf_counter()
    prob = synth.make_problem(cfg)
    base = upload(prob, dev)
    gen_s = time.perf_counter() - t0
    P = dsa.make_problem(**base.fields)
    L = dsa.make_layout(base.row_seq, base.row_len, base.page_table)

    # distinct copies of every per-step input, enough to exceed the 256 MiB Infinity Cache several times
    prefill = prob.rows_per_seq > 1
    touched = sum(cost.decode_row_bytes(int(n), prob.k, prob.H_I, prob.d_I, prob.H, prob.d_c,
                                        fp8_entries=prob.kv_dtype == "f8") for n in prob.row_len)
    copies = args.copies or (2 if prefill else max(2, min(64, int(np.ceil(3 * 256e6 / touched)))))
    names = ["q_idx", "q_idx_scale", "head_w", "k_idx_pool", "k_idx_scale", "q", "kv_pool"]
    sets = [{n: getattr(base, n) for n in names}]
    for _ in range(copies - 1):
        sets.append({n: getattr(base, n).clone() for n in names})
    R = prob.R
    ws = torch.empty(dsa.dsa_workspace_bytes(P, dsa.DSA_OP_STEP), dtype=torch.uint8, device=dev)
    idx = torch.empty((R, prob.k), dtype=torch.int32, device=dev)
    out = torch.empty((R, prob.H, prob.d_c), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((R, prob.H), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream

    def step(i):
        s = sets[i % copies]
        dsa.dsa_decode_step(P, L, s["q_idx"], s["q_idx_scale"], s["head_w"], s["k_idx_pool"], s["k_idx_scale"],
                            s["q"], s["kv_pool"], idx, out, lse, ws, sptr)

    graph = None
    if args.graph:
        # one graph walks every copy once; replays continue the rotation
        for i in range(copies):
            step(i)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(copies):
                s = sets[i]
                dsa.dsa_decode_step(P, L, s["q_idx"], s["q_idx_scale"], s["head_w"], s["k_idx_pool"],
                                    s["k_idx_scale"], s["q"], s["kv_pool"], idx, out, lse, ws,
                                    torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()

    def run(n_steps, offset=0):
        if graph is None:
            for i in range(n_steps):
                step(offset + i)
        else:
            for _ in range(n_steps // copies):
                graph.replay()
            for i in range(n_steps % copies):
                step(offset + i)

    run(args.warmup)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    run(args.steps, args.warmup)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    gpu_s = ev0.elapsed_time(ev1) / 1e3
    qps = args.steps * R / wall

    # per-phase mean launch times: each phase alone, back to back over the rotated copies, HIP events on the
    # stream the kernels run on
    ld = ((max(prob.max_row_len, 1) + 63) // 64) * 64
    scores = torch.empty((R, ld), dtype=torch.float32, device=dev)

    def timed(fn, iters):
        for i in range(min(iters, 20)):
            fn(i)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(iters):
            fn(i)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / iters  # microseconds per launch

    def ph_indexer(i):
        s = sets[i % copies]
        dsa.dsa_indexer_scores(P, L, s["q_idx"], s["q_idx_scale"], s["head_w"], s["k_idx_pool"], s["k_idx_scale"],
                               scores, ld, sptr)

    topk_ws = torch.empty(dsa.dsa_workspace_bytes(P, dsa.DSA_OP_TOPK), dtype=torch.uint8, device=dev)
    attn_ws = torch.empty(max(256, dsa.dsa_workspace_bytes(P, dsa.DSA_OP_ATTN)), dtype=torch.uint8, device=dev)

    def ph_topk(i):
        dsa.dsa_topk(P, L, scores, idx, topk_ws, ld, sptr)

    def ph_attn(i):
        s = sets[i % copies]
        dsa.dsa_sparse_mla_attn(P, L, s["q"], s["kv_pool"], idx, out, lse, attn_ws, sptr)

    us_idx = timed(ph_indexer, args.phase_iters)
    us_topk = timed(ph_topk, args.phase_iters)
    us_attn = timed(ph_attn, args.phase_iters)

    idx_bytes = sum(cost.indexer_row_bytes(int(n), prob.H_I, prob.d_I) for n in prob.row_len)
    idx_flops = sum(cost.indexer_row_flops(int(n), prob.H_I, prob.d_I) for n in prob.row_len)
    if prefill:
        # rows of one sequence share their keys: the tiled indexer is a GEMM, priced against the fp8 MFMA peak
        achieved = idx_flops / (us_idx * 1e-6) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": FP8_MFMA_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / FP8_MFMA_PEAK_TFLOPS, 4), "traffic": None,
                    "kernel": "indexer_f8_tiled_kernel", "flops_per_launch": idx_flops,
                    "us_per_launch": round(us_idx, 3)}
    else:
        achieved = idx_bytes / (us_idx * 1e-6) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": measured_traffic() if args.workload == "decode_128k" else None,
                    "kernel": "indexer_f8_kernel", "bytes_per_launch": idx_bytes, "us_per_launch": round(us_idx, 3)}
    step_bytes = touched
    result = {
        "metric": METRIC_PREFILL if prefill else METRIC,
        "value": round(qps, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3-indexer/fp8e4m3-latent-bf16-attention" if prob.kv_dtype == "f8"
                 else "fp8e4m3-indexer/bf16-attention",
        "data": "synthetic",
        "config": {"workload": args.workload, "rows": R, "context": int(prob.max_row_len), "k": prob.k,
                   "H_I": prob.H_I, "d_I": prob.d_I, "H": prob.H, "d_c": prob.d_c, "page_size": prob.page_size,
                   "input_copies": copies, "graph": bool(args.graph)},
        "roofline": roofline,
        "end_to_end": {"algorithmic_bytes_per_step": step_bytes,
                       "hbm_frac": round(step_bytes / (wall / args.steps) / (HBM_PEAK_GBS * 1e9), 4),
                       "gpu_event_ms_per_step": round(gpu_s / args.steps * 1e3, 5)},
        "phases_us": {"indexer": round(us_idx, 3), "topk": round(us_topk, 3), "attention": round(us_attn, 3)},
        "gen_seconds": round(gen_s, 2),
    }

    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["calib_copy_bytes"] = n
        del src, dst

    if not args.no_cpu_baseline:
        import copy
        import oracle
        # bounded sample: consecutive groups of up to 8 rows of the same workload, until the time is spent
        chunk = min(R, 8)
        rows_done, reps, t_c = 0, 0, time.perf_counter()
        while True:
            rows = (np.arange(chunk) + reps * chunk) % R
            sub = copy.copy(prob)
            sub.R = chunk
            for name in ("q_idx", "q_idx_scale", "head_w", "q", "row_seq", "row_len"):
                a = getattr(prob, name)
                setattr(sub, name, None if a is None else np.ascontiguousarray(a[rows]))
            oracle.decode_step(sub)
            reps += 1
            rows_done += chunk
            el = time.perf_counter() - t_c
            if el >= args.cpu_seconds or reps >= 1000:
                break
        result["cpu_baseline"] = {"value": round(rows_done / el, 3), "unit": "queries/s", "cores": oracle.threads(),
                                  "kind": "oracle",
                                  "sample": f"{rows_done} query rows of {args.workload} in {reps} call(s) of "
                                            f"{chunk} row(s), fp64 oracle, {el:.1f} s"}
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
