#!/usr/bin/env python3
"""Benchmark of the DSA decode step (indexer + top-k + sparse MLA attention) on one MI355X.

Workload (default): decode_128k, one query row over a 131072-position cache, 64 fp8 indexer heads of width
64, top-k 2048, 128 bf16 attention heads over a 512-wide latent.  Inputs are seeded synthetic data already
resident in HBM; consecutive steps rotate through enough distinct input copies that the 256 MiB Infinity
Cache cannot serve one step's bytes to a later step.

Timing protocol: --warmup eager steps, then exactly --steps steps captured in one HIP graph (one untimed
replay), then --repeats timed replays, each bracketed by torch.cuda.synchronize(); the line reports the median
repeat (every repeat is listed).  `--no-graph` launches every timed step from the host instead.

Prints one JSON line.  `value` = query rows completed per second of wall time.  `roofline` = the whole step
against the 8 TB/s HBM peak: algorithmic bytes per step (SURVEY-style count: indexer keys and scales, indexer
query, gathered latent rows, attention query in and output out) over the measured time per step; its
`traffic` is the HBM bytes per step that the FETCH_SIZE / WRITE_SIZE counter runs in profiles/ measured, while
they were taken on the current kernel sources.  `phases` times each phase alone (HIP events on the launch
stream, graph-replayed) with its own algorithmic bytes.  `cpu_baseline` = the fp64 CPU oracle timed on this
host over a bounded sample of the same workload.

Other modes: `--sweep` times the step over context lengths (k = 2048) and budgets (n = 131072) and fits the
affine cost model t = a + b * n (d_I + 4) and t = a + c * k d_c 2; `--crossover` times the sparse step against
dense attention; `--append` times the indexer-key append; `--summarize-pmc DIR` / `--summarize-trace DIR`
turn rocprofv3 CSV output into the committed summaries.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP8_MFMA_PEAK_TFLOPS = 5000.0  # dense OCP fp8 MFMA, MI355X
METRIC = "DSA decode queries/s @T=128K, k=2048 (indexer+topk+attn); % HBM roofline"
METRIC_PREFILL = "DSA chunked-prefill query rows/s (indexer+topk+attn); indexer % fp8 MFMA peak"
CSRC = os.path.join(ROOT, "long_context_sparse_indexer_amd", "csrc")
PMC_FILE = os.path.join(ROOT, "profiles", "decode_128k_step_pmc.json")
IN_NAMES = ["q_idx", "q_idx_scale", "head_w", "k_idx_pool", "k_idx_scale", "q", "kv_pool"]


def kernel_source_hash() -> str:
    """Hash of every kernel source: a counter record is valid only for the sources it was taken on."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".h")):
            with open(os.path.join(CSRC, f), "rb") as fh:
                h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per decode_128k step from the committed counter record, if taken on the current sources."""
    try:
        with open(PMC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_step")


# ------------------------------------------------------------------------------------------ timing helpers

def cache_flush(torch, _buf=[]):
    """Read and write 768 MiB (3x the Infinity Cache) so that no timed region starts with a warm cache."""
    if not _buf:
        _buf.append(torch.zeros(768 << 20, dtype=torch.uint8, device="cuda"))
    _buf[0].add_(1)


def time_steps(torch, enqueue, steps: int, warmup: int, graph: bool, repeats: int, stream):
    """Wall and event time of `repeats` timed regions of exactly `steps` steps (enqueue(i) queues step i); the
    caches are flushed before each region."""
    for i in range(warmup):
        enqueue(i)
    torch.cuda.synchronize()
    g = None
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                enqueue(warmup + i)
        g.replay()  # first replay uploads the graph: untimed
        torch.cuda.synchronize()
    walls, gpus = [], []
    for _ in range(repeats):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        cache_flush(torch)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        a.record(stream)
        if g is not None:
            g.replay()
        else:
            for i in range(steps):
                enqueue(warmup + i)
        b.record(stream)
        torch.cuda.synchronize()
        walls.append(time.perf_counter() - t0)
        gpus.append(a.elapsed_time(b) / 1e3)
    del g
    return walls, gpus


def median_us_per_call(torch, fn, iters: int, stream, repeats: int = 5) -> float:
    """Median over repeats of the mean duration of `iters` back-to-back calls replayed from a HIP graph."""
    for i in range(min(iters, 8)):
        fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(iters):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(repeats):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e3 / iters)
    del g
    return statistics.median(ts)


class Rig:
    """A workload on the device with `copies` distinct input sets and the step's output buffers."""

    def __init__(self, torch, prob, copies: int, dev):
        import long_context_sparse_indexer_amd as dsa
        from synth.device import upload
        self.dsa, self.prob = dsa, prob
        self.base = upload(prob, dev)
        self.P = dsa.make_problem(**self.base.fields)
        self.L = dsa.make_layout(self.base.row_seq, self.base.row_len, self.base.page_table)
        self.copies = copies
        self.sets = [{n: getattr(self.base, n) for n in IN_NAMES}]
        for _ in range(copies - 1):
            self.sets.append({n: getattr(self.base, n).clone() for n in IN_NAMES})
        R = prob.R
        out_dt = torch.float32 if prob.kv_dtype == "f32" else torch.bfloat16
        self.ws = torch.empty(max(256, dsa.dsa_workspace_bytes(self.P, dsa.DSA_OP_STEP)), dtype=torch.uint8,
                              device=dev)
        self.idx = torch.empty((R, prob.k), dtype=torch.int32, device=dev)
        self.out = torch.empty((R, prob.H, prob.d_c), dtype=out_dt, device=dev)
        self.lse = torch.empty((R, prob.H), dtype=torch.float32, device=dev)

    def step(self, i, P=None):
        # the current stream at call time: inside a graph capture that is torch's capture stream
        s = self.sets[i % self.copies]
        self.dsa.dsa_decode_step(P or self.P, self.L, s["q_idx"], s["q_idx_scale"], s["head_w"], s["k_idx_pool"],
                                 s["k_idx_scale"], s["q"], s["kv_pool"], self.idx, self.out, self.lse, self.ws)


def auto_copies(prob, prefill: bool) -> int:
    import numpy as np
    from long_context_sparse_indexer_amd import cost
    touched = sum(cost.decode_row_bytes(int(n), prob.k, prob.H_I, prob.d_I, prob.H, prob.d_c,
                                        fp8_entries=prob.kv_dtype == "f8") for n in prob.row_len)
    # the steps of one timed region touch 3x the 256 MiB Infinity Cache before an input set comes round again
    return 2 if prefill else max(2, min(512, int(np.ceil(3 * 256e6 / touched))))


def step_bytes(prob) -> int:
    from long_context_sparse_indexer_amd import cost
    return sum(cost.decode_row_bytes(int(n), prob.k, prob.H_I, prob.d_I, prob.H, prob.d_c,
                                     fp8_entries=prob.kv_dtype == "f8") for n in prob.row_len)


# ------------------------------------------------------------------------------------------------ modes

def sweep(steps: int, repeats: int) -> int:
    """Step time over context lengths at k = 2048 and over budgets at n = 131072 (batch 1, decode_128k recipe),
    with least-squares fits of the affine cost model; one JSON line per point, then one per fit."""
    import numpy as np
    import torch

    import synth
    from long_context_sparse_indexer_amd import cost

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    pts_n, pts_k = [], []

    def run_point(rig, prob, P=None, k=None):
        walls, _ = time_steps(torch, lambda i: rig.step(i, P), steps, 8, True, repeats, stream)
        return statistics.median(walls) / steps * 1e6

    for n in (16384, 32768, 65536, 131072, 262144, 524288, 1048576):
        prob = synth.make_problem(synth.get("decode_128k", lengths=[n], seed=21))
        rig = Rig(torch, prob, auto_copies(prob, False), dev)
        us = run_point(rig, prob)
        rec = {"sweep": "context", "n": n, "k": prob.k, "us_per_step": round(us, 3),
               "index_bytes": n * (prob.d_I + 4), "step_bytes": step_bytes(prob), "input_copies": rig.copies}
        print(json.dumps(rec), flush=True)
        pts_n.append(rec)
        if n == 131072:
            for k in (256, 512, 1024, 2048, 4096):
                prob.k = k
                rig.P = rig.dsa.make_problem(**{**rig.base.fields, "topk": k})
                rig.ws = torch.empty(max(256, rig.dsa.dsa_workspace_bytes(rig.P, rig.dsa.DSA_OP_STEP)),
                                     dtype=torch.uint8, device=dev)
                rig.idx = torch.empty((prob.R, k), dtype=torch.int32, device=dev)
                us = run_point(rig, prob)
                rec = {"sweep": "budget", "n": n, "k": k, "us_per_step": round(us, 3),
                       "gather_bytes": k * prob.d_c * 2, "step_bytes": step_bytes(prob)}
                print(json.dumps(rec), flush=True)
                pts_k.append(rec)
        del rig
        torch.cuda.empty_cache()

    def fit(xs, ys):
        A = np.vstack([np.ones(len(xs)), np.asarray(xs, np.float64)]).T
        coef, *_ = np.linalg.lstsq(A, np.asarray(ys, np.float64), rcond=None)
        pred = A @ coef
        ss_res = float(((np.asarray(ys) - pred) ** 2).sum())
        ss_tot = float(((np.asarray(ys) - np.mean(ys)) ** 2).sum()) or 1.0
        return float(coef[0]), float(coef[1]), 1.0 - ss_res / ss_tot, [round(float(p), 3) for p in pred]

    a, b, r2, pred = fit([p["index_bytes"] for p in pts_n], [p["us_per_step"] for p in pts_n])
    print(json.dumps({"fit": "context", "model": "us = a + b * n (d_I + 4)", "a_us": round(a, 3),
                      "b_us_per_MB": round(b * 1e6, 4), "marginal_GBps": round(1e-3 / b, 1) if b > 0 else None,
                      "r2": round(r2, 5), "predicted_us": pred}), flush=True)
    a, c, r2, pred = fit([p["gather_bytes"] for p in pts_k], [p["us_per_step"] for p in pts_k])
    print(json.dumps({"fit": "budget", "model": "us = a + c * k d_c 2", "a_us": round(a, 3),
                      "c_us_per_MB": round(c * 1e6, 4), "marginal_GBps": round(1e-3 / c, 1) if c > 0 else None,
                      "r2": round(r2, 5), "predicted_us": pred}), flush=True)
    return 0


def crossover(lengths, rows: int, steps: int) -> int:
    """Sparse step vs dense attention, one JSON line per context length (graph replay, rotated inputs)."""
    import numpy as np
    import torch

    import long_context_sparse_indexer_amd as dsa
    from long_context_sparse_indexer_amd import cost
    import synth
    from synth.device import upload

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    for n in lengths:
        prob = synth.make_problem(synth.get("decode_128k", lengths=[n] * rows, seed=7))
        base = upload(prob, dev)
        P = dsa.make_problem(**base.fields)
        L = dsa.make_layout(base.row_seq, base.row_len, base.page_table)
        sparse_bytes = cost.decode_row_bytes(n, prob.k, prob.H_I, prob.d_I, prob.H, prob.d_c)
        touched = rows * max(sparse_bytes, n * prob.d_c * 2)
        copies = max(2, min(32, int(np.ceil(3 * 256e6 / touched))))
        sets = [{m: getattr(base, m) for m in IN_NAMES}] + [{m: getattr(base, m).clone() for m in IN_NAMES}
                                                            for _ in range(copies - 1)]
        idx = torch.empty((prob.R, prob.k), dtype=torch.int32, device=dev)
        out = torch.empty((prob.R, prob.H, prob.d_c), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((prob.R, prob.H), dtype=torch.float32, device=dev)
        ws_bytes = max(dsa.dsa_workspace_bytes(P, dsa.DSA_OP_STEP), dsa.dsa_workspace_bytes(P, dsa.DSA_OP_DENSE))
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

        def sparse(i):
            s = sets[i % copies]
            dsa.dsa_decode_step(P, L, s["q_idx"], s["q_idx_scale"], s["head_w"], s["k_idx_pool"], s["k_idx_scale"],
                                s["q"], s["kv_pool"], idx, out, lse, ws)

        def dense(i):
            s = sets[i % copies]
            dsa.dsa_dense_mla_attn(P, L, s["q"], s["kv_pool"], out, lse, ws)

        res = {mode: median_us_per_call(torch, fn, max(copies, min(steps, 4 * copies)), stream)
               for mode, fn in (("sparse", sparse), ("dense", dense))}
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
    stream = torch.cuda.current_stream()
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

            def call(i):
                dsa.dsa_indexer_key_append(P, L, pos, c, w, pool, scale)
            us = median_us_per_call(torch, call, max(10, min(steps, 100)), stream)
            flops = 2.0 * rows * prob.d_c * d_I
            print(json.dumps({"append": True, "tokens": rows, "d_c": prob.d_c, "d_I": d_I, "us_per_call": round(us, 2),
                              "tokens_per_s": round(rows / us * 1e6, 1),
                              "fp64_tflops": round(flops / us * 1e-6, 3), "fp64_peak_tflops": 78.6}), flush=True)
            del d, pool, scale
            torch.cuda.empty_cache()
    # indexer-query projection: h [R, 7168] bf16 through W_QI (64 heads x 64) and W_w, e4m3 codes + scales
    for rows in (1, 64):
        H_I, d_I, d_model = 64, 64, 7168
        inp = synth.query_proj_inputs(rows, d_model, H_I, d_I, "bf16", 10)
        h, wq, ww = (torch.from_numpy(inp[k].view(np.int16)).to(dev) for k in ("h", "w_q", "w_w"))
        q = torch.empty((rows, H_I, d_I), dtype=torch.uint8, device=dev)
        qs = torch.empty((rows, H_I), dtype=torch.float32, device=dev)
        hw = torch.empty((rows, H_I), dtype=torch.float32, device=dev)
        P = dsa.make_problem(num_rows=rows, idx_heads=H_I, idx_dim=d_I, idx_dtype="f8", kv_dtype="bf16", topk=1,
                             max_pages=1, num_pages=1, max_row_len=0)

        def qcall(i):
            dsa.dsa_indexer_query_proj(P, d_model, h, wq, ww, q, qs, hw)
        us = median_us_per_call(torch, qcall, max(10, min(steps, 100)), stream)
        wbytes = d_model * (H_I * d_I + H_I) * 2
        print(json.dumps({"query_proj": True, "tokens": rows, "d_model": d_model, "H_I": H_I, "d_I": d_I,
                          "us_per_call": round(us, 2), "tokens_per_s": round(rows / us * 1e6, 1),
                          "weight_read_gbps": round(wbytes / us * 1e-3, 1),
                          "fp64_tflops": round(2.0 * rows * d_model * (H_I * d_I + H_I) / us * 1e-6, 3)}),
              flush=True)
    return 0


def _read_csv(path):
    import csv
    with open(path, newline="") as fh:
        return list(csv.DictReader(fh))


def summarize_trace(d: str) -> int:
    """Mean duration per kernel from a rocprofv3 `--kernel-trace --stats -f csv` run (its kernel_stats.csv)."""
    files = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        print(f"no kernel_stats.csv under {d}", file=sys.stderr)
        return 1
    rows = _read_csv(files[0])
    print("| kernel | calls | mean duration (us) | share of traced time |")
    print("|---|---:|---:|---:|")
    for r in rows:
        print(f"| {r['Name']} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |")
    return 0


FLUSH_BYTES = 768 << 20  # the cache flush reads and writes this many bytes once (cache_flush)


def summarize_pmc(fetch_dir: str, write_dir: str, step_kernels: list[str]) -> int:
    """Per-kernel FETCH_SIZE / WRITE_SIZE means (KiB per dispatch) from two `--pmc` runs of the bench, each scaled by
    what the same counter reads for the bench's cache flush, a plain elementwise pass that reads and writes
    FLUSH_BYTES once; then the HBM bytes of one step (one dispatch of each kernel whose name contains one of
    step_kernels).  Prints the record bench.py reads for `traffic`."""
    def per_kernel(d, counter):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        acc = {}
        for r in _read_csv(files[0]):
            if r.get("Counter_Name") != counter:
                continue
            acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in acc.items()}

    fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    flush = [k for k in fetch if "CUDAFunctorOnSelf_add<unsigned char>" in k]
    if not flush:
        print("no cache-flush dispatch in the counter runs", file=sys.stderr)
        return 1
    fscale = FLUSH_BYTES / (fetch[flush[0]] * 1024)
    wscale = FLUSH_BYTES / (write[flush[0]] * 1024)
    kern = {}
    for k in sorted(set(fetch) | set(write)):
        if k == flush[0] or "copyBuffer" in k:
            continue
        kern[k] = {"fetch_kib": round(fetch.get(k, 0.0), 1), "write_kib": round(write.get(k, 0.0), 1),
                   "hbm_read_bytes": round(fetch.get(k, 0.0) * 1024 * fscale),
                   "hbm_write_bytes": round(write.get(k, 0.0) * 1024 * wscale)}
    total, used = 0, []
    for s in step_kernels:
        m = [k for k in kern if s in k]
        if m:
            used.append(m[0])
            total += kern[m[0]]["hbm_read_bytes"] + kern[m[0]]["hbm_write_bytes"]
    rec = {"kernel_source_hash": kernel_source_hash(), "calibration": "cache flush, %d bytes read and written" % FLUSH_BYTES,
           "fetch_scale": round(fscale, 4), "write_scale": round(wscale, 4), "step_kernels": used,
           "hbm_bytes_per_step": total, "kernels": kern}
    print(json.dumps(rec, indent=1))
    return 0


# ------------------------------------------------------------------------------------------------- main

def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--repeats", type=int, default=7, help="timed graph replays of --steps steps (median reported)")
    ap.add_argument("--workload", default="decode_128k",
                    choices=["decode_128k", "batched_paged", "decode_1m", "prefill_chunk", "decode_128k_di128",
                             "decode_128k_fp8kv", "prefill_chunk_di128", "batched_paged_fp8kv"])
    ap.add_argument("--copies", type=int, default=0, help="distinct input copies to rotate (0 = auto)")
    ap.add_argument("--phase-iters", type=int, default=64)
    ap.add_argument("--graph", dest="graph", action="store_true", default=True,
                    help="replay the timed steps from a captured HIP graph (default)")
    ap.add_argument("--no-graph", dest="graph", action="store_false", help="launch every step from the host")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-phases", action="store_true", help="skip the per-phase timings")
    ap.add_argument("--sweep", action="store_true", help="context and budget sweeps with affine fits, then exit")
    ap.add_argument("--crossover", action="store_true",
                    help="time the sparse step against dense attention over context lengths, then exit")
    ap.add_argument("--crossover-rows", type=int, default=1)
    ap.add_argument("--append", action="store_true",
                    help="time the indexer-key append for 1, 64 and 4096 tokens at d_I = 128 and 64, then exit")
    ap.add_argument("--summarize-trace", metavar="DIR")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--step-kernels", default="", help="';'-separated parts of the names of one step's kernels")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (see the sharding design); "
              "run with --gpus 1", file=sys.stderr)
        return 2
    if args.summarize_trace:
        return summarize_trace(args.summarize_trace)
    if args.summarize_pmc:
        return summarize_pmc(*args.summarize_pmc, [s for s in args.step_kernels.split(";") if s])
    if args.sweep:
        return sweep(args.steps, args.repeats)
    if args.crossover:
        return crossover([2048, 4096, 8192, 16384, 32768, 65536, 131072], args.crossover_rows, min(args.steps, 400))
    if args.append:
        return append_sweep(min(args.steps, 1000))

    import numpy as np
    import torch

    import long_context_sparse_indexer_amd as dsa
    from long_context_sparse_indexer_amd import cost
    import synth

    torch.cuda.init()
    dev = torch.device("cuda:0")
    cfg = synth.get(args.workload)
    t0 = time.perf_counter()
    prob = synth.make_problem(cfg)
    gen_s = time.perf_counter() - t0
    prefill = prob.rows_per_seq > 1
    copies = args.copies or auto_copies(prob, prefill)
    rig = Rig(torch, prob, copies, dev)
    R = prob.R
    stream = torch.cuda.current_stream()

    walls, gpus = time_steps(torch, lambda i: rig.step(i), args.steps, args.warmup, args.graph,
                             args.repeats, stream)
    wall = statistics.median(walls)
    qps = args.steps * R / wall
    s_per_step = wall / args.steps
    sbytes = step_bytes(prob)

    # each phase alone, graph-replayed back to back over the rotated copies, HIP events on the launch stream
    phases = {}
    if not args.no_phases:
        ld = ((max(prob.max_row_len, 1) + 63) // 64) * 64
        scores = torch.empty((R, ld), dtype=torch.float32, device=dev)
        P, L, sets = rig.P, rig.L, rig.sets
        topk_ws = torch.empty(max(256, dsa.dsa_workspace_bytes(P, dsa.DSA_OP_TOPK)), dtype=torch.uint8, device=dev)
        attn_ws = torch.empty(max(256, dsa.dsa_workspace_bytes(P, dsa.DSA_OP_ATTN)), dtype=torch.uint8, device=dev)

        def ph_indexer(i):
            s = sets[i % copies]
            dsa.dsa_indexer_scores(P, L, s["q_idx"], s["q_idx_scale"], s["head_w"], s["k_idx_pool"], s["k_idx_scale"],
                                   scores, ld)

        def ph_topk(i):
            dsa.dsa_topk(P, L, scores, rig.idx, topk_ws, ld)

        def ph_attn(i):
            s = sets[i % copies]
            dsa.dsa_sparse_mla_attn(P, L, s["q"], s["kv_pool"], rig.idx, rig.out, rig.lse, attn_ws)

        ph_indexer(0)
        ph_topk(0)
        iters = max(args.phase_iters, copies)
        us_idx = median_us_per_call(torch, ph_indexer, iters, stream)
        us_topk = median_us_per_call(torch, ph_topk, iters, stream)
        us_attn = median_us_per_call(torch, ph_attn, iters, stream)
        idx_bytes = sum(cost.indexer_row_bytes(int(n), prob.H_I, prob.d_I) for n in prob.row_len)
        attn_bytes = sbytes - idx_bytes
        phases = {
            "indexer": {"us": round(us_idx, 3), "algorithmic_bytes": idx_bytes,
                        "hbm_frac": round(idx_bytes / (us_idx * 1e-6) / (HBM_PEAK_GBS * 1e9), 4)},
            "topk": {"us": round(us_topk, 3), "algorithmic_bytes": 0, "hbm_frac": 0.0},
            "attention": {"us": round(us_attn, 3), "algorithmic_bytes": attn_bytes,
                          "hbm_frac": round(attn_bytes / (us_attn * 1e-6) / (HBM_PEAK_GBS * 1e9), 4)},
        }
        if prefill:
            idx_flops = sum(cost.indexer_row_flops(int(n), prob.H_I, prob.d_I) for n in prob.row_len)
            phases["indexer"]["tflops"] = round(idx_flops / (us_idx * 1e-6) / 1e12, 1)
            phases["indexer"]["fp8_mfma_frac"] = round(idx_flops / (us_idx * 1e-6) / 1e12 / FP8_MFMA_PEAK_TFLOPS, 4)
        del scores, topk_ws, attn_ws

    if prefill:
        # the prefill metric prices the tiled indexer against the fp8 MFMA peak
        ph = phases.get("indexer", {})
        roofline = {"bound": "mfma", "achieved": ph.get("tflops"), "peak": FP8_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": ph.get("fp8_mfma_frac"), "traffic": None, "scope": "indexer phase (tiled fp8 GEMM)"}
    else:
        achieved = sbytes / s_per_step / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": measured_traffic() if args.workload == "decode_128k" else None,
                    "scope": "whole step", "algorithmic_bytes_per_step": sbytes}
    if phases:
        dom = max(phases, key=lambda k: phases[k]["us"])
        roofline["longest_phase"] = dom

    result = {
        "metric": METRIC_PREFILL if prefill else METRIC,
        "value": round(qps, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(s_per_step * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3-indexer/fp8e4m3-latent-bf16-attention" if prob.kv_dtype == "f8"
                 else "fp8e4m3-indexer/bf16-attention",
        "data": "synthetic",
        "config": {"workload": args.workload, "rows": R, "context": int(prob.max_row_len), "k": prob.k,
                   "H_I": prob.H_I, "d_I": prob.d_I, "H": prob.H, "d_c": prob.d_c, "page_size": prob.page_size,
                   "input_copies": copies, "graph": bool(args.graph),
                   "timed_graph_replays": args.repeats if args.graph else 0},
        "roofline": roofline,
        "repeats_ms_per_step": [round(w / args.steps * 1e3, 5) for w in walls],
        "gpu_event_ms_per_step": round(statistics.median(gpus) / args.steps * 1e3, 5),
        "phases": phases,
        "gen_seconds": round(gen_s, 2),
    }

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
