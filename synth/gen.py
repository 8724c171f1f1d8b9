"""Seeded synthetic inputs for the DSA decode step.

This module only draws random numbers and stores them in the byte formats the step consumes: bf16 for the
latent cache and queries, OCP e4m3fn codes plus one fp32 scale per 64-vector for the indexer operands.  It
computes none of the method's steps (no scoring, no selection, no attention); both the CPU oracle and the
GPU path receive the arrays it returns.

Recipe (per sequence, fp32 masters, "N(0, v)" means variance v):
  latent c[s] ~ N(0, 1) over d_c = 512 dims, stored rounded to the latent dtype;
  W_KI ~ N(0, 1/d_c) shared by every sequence of a workload; indexer keys k_I = c_stored @ W_KI, as the
    indexer key projection of the lizeman DSA page (section 3 sketch) writes it;
  indexer queries q_I[j] ~ N(0, 1/d_I) for each of the H_I heads; head weights w[j] ~ U(0, 1);
  attention queries q[h] ~ N(0, 1/d_c) for each of the H heads (already in latent space);
  boosted positions (random anchors drawn without replacement outside the most recent window, plus that
    window) get k_I[s] += 0.5 * mean_j q_I[j], which makes the score spiky at planted positions;
  fp8 operands: scale = amax / 448 per d_I-vector (1 for an all-zero vector), code = e4m3fn(RNE(x / scale));
  an fp8 latent cache ("f8" latent dtype) stores 656-byte entries: the latent quantised the same way per
    128-value tile, the 4 tile scales, and 64 RoPE values r[s] ~ N(0, 1) as bf16; its queries gain 64 RoPE
    dims ~ N(0, 1/576) (drawn after every other value of the sequence); k_I uses the dequantised latent.
Pages are 64 positions; a paged workload places every logical page of every sequence at a random physical
page of one shared pool, the others place them in order.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

E4M3_MAX = 448.0


@dataclasses.dataclass
class Problem:
    cfg: dict
    R: int
    S: int
    H_I: int
    d_I: int
    H: int
    d_c: int
    k: int
    page_size: int
    max_pages: int
    num_pages: int
    idx_dtype: str
    kv_dtype: str
    softmax_scale: float
    q_idx: np.ndarray            # [R, H_I, d_I] uint8 e4m3fn codes | float32
    q_idx_scale: np.ndarray | None  # [R, H_I] float32 (fp8 only)
    head_w: np.ndarray           # [R, H_I] float32
    k_idx_pool: np.ndarray       # [num_pages * page_size, d_I] uint8 | float32
    k_idx_scale: np.ndarray | None  # [num_pages * page_size] float32 (fp8 only)
    q: np.ndarray                # [R, H, d_c] uint16 bf16 bits | float32
    kv_pool: np.ndarray          # [num_pages * page_size, d_c] uint16 | float32
    row_seq: np.ndarray          # [R] int32
    row_len: np.ndarray          # [R] int32
    page_table: np.ndarray       # [S, max_pages] int32
    boosted: list                # per sequence: int64 positions that were boosted
    rows_per_seq: int = 1        # consecutive rows sharing one sequence (a chunked prefill: rows per sequence)

    @property
    def max_row_len(self) -> int:
        return int(self.row_len.max()) if self.R else 0


def _child(seed: int, *key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=tuple(key)))


def _round_kv(x: np.ndarray, kv_dtype: str):
    """(stored bits or values, fp32 value of what is stored)."""
    if kv_dtype == "f32":
        return x, x
    t = torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy(), t.to(torch.float32).numpy()


def _quant_rows(x: np.ndarray):
    """Per-64-vector e4m3fn quantisation of the last axis: (codes uint8, scale float32)."""
    amax = np.abs(x).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    y = np.clip(x / scale[..., None], -E4M3_MAX, E4M3_MAX).astype(np.float32)
    codes = torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    return codes, scale


def _fp8_latent(c: np.ndarray, rope: np.ndarray):
    """656-byte latent cache entries: 512 e4m3 codes quantised per 128-value tile (scale = tile amax / 448, 1 for
    a zero tile), the 4 fp32 tile scales, the 64 RoPE values as bf16; and the fp32 value of the stored latent."""
    n = c.shape[0]
    codes, scale = _quant_rows(c.reshape(n, 4, 128))
    deq = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy() * scale[..., None]
    ent = np.zeros((n, 656), np.uint8)
    ent[:, :512] = codes.reshape(n, 512)
    ent[:, 512:528] = np.ascontiguousarray(scale, np.float32).view(np.uint8).reshape(n, 16)
    rope_bits, _ = _round_kv(rope, "bf16")
    ent[:, 528:] = np.ascontiguousarray(rope_bits).view(np.uint8).reshape(n, 128)
    return ent, deq.reshape(n, 512).astype(np.float32)


def _draw_sequence(rng: np.random.Generator, n: int, cfg: dict, W_KI: np.ndarray):
    d_c, d_I, H_I, H = cfg["d_c"], cfg["d_I"], cfg["H_I"], cfg["H"]
    c = rng.standard_normal((n, d_c), dtype=np.float32)
    q_I = rng.standard_normal((H_I, d_I), dtype=np.float32) * np.float32(math.sqrt(1.0 / d_I))
    w = rng.random(H_I, dtype=np.float32)
    q = rng.standard_normal((H, d_c), dtype=np.float32) * np.float32(math.sqrt(1.0 / d_c))
    W = min(cfg["recent"], n)
    A = min(cfg["anchors"], n - W)
    anchors = rng.choice(n - W, size=A, replace=False) if A > 0 else np.zeros(0, np.int64)
    boosted = np.sort(np.concatenate([anchors.astype(np.int64), np.arange(n - W, n, dtype=np.int64)]))
    if cfg["kv_dtype"] == "f8":
        # RoPE parts of the cache entries and of the query, drawn after everything else
        c_bits, c_val = _fp8_latent(c, rng.standard_normal((n, 64), dtype=np.float32))
        q = np.concatenate([q, rng.standard_normal((H, 64), dtype=np.float32) * np.float32(math.sqrt(1.0 / 576))],
                           axis=1)
    else:
        c_bits, c_val = _round_kv(c, cfg["kv_dtype"])
    del c
    k_I = c_val @ W_KI
    k_I[boosted] += np.float32(0.5) * q_I.mean(axis=0)
    return dict(c_bits=c_bits, k_I=k_I, q_I=q_I, w=w, q=q, boosted=boosted)


def _extra_row(rng: np.random.Generator, cfg: dict):
    d_c, d_I, H_I, H = cfg["d_c"], cfg["d_I"], cfg["H_I"], cfg["H"]
    q_I = rng.standard_normal((H_I, d_I), dtype=np.float32) * np.float32(math.sqrt(1.0 / d_I))
    w = rng.random(H_I, dtype=np.float32)
    q = rng.standard_normal((H, d_c), dtype=np.float32) * np.float32(math.sqrt(1.0 / d_c))
    if cfg["kv_dtype"] == "f8":
        q = np.concatenate([q, rng.standard_normal((H, 64), dtype=np.float32) * np.float32(math.sqrt(1.0 / 576))],
                           axis=1)
    return q_I, w, q


def make_problem(cfg: dict) -> Problem:
    """Generate every input of one workload (see synth.configs)."""
    seed, ps = cfg["seed"], cfg["page_size"]
    d_c, d_I, H_I, H = cfg["d_c"], cfg["d_I"], cfg["H_I"], cfg["H"]
    W_KI = _child(seed, 0).standard_normal((d_c, d_I), dtype=np.float32) * np.float32(math.sqrt(1.0 / d_c))

    if cfg["kind"] == "prefill" and "cache_len" in cfg:
        lengths = [cfg["cache_len"]]
    elif "lengths" in cfg:
        lengths = list(cfg["lengths"])
    else:
        lo, hi = cfg["length_range"]
        lengths = _child(seed, 1).integers(lo, hi, endpoint=True, size=cfg["batch"]).tolist()
    S = len(lengths)
    pages_per = [-(-n // ps) for n in lengths]
    num_pages = max(1, sum(pages_per))
    max_pages = max(1, max(pages_per))
    if cfg.get("paged"):
        perm = _child(seed, 2).permutation(num_pages).astype(np.int32)
    else:
        perm = np.arange(num_pages, dtype=np.int32)
    page_table = np.zeros((S, max_pages), np.int32)
    off = 0
    for b, npg in enumerate(pages_per):
        page_table[b, :npg] = perm[off:off + npg]
        off += npg

    f8 = cfg["idx_dtype"] == "f8"
    kv_np = {"bf16": np.uint16, "f32": np.float32, "f8": np.uint8}[cfg["kv_dtype"]]
    k_pool = np.zeros((num_pages * ps, d_I), np.uint8 if f8 else np.float32)
    k_scale = np.ones(num_pages * ps, np.float32) if f8 else None
    kv_pool = np.zeros((num_pages * ps, 656 if cfg["kv_dtype"] == "f8" else d_c), kv_np)

    q_I_rows, w_rows, q_rows, row_seq, row_len, boosted = [], [], [], [], [], []
    for b, n in enumerate(lengths):
        seq = _draw_sequence(_child(seed, 3, b), n, cfg, W_KI)
        phys = (page_table[b, np.arange(n) // ps].astype(np.int64) * ps + np.arange(n) % ps)
        kv_pool[phys] = seq["c_bits"]
        if f8:
            codes, sc = _quant_rows(seq["k_I"])
            k_pool[phys] = codes
            k_scale[phys] = sc
        else:
            k_pool[phys] = seq["k_I"]
        boosted.append(seq["boosted"])
        if cfg["kind"] == "decode":
            q_I_rows.append(seq["q_I"]); w_rows.append(seq["w"]); q_rows.append(seq["q"])
            row_seq.append(b); row_len.append(n)
        else:
            # causal chunk: the row at 1-based position p sees positions 0..p-1; the last row is the
            # sequence's own query, the others are fresh draws
            rows = cfg["rows"]
            assert 1 <= rows <= n, "a prefill chunk needs at least `rows` cached positions per sequence"
            first = n - rows + 1
            rng = _child(seed, 4, b)
            for r in range(rows - 1):
                a, bw, c = _extra_row(rng, cfg)
                q_I_rows.append(a); w_rows.append(bw); q_rows.append(c)
            q_I_rows.append(seq["q_I"]); w_rows.append(seq["w"]); q_rows.append(seq["q"])
            row_seq.extend([b] * rows)
            row_len.extend(range(first, first + rows))
        del seq

    R = len(row_seq)
    q_I = np.stack(q_I_rows) if R else np.zeros((0, H_I, d_I), np.float32)
    if f8:
        q_idx, q_idx_scale = _quant_rows(q_I)
    else:
        q_idx, q_idx_scale = q_I.astype(np.float32), None
    q_width = d_c + 64 if cfg["kv_dtype"] == "f8" else d_c
    q_all = np.stack(q_rows) if R else np.zeros((0, H, q_width), np.float32)
    q_bits, _ = _round_kv(q_all, "bf16" if cfg["kv_dtype"] == "f8" else cfg["kv_dtype"])
    return Problem(
        cfg=cfg, R=R, S=S, H_I=H_I, d_I=d_I, H=H, d_c=d_c, k=cfg["k"], page_size=ps, max_pages=max_pages,
        num_pages=num_pages, idx_dtype=cfg["idx_dtype"], kv_dtype=cfg["kv_dtype"],
        softmax_scale=float(cfg["softmax_scale"]),
        q_idx=np.ascontiguousarray(q_idx), q_idx_scale=q_idx_scale,
        head_w=np.ascontiguousarray(np.stack(w_rows).astype(np.float32)) if R else np.zeros((0, H_I), np.float32),
        k_idx_pool=k_pool, k_idx_scale=k_scale, q=np.ascontiguousarray(q_bits), kv_pool=kv_pool,
        row_seq=np.asarray(row_seq, np.int32), row_len=np.asarray(row_len, np.int32),
        page_table=page_table, boosted=boosted,
        rows_per_seq=cfg["rows"] if cfg["kind"] == "prefill" else 1)


def append_inputs(prob: Problem, seed: int) -> dict:
    """Inputs of the indexer-key append for the problem's rows: the newest token of each row (position
    row_len - 1; rows with no position get -1 and are skipped).

      c [R, d_c]: latent rows ~ N(0, 1), stored in the problem's latent dtype; row 0 is all zero when R > 1
        (a zero key);
      w [d_c, d_I]: W_KI ~ N(0, 1/d_c) in the same dtype;
      k32 [R, d_I]: fp32 keys for the append of already-projected keys, ~ N(0, 1) with one entry per row
        30x larger (its small neighbours then fall among the e4m3 subnormals) and a zero row 0 when R > 1.
    """
    rng = _child(seed, 7)
    d_c, d_I, R = prob.d_c, prob.d_I, prob.R
    c = rng.standard_normal((R, d_c), dtype=np.float32)
    w = rng.standard_normal((d_c, d_I), dtype=np.float32) * np.float32(math.sqrt(1.0 / d_c))
    k32 = rng.standard_normal((R, d_I), dtype=np.float32)
    k32[np.arange(R), rng.integers(0, d_I, R)] *= np.float32(30.0)
    if R > 1:
        c[0] = 0.0
        k32[0] = 0.0
    c_bits, _ = _round_kv(c, prob.kv_dtype)
    w_bits, _ = _round_kv(w, prob.kv_dtype)
    positions = np.where(prob.row_len > 0, prob.row_len - 1, -1).astype(np.int32)
    return dict(c=np.ascontiguousarray(c_bits), w=np.ascontiguousarray(w_bits), k32=k32, positions=positions)


def query_proj_inputs(R: int, d_model: int, H_I: int, d_I: int, act_dtype: str, seed: int) -> dict:
    """Inputs of the indexer-query projection for R tokens.

      h [R, d_model]: hidden states ~ N(0, 1) in act_dtype ("bf16" bit patterns or "f32"); row 0 is all zero when
        R > 1 (every head then has scale 1 and zero codes), and one entry per row is 30x larger;
      w_q [d_model, H_I * d_I]: W_QI ~ N(0, 1/d_model); the columns of head H_I - 1 are zero when H_I > 1 (a zero
        head in every row);
      w_w [d_model, H_I]: the head-weight projection ~ N(0, 1/d_model).
    """
    rng = _child(seed, 8)
    h = rng.standard_normal((R, d_model), dtype=np.float32)
    if R:
        h[np.arange(R), rng.integers(0, d_model, R)] *= np.float32(30.0)
    if R > 1:
        h[0] = 0.0
    sd = np.float32(math.sqrt(1.0 / d_model))
    w_q = rng.standard_normal((d_model, H_I * d_I), dtype=np.float32) * sd
    if H_I > 1:
        w_q[:, (H_I - 1) * d_I:] = 0.0
    w_w = rng.standard_normal((d_model, H_I), dtype=np.float32) * sd
    out = {}
    for name, a in (("h", h), ("w_q", w_q), ("w_w", w_w)):
        bits, _ = _round_kv(a, act_dtype)
        out[name] = np.ascontiguousarray(bits)
    return out
