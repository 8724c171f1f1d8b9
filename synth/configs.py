"""Named synthetic workloads for the DSA decode step.

Each entry fixes shapes, dtypes, paging, the boosted-position recipe and the seed.  The sizes follow the
regimes the pages discuss:
  * a 128K-token context with a top-k budget of 2048 (DeepSeek Sparse Attention explained, "How Does the
    Selector Pick 1,024?" and the V3.2-Exp column of its config table; kiadev "How DSA works"),
  * 64 indexer heads of a narrow width and one shared indexer key per position ("How Does the Lightning
    Indexer Score a Token?"; milos-mitrovic "How Does the Lightning Indexer Pick Which Tokens Matter?"),
  * one 512-wide latent row shared by every query head (lizeman DSA page, section 1 and section 2),
  * million-token windows (DeepSeek Sparse Attention explained, introduction).
"""
from __future__ import annotations

import copy

# idx_dtype: "f8" = OCP e4m3fn codes with one fp32 scale per 64-vector, "f32" = plain fp32
# kv_dtype:  "bf16" or "f32" (latent pool, attention queries and outputs)
CONFIGS = {
    # one query at position 4096 over a 4095-entry cache, fp32 throughout
    "tiny_fp32": dict(
        kind="decode", batch=1, lengths=[4095], H_I=4, d_I=64, k=256, H=16, d_c=512,
        idx_dtype="f32", kv_dtype="f32", anchors=32, recent=0, paged=False, seed=0, page_size=64,
        softmax_scale=1.0),
    # single-sequence decode at T = 128K
    "decode_128k": dict(
        kind="decode", batch=1, lengths=[131072], H_I=64, d_I=64, k=2048, H=128, d_c=512,
        idx_dtype="f8", kv_dtype="bf16", anchors=256, recent=512, paged=False, seed=1, page_size=64,
        softmax_scale=1.0),
    # 64 sequences, lengths uniform in [16384, 65536], random page table
    "batched_paged": dict(
        kind="decode", batch=64, length_range=(16384, 65536), H_I=64, d_I=64, k=2048, H=128, d_c=512,
        idx_dtype="f8", kv_dtype="bf16", anchors=256, recent=512, paged=True, seed=2, page_size=64,
        softmax_scale=1.0),
    # chunked prefill: 4096 consecutive query positions over the decode_128k cache, causal
    "prefill_chunk": dict(
        kind="prefill", cache_len=131072, rows=4096, H_I=64, d_I=64, k=2048, H=128, d_c=512,
        idx_dtype="f8", kv_dtype="bf16", anchors=256, recent=512, paged=False, seed=1, page_size=64,
        softmax_scale=1.0),
    # the shipped indexer shape: 64 heads x 128 dims (132 B per cached position) over the decode_128k row
    "decode_128k_di128": dict(
        kind="decode", batch=1, lengths=[131072], H_I=64, d_I=128, k=2048, H=128, d_c=512,
        idx_dtype="f8", kv_dtype="bf16", anchors=256, recent=512, paged=False, seed=6, page_size=64,
        softmax_scale=1.0),
    # single-sequence decode at T = 128K over the 656-byte FP8 latent cache (512 e4m3 + 4 scales + 64 RoPE dims)
    "decode_128k_fp8kv": dict(
        kind="decode", batch=1, lengths=[131072], H_I=64, d_I=64, k=2048, H=128, d_c=512,
        idx_dtype="f8", kv_dtype="f8", anchors=256, recent=512, paged=False, seed=10, page_size=64,
        softmax_scale=1.0),
    # the batched decode over the FP8 latent cache
    "batched_paged_fp8kv": dict(
        kind="decode", batch=64, length_range=(16384, 65536), H_I=64, d_I=64, k=2048, H=128, d_c=512,
        idx_dtype="f8", kv_dtype="f8", anchors=256, recent=512, paged=True, seed=12, page_size=64,
        softmax_scale=1.0),
    # the chunked prefill with the shipped indexer shape (64 heads x 128 dims)
    "prefill_chunk_di128": dict(
        kind="prefill", cache_len=131072, rows=4096, H_I=64, d_I=128, k=2048, H=128, d_c=512,
        idx_dtype="f8", kv_dtype="bf16", anchors=256, recent=512, paged=False, seed=11, page_size=64,
        softmax_scale=1.0),
    # chunked prefill of several paged sequences at once (rows consecutive rows per sequence)
    "prefill_paged": dict(
        kind="prefill", batch=3, length_range=(3000, 9000), rows=37, H_I=64, d_I=64, k=2048, H=32, d_c=512,
        idx_dtype="f8", kv_dtype="bf16", anchors=64, recent=128, paged=True, seed=5, page_size=64,
        softmax_scale=1.0),
    # 8 sequences of 2^20 tokens
    "decode_1m": dict(
        kind="decode", batch=8, lengths=[1048576] * 8, H_I=64, d_I=64, k=2048, H=128, d_c=512,
        idx_dtype="f8", kv_dtype="bf16", anchors=1024, recent=2048, paged=False, seed=4, page_size=64,
        softmax_scale=1.0),
}

ORDER = ["tiny_fp32", "decode_128k", "batched_paged", "prefill_chunk", "decode_1m", "prefill_paged",
         "decode_128k_di128", "decode_128k_fp8kv", "prefill_chunk_di128", "batched_paged_fp8kv"]


def get(name: str, **overrides) -> dict:
    """A copy of a named workload with fields replaced (used for scaled-down test cases)."""
    cfg = copy.deepcopy(CONFIGS[name])
    cfg["name"] = name
    cfg.update(overrides)
    return cfg
