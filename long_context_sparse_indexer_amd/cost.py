"""Bytes and operation counts of the DSA step (the roofline denominators).

The closed forms below reproduce the figures the pages print (pinned in tests/test_cost_model.py):
  * lizeman DSA page, section 2 "Total per-token cost": t*d_I indexer ops + K*d_c attention ops per token
    against t*d_c for full MLA, and the indexer parameter overhead (d_model + d_c) * d_I per layer;
  * DeepSeek Sparse Attention explained, "How Much Arithmetic Does This Actually Save?": multiply-adds per
    (query, key) pair for attention (heads * (576 + 512)) and for the indexer (index heads * index width),
    and the totals over a full 128K x 128K prefill grid;
  * same page, "Why Is Decoding Held Back by Memory?" (576-number bf16 entry, 1,152 B per layer) and "What
    Does the GPU Actually Run?" (656-byte fp8 entry: 512 e4m3 values, 4 fp32 scales, 64 bf16 rope dims);
  * milos-mitrovic, "What Does DSA Actually Cost in Compute and Memory?": KV bytes read per decode step at
    131K context, dense MLA vs DSA, with an fp8 indexer key of about 132 bytes per position.
"""
from __future__ import annotations


# ----------------------------------------------------------------------------------- per-entry sizes

def indexer_key_bytes(d_I: int, code_bytes: int = 1, scale_bytes: int = 4) -> int:
    """One position of the indexer key cache: d_I fp8 codes plus one fp32 scale."""
    return d_I * code_bytes + scale_bytes


def latent_entry_bytes_bf16(d_c: int = 512, rope: int = 64) -> int:
    return 2 * (d_c + rope)


def latent_entry_bytes_fp8(d_c: int = 512, rope: int = 64, tile: int = 128) -> int:
    """fp8 latent values, one fp32 scale per `tile` values, bf16 rope dims."""
    return d_c + 4 * (d_c // tile) + 2 * rope


# ------------------------------------------------------------------------------------ operation counts

def per_token_ops(t: int, d_I: int, K: int, d_c: int) -> dict:
    """Per-query operation counts in the lizeman accounting (one op per stored number touched)."""
    idx, att, dense = t * d_I, K * d_c, t * d_c
    return dict(indexer=idx, attention=att, dsa=idx + att, dense=dense, ratio=dense / (idx + att))


def indexer_params_per_layer(d_model: int, d_c: int, d_I: int) -> int:
    return (d_model + d_c) * d_I


def macs_per_pair(heads: int = 128, d_qk: int = 576, d_v: int = 512, index_heads: int = 64,
                  index_dim: int = 128) -> dict:
    att = heads * d_qk + heads * d_v
    idx = index_heads * index_dim
    return dict(attention=att, indexer=idx, ratio=att / idx)


def prefill_grid_macs(T: int, k: int, per_pair: dict) -> dict:
    dense = T * T * per_pair["attention"]
    idx = T * T * per_pair["indexer"]
    sparse = T * k * per_pair["attention"]
    return dict(dense=dense, indexer=idx, sparse=sparse, dsa=idx + sparse, block_ratio=dense / (idx + sparse),
                attention_ratio=dense / sparse, indexer_over_sparse=idx / sparse)


def decode_kv_read_bytes(n: int, k: int, layers: int, entry_bytes: int, key_bytes: int) -> dict:
    """Bytes a decode step reads over all layers: whole latent cache (dense) vs keys + k entries (DSA)."""
    return dict(dense=n * entry_bytes * layers, dsa=(n * key_bytes + min(k, n) * entry_bytes) * layers)


# ----------------------------------------------------------------- this library's decode row, one layer

FP8_ENTRY_BYTES = 656  # 512 e4m3 latent values + 4 fp32 tile scales + 64 bf16 RoPE values
FP8_QUERY_WIDTH = 576  # latent dims + RoPE dims


def decode_row_bytes(n: int, k: int, H_I: int = 64, d_I: int = 64, H: int = 128, d_c: int = 512,
                     kv_bytes: int = 2, idx_code_bytes: int = 1, fp8_entries: bool = False) -> int:
    """Algorithmic HBM bytes of one decode row: indexer keys + scales, indexer query + scales + weights,
    the k_eff gathered latent rows, and the attention query in / output out.  fp8_entries: the latent cache holds
    656-byte FP8 entries and the bf16 query is 576 wide."""
    keff = min(k, n)
    scale = 4 if idx_code_bytes == 1 else 0
    indexer = n * (d_I * idx_code_bytes + scale) + H_I * (d_I * idx_code_bytes + scale + 4)
    if fp8_entries:
        return indexer + keff * FP8_ENTRY_BYTES + H * (FP8_QUERY_WIDTH + d_c) * 2
    return indexer + keff * d_c * kv_bytes + 2 * H * d_c * kv_bytes


def indexer_row_bytes(n: int, H_I: int = 64, d_I: int = 64, idx_code_bytes: int = 1) -> int:
    """Algorithmic bytes of the indexer for one row: keys + scales read, query + scales + weights read."""
    scale = 4 if idx_code_bytes == 1 else 0
    return n * (d_I * idx_code_bytes + scale) + H_I * (d_I * idx_code_bytes + scale + 4)


def indexer_row_flops(n: int, H_I: int = 64, d_I: int = 64) -> int:
    return 2 * n * H_I * d_I


def attention_row_flops(k: int, n: int, H: int = 128, d_c: int = 512) -> int:
    keff = min(k, n)
    return 2 * 2 * H * keff * d_c
