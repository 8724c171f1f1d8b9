"""The cost model reproduces the byte and operation figures the pages print."""
import math

from long_context_sparse_indexer_amd import cost


def test_lizeman_per_token_ops():
    # lizeman DSA page, section 2 "Total per-token cost": t = 128K, K = 2K, d_I = 64, d_c = 512
    c = cost.per_token_ops(128_000, 64, 2_000, 512)
    assert round(c["indexer"] / 1e6, 1) == 8.2
    assert round(c["attention"] / 1e6, 1) == 1.0
    assert round(c["dsa"] / 1e6, 1) == 9.2
    assert round(c["dense"] / 1e7, 1) == 6.6
    assert round(c["ratio"]) == 7


def test_lizeman_parameter_overhead():
    per_layer = cost.indexer_params_per_layer(7168, 512, 64)
    assert round(per_layer / 1e4) * 1e4 == 490_000
    assert round(per_layer * 61 / 1e6) == 30


def test_kgptalkie_pair_costs_and_grid_totals():
    # "How Much Arithmetic Does This Actually Save?"
    p = cost.macs_per_pair(heads=128, d_qk=576, d_v=512, index_heads=64, index_dim=128)
    assert p["attention"] == 139_264 and p["indexer"] == 8_192 and round(p["ratio"]) == 17
    g = cost.prefill_grid_macs(131_072, 2_048, p)
    assert round(g["dense"] / 1e12) == 2_393
    assert round(g["indexer"] / 1e12) == 141
    assert round(g["sparse"] / 1e12) == 37
    assert round(g["dsa"] / 1e12) == 178
    assert round(g["attention_ratio"]) == 64
    assert round(g["block_ratio"], 1) == 13.4
    assert round(g["indexer_over_sparse"], 1) == 3.8


def test_kgptalkie_cache_entry_sizes():
    assert cost.latent_entry_bytes_bf16(512, 64) == 1_152
    assert cost.latent_entry_bytes_bf16(512, 64) * 62 == 71_424
    assert round(71_424 * 131_072 / 2 ** 30, 2) == 8.72          # "8.72 GB" at 128K is GiB
    assert cost.latent_entry_bytes_fp8(512, 64, tile=128) == 656  # 512 e4m3 + 4 fp32 + 64 bf16


def test_milos_decode_read_bytes_at_131k():
    # "What Does DSA Actually Cost in Compute and Memory?": 5.2 GB dense MLA vs 1.1 GB DSA, ~132 B per key
    key = cost.indexer_key_bytes(128)
    assert key == 132
    b = cost.decode_kv_read_bytes(131_072, 2_048, 61, cost.latent_entry_bytes_fp8(), key)
    assert round(b["dense"] / 1e9, 1) == 5.2
    assert round(b["dsa"] / 1e9, 1) == 1.1


def test_decode_row_bytes_of_the_128k_workload():
    b = cost.decode_row_bytes(131_072, 2_048)
    assert b == 131_072 * 68 + 64 * 72 + 2_048 * 1_024 + 2 * 128 * 1_024 == 11_276_800
    assert cost.decode_row_bytes(100, 2_048) == 100 * 68 + 64 * 72 + 100 * 1_024 + 2 * 128 * 1_024
    # FP8 latent entries: 656 bytes gathered per selected position, a 576-wide query in and 512-wide output out
    assert cost.decode_row_bytes(100, 2_048, fp8_entries=True) == 100 * 68 + 64 * 72 + 100 * 656 + 128 * 1_088 * 2
    assert math.isclose(cost.attention_row_flops(2048, 131072) / 1e6, 536.870912)
