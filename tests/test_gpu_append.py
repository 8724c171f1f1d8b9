"""GPU parity of the indexer-key append (dsa_indexer_key_append) against the oracle.

The codes and scales are integers and fp32 values decided in a fixed order on both sides (exact fp64 products
summed over d ascending, one rounding to fp32, IEEE fp32 divisions), so the whole written pool must match the
oracle's bit for bit, and every pool row that no token addresses must keep its old bytes.
"""
import dataclasses

import numpy as np
import pytest
import torch

import long_context_sparse_indexer_amd as dsa
import oracle
import synth
from harness import check_scores, say
from synth.device import upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsa.lib()


def _append(prob, app, project, positions=None):
    """Append on the GPU and in the oracle over a pool pre-filled with sentinels; both pools (host arrays)."""
    positions = app["positions"] if positions is None else positions
    f8 = prob.idx_dtype == "f8"
    rows = prob.num_pages * prob.page_size
    if f8:
        pool0 = np.full((rows, prob.d_I), 0xAA, np.uint8)
        scale0 = np.full(rows, -5.0, np.float32)
    else:
        pool0 = np.full((rows, prob.d_I), -5.0, np.float32)
        scale0 = None
    dev = "cuda:0"
    d = upload(prob, dev)
    P = dsa.make_problem(**d.fields)
    L = dsa.make_layout(d.row_seq, d.row_len, d.page_table)
    pool = torch.from_numpy(pool0.copy()).to(dev)
    scale = torch.from_numpy(scale0.copy()).to(dev) if f8 else None
    pos = torch.from_numpy(np.ascontiguousarray(positions, np.int32)).to(dev)
    if project:
        src = torch.from_numpy(app["c"].view(np.int16) if prob.kv_dtype == "bf16" else app["c"]).to(dev)
        w = torch.from_numpy(app["w"].view(np.int16) if prob.kv_dtype == "bf16" else app["w"]).to(dev)
    else:
        src, w = torch.from_numpy(app["k32"]).to(dev), None
    dsa.dsa_indexer_key_append(P, L, pos, src, w, pool, scale)
    torch.cuda.synchronize()
    got_pool = pool.cpu().numpy()
    got_scale = scale.cpu().numpy() if f8 else None
    k32 = oracle.key_projection(app["c"], app["w"], prob.kv_dtype).astype(np.float32) if project else app["k32"]
    ref_pool, ref_scale = oracle.key_append(k32, positions, prob.row_seq, prob.page_table, prob.page_size, pool0,
                                            scale0)
    return got_pool, got_scale, ref_pool, ref_scale


def _check(prob, app, project, positions=None):
    positions = app["positions"] if positions is None else positions
    pos = np.asarray(positions)
    say(f"append case R={prob.R} d_I={prob.d_I} idx={prob.idx_dtype} kv={prob.kv_dtype} project={project} "
        f"written={((pos >= 0) & (pos < prob.max_pages * prob.page_size)).sum()}")
    got_pool, got_scale, ref_pool, ref_scale = _append(prob, app, project, positions)
    bad = np.argwhere(got_pool != ref_pool) if got_pool.dtype == np.uint8 else \
        np.argwhere(got_pool.view(np.uint32) != ref_pool.view(np.uint32))
    assert bad.size == 0, f"{len(bad)} pool entries differ, first at {bad[:4].tolist()}"
    if ref_scale is not None:
        assert np.array_equal(got_scale.view(np.uint32), ref_scale.view(np.uint32)), "scales differ"
    say("  ok: pool and scales bit-exact")
    return got_pool, got_scale


@pytest.mark.parametrize("d_I", [64, 128])
def test_append_fp32_keys_into_fp8_cache(d_I):
    prob = synth.make_problem(synth.get("batched_paged", batch=37, length_range=(100, 3000), d_I=d_I, anchors=4,
                                        recent=4))
    _check(prob, synth.append_inputs(prob, 1), project=False)


@pytest.mark.parametrize("d_I", [64, 128])
def test_append_bf16_projection_into_fp8_cache(d_I):
    # 37 tokens: several 8- or 16-token blocks and a ragged one; token 0 has a zero latent row (scale 1, zero codes)
    prob = synth.make_problem(synth.get("batched_paged", batch=37, length_range=(100, 3000), d_I=d_I, anchors=4,
                                        recent=4))
    _check(prob, synth.append_inputs(prob, 2), project=True)


@pytest.mark.parametrize("d_I", [64, 128])
def test_append_single_token(d_I):
    # one token: the single-row launch, where one wave runs the chains and the others stage W_KI
    prob = synth.make_problem(synth.get("batched_paged", batch=1, length_range=(100, 3000), d_I=d_I, anchors=4,
                                        recent=4))
    _check(prob, synth.append_inputs(prob, 11), project=True)


def test_append_skips_rows_and_prefill_positions():
    # a chunked-prefill layout: 24 consecutive positions of one sequence, written by 24 rows; rows with a
    # negative position or one beyond the page table's reach are skipped
    prob = synth.make_problem(synth.get("prefill_chunk", cache_len=6000, rows=24, H=32, d_I=128))
    app = synth.append_inputs(prob, 3)
    pos = app["positions"].copy()
    pos[3] = -1
    pos[7] = prob.max_pages * prob.page_size  # out of reach
    pos[11] = -100
    _check(prob, app, project=True, positions=pos)


def test_append_fp32_latent_and_fp32_cache():
    # fp32 latent rows (W_KI read from global memory) into an fp8 cache, and into an fp32 cache
    prob = synth.make_problem(synth.get("batched_paged", batch=9, length_range=(100, 900), kv_dtype="f32", H=16,
                                        anchors=4, recent=4))
    _check(prob, synth.append_inputs(prob, 4), project=True)
    prob32 = synth.make_problem(synth.get("tiny_fp32", lengths=[1000, 4095, 17], d_I=40))
    _check(prob32, synth.append_inputs(prob32, 5), project=True)
    _check(prob32, synth.append_inputs(prob32, 6), project=False)


def test_append_then_score_every_position():
    # every position of a 3000-token sequence written by the append (one row per position), then scored by the
    # indexer against the oracle's scores over the oracle's pool
    base = synth.make_problem(synth.get("decode_128k", lengths=[3000], d_I=128, anchors=16, recent=32))
    n = 3000
    rows = dataclasses.replace(base, R=n, row_seq=np.zeros(n, np.int32), row_len=np.full(n, n, np.int32),
                               rows_per_seq=1)
    app = synth.append_inputs(rows, 8)
    app["positions"] = np.arange(n, dtype=np.int32)
    pool, scale = _check(rows, app, project=True)
    prob = dataclasses.replace(base, k_idx_pool=pool, k_idx_scale=scale)
    d = upload(prob, "cuda:0")
    P = dsa.make_problem(**d.fields)
    L = dsa.make_layout(d.row_seq, d.row_len, d.page_table)
    ld = (n + 63) // 64 * 64
    scores = torch.empty((1, ld), dtype=torch.float32, device="cuda:0")
    dsa.dsa_indexer_scores(P, L, d.q_idx, d.q_idx_scale, d.head_w, d.k_idx_pool, d.k_idx_scale, scores, ld)
    torch.cuda.synchronize()
    ref = oracle.indexer_scores(prob.q_idx, prob.q_idx_scale, prob.head_w, pool, scale, prob.row_seq, prob.row_len,
                                prob.page_table, prob.page_size, prob.idx_dtype)
    ratio = check_scores(prob, scores.cpu().numpy(), ref)
    say(f"  ok: scores over the appended cache within {ratio:.3f} of the fp32 bound")
