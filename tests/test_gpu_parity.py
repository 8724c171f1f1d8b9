"""GPU parity: every kernel of the HIP path, called through the C ABI, against the CPU oracle.

Run on an MI355X (gfx950).  Sizes span several indexer tiles (512 positions), several top-k chunks (4096
scores) and attention chunks (64 slots), each with a ragged tail; the decode_128k case runs at full size.
"""
import math

import numpy as np
import pytest
import torch

import long_context_sparse_indexer_amd as dsa
import oracle
import synth
from harness import full_check, gpu_step, say, check_topk_exact, sampled_check, check_attention

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsa.lib()


def _run(cfg, fields=None, mutate=None):
    say(f"case {cfg.get('name')} {({k: v for k, v in cfg.items() if k not in ('name',)})}")
    prob = synth.make_problem(cfg)
    if mutate:
        mutate(prob)
    res, err = full_check(prob, fields)
    say(f"  ok: score err {err['score_ratio']:.3f} of bound, attention err {err['attn_err']:.2e}, "
        f"end-to-end err {err['e2e_err']:.2e} ({err['swapped']} of {prob.R} rows with a tie-band swap)")
    return prob, res


def test_tiny_fp32_full():
    _run(synth.get("tiny_fp32"))


def test_tiny_fp32_short_and_ragged():
    _run(synth.get("tiny_fp32", lengths=[1000], k=256, H=3, H_I=3, d_I=40, anchors=4))
    _run(synth.get("tiny_fp32", lengths=[200], k=256, H=5, anchors=4))  # k > n: read in full


def test_decode_fp8_bf16_ragged():
    _run(synth.get("decode_128k", lengths=[20000], anchors=64, recent=96))


def test_decode_128k_full_size():
    _run(synth.get("decode_128k"))


def test_batched_paged_mixed_lengths():
    _run(synth.get("batched_paged", batch=6, length_range=(3000, 9000)))


def test_batched_short_empty_and_tiny_rows():
    # one empty row, one single-position row, one row shorter than k, one longer
    _run(synth.get("batched_paged", batch=4, lengths=[0, 1, 1500, 6000], anchors=8, recent=8))


def test_indexer_ranked_floor_rows():
    # rows of 16K..2^20 positions take the top-k floor that the fused step's indexer ranks from sampled keys
    # (the separate calls rank the filter's own sample, and the two selections must agree bit for bit): the
    # shortest such row and one just below it, k = 4096 at 2^17 and k = 2048 at 2^18 (the rule's edges), and a
    # paged batch with rows on both sides of 16K
    _run(synth.get("decode_128k", lengths=[16384], H=16, anchors=64, recent=96))
    _run(synth.get("decode_128k", lengths=[16383], H=16, anchors=64, recent=96))
    _run(synth.get("decode_128k", lengths=[1 << 17], k=4096, H=16))
    _run(synth.get("decode_128k", lengths=[1 << 18], H=16))
    _run(synth.get("decode_128k", lengths=[600001], H=16))  # 4096 samples, taken in eight rounds
    _run(synth.get("batched_paged", batch=4, lengths=[9000, 16384, 40000, 70001], H=32))


def _scale_sampled_keys(prob, factor):
    """Multiplies the key scale of the positions the fused indexer samples for a row's floor (runs of four, run j
    of `runs` at j n / runs rounded down to a multiple of four; 128 runs for a single row of up to 2^17 positions
    with k <= 2048, 256 up to 2^18 positions, else 1024): every score of row 0 there scales by `factor`."""
    n = int(prob.row_len[0])
    runs = 128 if prob.R == 1 and n <= (1 << 17) and min(prob.k, n) <= 2048 else 256 if n <= (1 << 18) else 1024
    pos = np.array([((j * n) // runs) // 4 * 4 + c for j in range(runs) for c in range(4)])
    ps = prob.page_size
    phys = prob.page_table[prob.row_seq[0], pos // ps].astype(np.int64) * ps + pos % ps
    prob.k_idx_scale[phys] *= np.float32(factor)


def test_indexer_floor_misjudged_either_way():
    # sampled keys scaled up 8x: the floor sits above all but a few dozen scores, fewer than k, so the row is selected
    # over its stored scores; scaled down 8x: nearly every score reaches the floor, the candidate list overflows,
    # and the same rescan settles it.  Both stay exact.
    _run(synth.get("decode_128k", lengths=[1 << 17], H=16), mutate=lambda p: _scale_sampled_keys(p, 8.0))
    _run(synth.get("decode_128k", lengths=[40000], H=16, anchors=64, recent=96),
         mutate=lambda p: _scale_sampled_keys(p, 0.125))
    _run(synth.get("decode_128k", lengths=[1 << 19], H=16), mutate=lambda p: _scale_sampled_keys(p, 8.0))


def test_index_heads_32_and_small_budgets():
    _run(synth.get("decode_128k", lengths=[9000], H_I=32, k=100, anchors=16, recent=32))
    _run(synth.get("decode_128k", lengths=[5000], k=1, H=16, anchors=16, recent=32))


def test_index_dim_128_and_shipped_budgets():
    # the shipped indexer shape (64 heads x 128 dims: two chained fp8 MFMAs per unit) at budgets 2048, 1024 and
    # 512; decode rows, a paged batch, 32 index heads, and chunked-prefill rows (the per-row kernel serves them)
    _run(synth.get("decode_128k", lengths=[20000], d_I=128, anchors=64, recent=96))
    _run(synth.get("batched_paged", batch=5, length_range=(3000, 9000), d_I=128, k=1024, H=32))
    _run(synth.get("decode_128k", lengths=[9000], H_I=32, d_I=128, k=512, H=16, anchors=16, recent=32))
    _run(synth.get("prefill_chunk", cache_len=6000, rows=24, H=32, d_I=128, k=1024))


def test_large_budgets_multi_chunk_splits():
    # k = 8000 over one row: the 16-head kernel runs two 64-slot chunks per split (63 splits, register gathers
    # double-buffered); k = 8192 over two rows: the all-heads kernel with splits of its own, merged by the combine
    _run(synth.get("decode_128k", lengths=[100000], k=8000, anchors=64, recent=128))
    _run(synth.get("decode_128k", lengths=[40000, 30000], k=8192, H=128, anchors=64, recent=128))  # 128 splits


def test_softmax_scale_and_signed_weights():
    def signed(prob):
        rng = np.random.default_rng(123)
        prob.head_w[:] = rng.uniform(-1, 1, size=prob.head_w.shape).astype(np.float32)
    prob, res = _run(synth.get("decode_128k", lengths=[7000], softmax_scale=1 / math.sqrt(512), H=32,
                               anchors=16, recent=32), mutate=signed)
    assert (res.scores[0, :7000] < 0).any()


def test_prefill_chunk_rows_share_the_cache():
    prob, res = _run(synth.get("prefill_chunk", cache_len=9000, rows=40, H=32))
    assert prob.row_len.tolist() == list(range(8961, 9001))


def test_prefill_several_paged_sequences():
    # 3 paged sequences x 37 causal rows: tiles of 16 rows never straddle two sequences, the last is ragged
    prob, res = _run(synth.get("prefill_paged"))
    assert prob.rows_per_seq == 37 and prob.R == 111


@pytest.mark.parametrize("rows,H_I", [(8, 64), (9, 64), (16, 32), (23, 32)])
def test_prefill_tiled_row_groups(rows, H_I):
    # row tiles of 16 made of two 8-row groups: exactly one group, a group plus one row, 32 heads, ragged
    _run(synth.get("prefill_paged", rows=rows, H_I=H_I, batch=2, k=700, H=16))


@pytest.mark.parametrize("rows,H_I", [(8, 64), (9, 64), (23, 32)])
def test_prefill_tiled_index_dim_128(rows, H_I):
    # the shipped 64 x 128 indexer keys through the tiled kernel: two chained fp8 MFMAs per unit and a 128-wide
    # linear term over eight bf16 K-steps
    _run(synth.get("prefill_paged", rows=rows, H_I=H_I, batch=2, k=700, H=16, d_I=128))


def test_prefill_selection_ties_take_the_fallback():
    # zero head weights make every score 0: each row's 9000 candidates tie at the threshold, more than the resolve
    # sorts out itself, so every row goes to the fallback, which must take the lowest positions
    def zero_weights(p):
        p.head_w[:] = 0.0
    prob, res = _run(synth.get("prefill_chunk", cache_len=9000, rows=24, H=16), mutate=zero_weights)
    for r in range(prob.R):
        keff = min(prob.k, int(prob.row_len[r]))
        assert np.array_equal(res.idx_step[r, :keff], np.arange(keff)), f"row {r}: not the lowest positions"


def test_prefill_selection_rows_past_the_candidate_list():
    # zero head weights again, on rows longer than the candidate list (20000 positions): the filter overflows
    def zero_weights(p):
        p.head_w[:] = 0.0
    _run(synth.get("prefill_chunk", cache_len=20000, rows=16, H=16, k=512), mutate=zero_weights)


def test_tiled_scores_leave_positions_past_each_row_untouched():
    # rows of one sequence (the tiled indexer) into a score buffer whose stride is tight and no multiple of the
    # 512-position pass: every entry at or past a row's length keeps its sentinel, every entry before it is written
    from synth.device import upload
    prob = synth.make_problem(synth.get("prefill_chunk", cache_len=9000, rows=24, H=16))
    say(f"sentinel case R={prob.R} n={int(prob.row_len.min())}..{int(prob.row_len.max())}")
    d = upload(prob, "cuda:0")
    P = dsa.make_problem(**d.fields)
    L = dsa.make_layout(d.row_seq, d.row_len, d.page_table)
    ld = (int(prob.row_len.max()) + 3) // 4 * 4 + 4
    assert ld % 512 != 0 and P.rows_per_seq >= 8
    sentinel = 12345.0
    scores = torch.full((prob.R, ld), sentinel, dtype=torch.float32, device="cuda:0")
    dsa.dsa_indexer_scores(P, L, d.q_idx, d.q_idx_scale, d.head_w, d.k_idx_pool, d.k_idx_scale, scores, ld)
    torch.cuda.synchronize()
    got = scores.cpu().numpy()
    for r in range(prob.R):
        n = int(prob.row_len[r])
        assert (got[r, n:] == sentinel).all(), f"row {r}: entries past n = {n} were written"
        assert not (got[r, :n] == sentinel).any(), f"row {r}: an entry below n = {n} was not written"
    say("  ok: only each row's visible positions were written")


def test_prefill_rows_through_the_per_row_kernel():
    # the same prefill chunk declared as independent rows runs the per-row kernel and must agree as well
    _run(synth.get("prefill_paged", rows=20, H=16), fields=dict(rows_per_seq=1))


@pytest.mark.parametrize("H", [96, 256])
def test_attention_head_counts(H):
    # 96 heads: three 32-head waves per block; 256 heads: two head groups of 128 per row
    _run(synth.get("batched_paged", batch=2, length_range=(2500, 5000), H=H, anchors=16, recent=32))


@pytest.mark.parametrize("batch", [1, 4])
def test_attention_wide_logit_range(batch):
    # logits spanning hundreds of units.  One row runs the 16-head kernel (online rescaling); four rows run
    # the all-heads kernel, where a later chunk's maximum far above the first chunk's forces the recompute
    # against exact per-head maxima
    _run(synth.get("batched_paged", batch=batch, length_range=(6000, 9000), softmax_scale=60.0, anchors=16,
                   recent=32))


@pytest.mark.parametrize("batch,H,k", [(8, 128, 2048), (16, 128, 2048), (32, 128, 2048), (64, 128, 2048),
                                         (64, 16, 4096)])
def test_split_merge_one_wave_per_row_head(batch, H, k):
    # 1024 or more (row, head) pairs.  The all-heads kernel splits each row 32, 16, 8 and 4 ways at 8, 16, 32 and
    # 64 rows; up to 16 splits are merged by one wave per pair, 32 by a block per pair.  The 16-head kernel
    # splits a 4096-slot budget 64 ways (block-per-pair merge)
    def rows(p):
        return [0, p.R // 2, p.R - 1]
    _sampled("batched_paged", rows, batch=batch, length_range=(k + 300, 2 * k + 700), H=H, k=k, anchors=16,
             recent=32)


def test_paged_equals_contiguous_bit_for_bit():
    cfg = synth.get("batched_paged", batch=3, length_range=(2500, 7000), H=32)
    a = gpu_step(synth.make_problem(cfg))
    b = gpu_step(synth.make_problem(dict(cfg, paged=False)))
    assert np.array_equal(a.idx, b.idx) and np.array_equal(a.out, b.out) and np.array_equal(a.lse, b.lse)


def test_rerun_is_bit_identical():
    prob = synth.make_problem(synth.get("decode_128k", lengths=[12000], H=64))
    a, b = gpu_step(prob), gpu_step(prob)
    assert np.array_equal(a.scores[:, :12000], b.scores[:, :12000])
    assert np.array_equal(a.idx, b.idx) and np.array_equal(a.out, b.out)


# ---------------------------------------------------------------------------- full-size workloads, sampled

def _sampled(name, rows_fn, **overrides):
    cfg = synth.get(name, **overrides)
    say(f"case {name} full size {overrides or ''}")
    prob = synth.make_problem(cfg)
    rows = rows_fn(prob)
    res, err = sampled_check(prob, rows)
    say(f"  ok: rows {list(rows)}: score err {err['score_ratio']:.3f} of bound, attention err {err['attn_err']:.2e}, "
        f"end-to-end err {err['e2e_err']:.2e} ({err['swapped']} rows with a tie-band swap)")
    return prob, res


def test_batched_paged_full_size():
    # the shortest and longest sequences plus a few others, out of 64 paged sequences
    def rows(p):
        order = np.argsort(p.row_len)
        return sorted({int(order[0]), int(order[-1]), 5, 31, 62})
    _sampled("batched_paged", rows)


def test_prefill_chunk_full_size():
    # first, last (= the decode_128k query) and interior rows of the 4096-row causal chunk
    prob, res = _sampled("prefill_chunk", lambda p: [0, 1, 1000, 2047, 4094, 4095])


@pytest.mark.slow
def test_decode_1m_full_size():
    # 8 sequences of 2^20 positions; two rows checked against the oracle
    _sampled("decode_1m", lambda p: [0, 7])


# ------------------------------------------------------------------------------- dense attention fallback

def _dense(cfg):
    say(f"dense case {({k: v for k, v in cfg.items() if k not in ('name',)})}")
    from synth.device import upload
    prob = synth.make_problem(cfg)
    d = upload(prob)
    P = dsa.make_problem(**d.fields)
    L = dsa.make_layout(d.row_seq, d.row_len, d.page_table)
    out_dt = torch.float32 if prob.kv_dtype == "f32" else torch.bfloat16
    out = torch.empty((prob.R, prob.H, prob.d_c), dtype=out_dt, device="cuda")
    lse = torch.empty((prob.R, prob.H), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(dsa.dsa_workspace_bytes(P, dsa.DSA_OP_DENSE), 256), dtype=torch.uint8, device="cuda")
    dsa.dsa_dense_mla_attn(P, L, d.q, d.kv_pool, out, lse, ws)
    torch.cuda.synchronize()
    width = max(1, int(prob.row_len.max()))
    idx = np.full((prob.R, width), -1, np.int32)
    for r in range(prob.R):
        idx[r, :prob.row_len[r]] = np.arange(prob.row_len[r], dtype=np.int32)
    err = check_attention(prob, out.float().cpu().numpy(), lse.cpu().numpy(), idx)
    say(f"  ok: dense attention err {err:.2e}")


def test_dense_attention_every_visible_position():
    # the short-context fallback: attention over positions 0 .. n_r - 1 of every row, no indexer or selection
    _dense(synth.get("decode_128k", lengths=[5000], anchors=64, recent=96))          # 16-head kernel, 40 splits
    _dense(synth.get("decode_128k", lengths=[60000], anchors=64, recent=96, H=32))   # 235 splits of 4 chunks
    _dense(synth.get("batched_paged", batch=4, lengths=[9000, 3000, 0, 1], H=128, anchors=8, recent=8))  # all heads
    _dense(synth.get("tiny_fp32", lengths=[1000, 4095], H=8))                         # fp32 path
    _dense(synth.get("decode_128k", lengths=[7000], anchors=64, recent=96, kv_dtype="f8", H=32))  # fp8 entries


# ----------------------------------------------------------------------------------- FP8 latent cache entries

def test_fp8_latent_entries_decode_and_paged():
    # 656-byte entries (e4m3 latent, 4 tile scales, bf16 RoPE) through the 16-head kernel: one long row with
    # several splits, and a paged batch with an empty, a one-position and a short row; 16 and 32 heads
    _run(synth.get("decode_128k", lengths=[20000], anchors=64, recent=96, kv_dtype="f8"))
    _run(synth.get("batched_paged", batch=5, lengths=[0, 1, 1500, 6000, 9000], anchors=8, recent=8, kv_dtype="f8",
                   H=16))
    _run(synth.get("batched_paged", batch=3, length_range=(3000, 9000), kv_dtype="f8", H=32, k=512))


def _large_fp8_latents(prob, seed=41):
    # every entry's 512 latent codes drawn from the e4m3 values of magnitude 256..448 (exponent field 15, signed)
    # with all four tile scales 1/60, so every dequantised latent value lies in [4.26, 7.47]
    rng = np.random.default_rng(seed)
    n = prob.kv_pool.shape[0]
    mag = rng.integers(0x78, 0x7F, size=(n, 512), dtype=np.uint8)
    prob.kv_pool[:, :512] = mag | (rng.integers(0, 2, size=(n, 512), dtype=np.uint8) << 7)
    prob.kv_pool[:, 512:528] = np.full((n, 4), 1.0 / 60.0, np.float32).view(np.uint8)


@pytest.mark.parametrize("batch,H", [(4, 16), (128, 128)])
def test_fp8_latent_large_values_one_and_two_positions(batch, H):
    # Rows of one and two positions over entries whose dequantised latent values lie in [4, 8): a one-position row's
    # output is its latent row, a two-position row's a convex combination of two.  Every product of a probability
    # and a tile scale reaches the MFMAs unrounded, so the only error left is the bf16 rounding of the output, at
    # most half a bf16 ulp of |o| (1/64 in [4, 8)); rounding those products to bf16 would add up to 8 * 2^-9.
    # 4 rows of 16 heads run the 16-head kernel; 128 rows of 128 heads (128 row-chunks) the all-heads kernel.
    say(f"case large fp8 latents batch={batch} H={H}")
    prob = synth.make_problem(synth.get("batched_paged", batch=batch, lengths=[1, 2] * (batch // 2), anchors=0,
                                        recent=0, kv_dtype="f8", H=H, k=64, seed=40))
    _large_fp8_latents(prob)
    res = gpu_step(prob)
    ref_o, ref_lse = oracle.sparse_attn_fp8(prob.q, prob.kv_pool, res.idx, prob.row_seq, prob.page_table,
                                            prob.page_size, prob.softmax_scale)
    # half a bf16 ulp (8 significant bits) of the larger of |o| and |o_gpu|, plus 2^-12 for the fp32 sums where a
    # two-position row's mixed signs bring o near zero
    mag = np.maximum(np.maximum(np.abs(ref_o), np.abs(res.out)), 1e-30)
    bound = np.exp2(np.floor(np.log2(mag)) - 8) + 2.0 ** -12
    err = np.abs(res.out - ref_o)
    say(f"  max err {err.max():.3e}, max |o| {np.abs(ref_o).max():.2f}, worst err / bound {(err / bound).max():.3f}")
    assert np.abs(ref_o).max() > 4.0
    assert (err <= bound).all()
    assert err.max() <= 2e-2
    assert np.abs(res.lse - ref_lse).max() <= 1e-3
    assert np.array_equal(res.out_step, res.out)


def test_fp8_latent_with_prefill_rows_and_wide_index_keys():
    # FP8 entries under chunked-prefill rows (the tiled indexer, rows of one sequence) and with the shipped
    # 64 x 128 indexer keys over a paged batch
    _run(synth.get("prefill_chunk", cache_len=6000, rows=24, H=32, kv_dtype="f8"))
    _run(synth.get("batched_paged", batch=3, length_range=(3000, 9000), d_I=128, k=1024, H=32, kv_dtype="f8"))


def test_fp8_latent_full_size():
    # the 128K decode workload over fp8 entries, checked element by element against the oracle
    _sampled("decode_128k_fp8kv", lambda p: [0])


def test_fp8_latent_all_heads_kernel():
    # 128 heads over fp8 entries with at least 128 (row, chunk) units run the all-heads kernel: a paged batch with
    # an empty, a one-position and a short row (160 units), and logits spanning hundreds of units, where a later
    # chunk's maximum far above the first chunk's forces the recompute against exact per-head maxima (128 units)
    _run(synth.get("batched_paged", batch=5, lengths=[0, 1, 1500, 6000, 9000], anchors=8, recent=8, kv_dtype="f8",
                   H=128))
    _run(synth.get("batched_paged", batch=4, length_range=(6000, 9000), softmax_scale=60.0, anchors=16, recent=32,
                   kv_dtype="f8", H=128))


def test_fp8_latent_all_heads_dense():
    # dense attention over fp8 entries through the all-heads kernel (every visible position of each row)
    _dense(synth.get("batched_paged", batch=4, lengths=[9000, 3000, 0, 1], H=128, anchors=8, recent=8,
                     kv_dtype="f8"))


def test_batched_paged_fp8kv_full_size():
    # 64 paged sequences over fp8 entries (the all-heads kernel with four splits per row), sampled rows
    def rows(p):
        order = np.argsort(p.row_len)
        return sorted({int(order[0]), int(order[-1]), 7, 40})
    _sampled("batched_paged_fp8kv", rows)


# ------------------------------------------------------------------------------- top-k on crafted scores

def _topk_only(scores_np, row_len, k):
    R, n = scores_np.shape
    ld = max(4, -(-n // 4) * 4)
    dev = "cuda"
    s = torch.zeros((R, ld), dtype=torch.float32, device=dev)
    s[:, :n] = torch.from_numpy(scores_np.astype(np.float32)).to(dev)
    pages = max(1, -(-max(max(row_len), 1) // 64))
    P = dsa.make_problem(num_rows=R, num_seqs=1, topk=k, page_size=64, max_pages=pages, num_pages=pages,
                         max_row_len=max(row_len))
    rl = torch.tensor(row_len, dtype=torch.int32, device=dev)
    rs = torch.zeros(R, dtype=torch.int32, device=dev)
    pt = torch.zeros((1, pages), dtype=torch.int32, device=dev)
    L = dsa.make_layout(rs, rl, pt)
    idx = torch.empty((R, k), dtype=torch.int32, device=dev)
    ws = torch.empty(dsa.dsa_workspace_bytes(P, dsa.DSA_OP_TOPK), dtype=torch.uint8, device=dev)
    dsa.dsa_topk(P, L, s, idx, ws, ld)
    torch.cuda.synchronize()
    return idx.cpu().numpy()


def _expect_exact(scores_np, row_len, k):
    got = _topk_only(scores_np, row_len, k)
    ref, _ = oracle.topk(scores_np.astype(np.float32).astype(np.float64), row_len, k)
    for r in range(len(row_len)):
        keff = min(k, row_len[r])
        assert np.array_equal(got[r, :keff], np.sort(ref[r, :keff])), f"row {r}"
        assert (got[r, keff:] == -1).all()


def test_topk_heavy_ties_in_lds_path():
    rng = np.random.default_rng(5)
    sc = rng.integers(0, 4, size=(3, 9000)).astype(np.float32)
    _expect_exact(sc, [9000, 8191, 4097], 2048)


def test_topk_all_equal_uses_the_row_rescan():
    sc = np.full((2, 20000), 0.5, np.float32)   # every score ties: candidates overflow the LDS list
    sc[1, 123] = 0.75
    _expect_exact(sc, [20000, 19999], 2048)


def test_topk_negative_zero_and_signs():
    rng = np.random.default_rng(6)
    sc = rng.standard_normal((2, 6000)).astype(np.float32)
    sc[0, ::7] = 0.0
    sc[0, 3::7] = -0.0
    sc[1] = -np.abs(sc[1])
    _expect_exact(sc, [6000, 6000], 3000)
    _expect_exact(sc, [6000, 6000], 5999)


def test_topk_staged_flush_and_ties():
    # one filter block's chunks hold 10000 tied candidates: more than it stages at once (it reserves list space
    # twice), fewer than the row's candidate list holds (the resolve keeps its LDS path); lowest positions win
    rng = np.random.default_rng(8)
    n = 1 << 20
    sc = rng.standard_normal((1, n)).astype(np.float32)
    sc[0, 300000:310000] = 100.0
    _expect_exact(sc, [n], 2048)


def test_topk_sample_overshoot_rescans_the_row():
    # a row of 2^17 is sampled as 1024 runs of four scores, one run every 128 positions; only the first 40 runs
    # hold high scores, so the sample's floor sits above all but 160 scores, fewer than k, and the resolve rescans
    # the whole row
    rng = np.random.default_rng(9)
    n = 1 << 17
    sc = rng.standard_normal((1, n)).astype(np.float32)
    for j in range(40):
        sc[0, 128 * j:128 * j + 4] = 50.0
    _expect_exact(sc, [n], 2048)


def test_topk_threshold_far_above_the_floor():
    # k + 100 scores near 1000 at random positions above a standard-normal bulk: the sample's floor lies in the
    # bulk, and the k-th largest score beyond the two octaves above it that the candidate histogram resolves (in
    # its open-ended top bin), so the resolve radix-selects its candidate list
    rng = np.random.default_rng(10)
    n = 1 << 17
    sc = rng.standard_normal((2, n)).astype(np.float32)
    for r in range(2):
        hi = rng.choice(n, 2148, replace=False)
        sc[r, hi] = 1000.0 + rng.standard_normal(len(hi)).astype(np.float32)
    _expect_exact(sc, [n, n - 77], 2048)


def test_topk_long_row_1m():
    rng = np.random.default_rng(7)
    n = 1 << 20
    sc = rng.standard_normal((1, n)).astype(np.float32) * 3 + 10
    _expect_exact(sc, [n], 2048)
