"""Pins of the CPU oracle against things other than itself.

Each check reduces an oracle function to a library routine, a closed form, a brute-force definition, a value
printed on the pages, or an invariant the method's definition implies, so that a dropped term, a wrong sign,
a wrong head/position index or a transposed operand in the oracle fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------------------------- codecs

def test_e4m3_all_codes_match_torch_cast():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.decode(codes, "f8")
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(mine[~nan], ref[~nan])


def test_e4m3_closed_forms():
    v = oracle.decode(np.array([0x7E, 0x01, 0x08, 0x38, 0xB8, 0x00, 0x80, 0x07], np.uint8), "f8")
    # largest finite 448, smallest subnormal 2^-9, smallest normal 2^-6, 1.0, -1.0, +0, -0, largest subnormal 7*2^-9
    assert list(v[:5]) == [448.0, 2.0 ** -9, 2.0 ** -6, 1.0, -1.0]
    assert v[5] == 0.0 and v[6] == 0.0 and math.copysign(1, v[6]) == -1
    assert v[7] == 7 * 2.0 ** -9


def test_bf16_matches_torch_cast():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2 ** 16, size=20000, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]  # drop inf/NaN patterns
    mine = oracle.decode(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(mine, ref)


# --------------------------------------------------------------------------------------------- indexer

def _contig_layout(n, S=1):
    """Identity page table for S sequences of n positions (page size 64)."""
    pages = -(-n // 64)
    return np.arange(S * pages, dtype=np.int32).reshape(S, pages)


def _rand_f8_problem(rng, R=2, H_I=8, d_I=64, n=300):
    q8 = rng.integers(0, 256, size=(R, H_I, d_I), dtype=np.uint8)
    k8 = rng.integers(0, 256, size=(-(-n // 64) * 64, d_I), dtype=np.uint8)
    q8[(q8 & 0x7F) == 0x7F] = 0x38  # no NaN codes
    k8[(k8 & 0x7F) == 0x7F] = 0x38
    sq = rng.uniform(0.5, 2.0, size=(R, H_I)).astype(np.float32)
    sk = rng.uniform(0.5, 2.0, size=k8.shape[0]).astype(np.float32)
    w = rng.uniform(-1.0, 1.0, size=(R, H_I)).astype(np.float32)
    return q8, sq, w, k8, sk


def _scores(q, sq, w, k, sk, n, dtype, pt=None, row_seq=None):
    R = q.shape[0]
    pt = _contig_layout(n) if pt is None else pt
    row_seq = np.zeros(R, np.int32) if row_seq is None else row_seq
    return oracle.indexer_scores(q, sq, w, k, sk, row_seq, np.full(R, n, np.int32), pt, 64, dtype)


def test_indexer_worked_example_from_the_pages():
    g = json.load(open(os.path.join(GOLDEN, "indexer_worked_example.json")))
    keys = np.array(g["keys_1based_tokens"], np.float32)
    n = keys.shape[0]
    pool = np.zeros((64, g["d_I"]), np.float32)
    pool[:n] = keys
    q = np.array(g["q_idx"], np.float32)[None]
    w = np.array(g["head_w"], np.float32)[None]
    sc = _scores(q, None, w, pool, None, n, "f32")
    assert np.allclose(sc[0], g["expected_scores"], atol=g["tolerance_abs"], rtol=0)
    for tok, val in g["printed_values"].items():
        assert abs(sc[0, int(tok) - 1] - val) < g["tolerance_abs"]
    assert (sc[0] < 0).any()  # signed head weights give negative scores
    idx, kth = oracle.topk(sc, [n], g["budget"])
    assert [i + 1 for i in idx[0]] == g["expected_kept_tokens_1based_in_order"]
    assert abs(kth[0] - 6.4) < g["tolerance_abs"]


def test_indexer_single_head_unit_weight_is_relu_of_matmul_f8_exact():
    """H_I = 1, w = 1, unit scales: I = max(0, q.k); with fp8 operands every dot is exact in fp64, so it must
    equal float64 numpy matmul of the torch-decoded codes bit for bit."""
    rng = np.random.default_rng(1)
    q8, _, _, k8, _ = _rand_f8_problem(rng, R=3, H_I=1, n=256)
    ones_q, ones_k = np.ones((3, 1), np.float32), np.ones(k8.shape[0], np.float32)
    sc = _scores(q8, ones_q, np.ones((3, 1), np.float32), k8, ones_k, 256, "f8")
    dq = torch.from_numpy(q8).view(torch.float8_e4m3fn).to(torch.float64).numpy()[:, 0, :]
    dk = torch.from_numpy(k8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ref = np.maximum(dq @ dk[:256].T, 0.0)
    assert np.array_equal(sc, ref)


def test_indexer_single_head_f32_is_relu_of_matmul():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((2, 1, 64)).astype(np.float32)
    k = rng.standard_normal((128, 64)).astype(np.float32)
    sc = _scores(q, None, np.ones((2, 1), np.float32), k, None, 128, "f32")
    ref = np.maximum(q[:, 0, :].astype(np.float64) @ k.astype(np.float64).T, 0.0)
    assert np.allclose(sc, ref, rtol=1e-12, atol=1e-12)


def test_indexer_is_sum_over_heads_of_single_head_scores():
    rng = np.random.default_rng(3)
    q8, sq, w, k8, sk = _rand_f8_problem(rng)
    full = _scores(q8, sq, w, k8, sk, 300, "f8")
    parts = sum(_scores(q8[:, j:j + 1], sq[:, j:j + 1], w[:, j:j + 1], k8, sk, 300, "f8") for j in range(q8.shape[1]))
    assert np.allclose(full, parts, rtol=1e-12, atol=1e-12)


def test_indexer_single_head_scales_and_weight_factor_out():
    """Positive scales and the head weight multiply the single-head score: w*sq*sk*max(0, dot of codes)."""
    rng = np.random.default_rng(4)
    q8, sq, w, k8, sk = _rand_f8_problem(rng, R=2, H_I=1)
    unit = _scores(q8, np.ones_like(sq), np.ones_like(w), k8, np.ones_like(sk), 300, "f8")
    scaled = _scores(q8, sq, w, k8, sk, 300, "f8")
    expect = unit * (w.astype(np.float64) * sq.astype(np.float64)) * sk[:300].astype(np.float64)[None, :]
    assert np.allclose(scaled, expect, rtol=1e-12, atol=1e-12)


def test_indexer_per_head_relu_nonnegative_and_zero_on_negative_dots():
    rng = np.random.default_rng(5)
    q8, sq, w, k8, sk = _rand_f8_problem(rng, R=1, H_I=4)
    for j in range(4):
        onehot = np.zeros((1, 4), np.float32)
        onehot[0, j] = 1.0
        sc = _scores(q8, sq, onehot, k8, sk, 300, "f8")
        dq = torch.from_numpy(q8[0, j]).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        dk = torch.from_numpy(k8[:300]).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        dots = dk @ dq
        assert (sc >= 0).all()
        assert (sc[0][dots <= 0] == 0).all() and (sc[0][dots > 0] > 0).all()


def test_indexer_weight_linearity_and_sign():
    rng = np.random.default_rng(6)
    q8, sq, w, k8, sk = _rand_f8_problem(rng)
    base = _scores(q8, sq, w, k8, sk, 300, "f8")
    assert np.array_equal(_scores(q8, sq, 2 * w, k8, sk, 300, "f8"), 2 * base)
    assert np.array_equal(_scores(q8, sq, -w, k8, sk, 300, "f8"), -base)


def test_indexer_paging_and_position_permutation():
    """A random page table over a permuted pool gives the same scores; permuting the cache permutes them."""
    rng = np.random.default_rng(7)
    q8, sq, w, k8, sk = _rand_f8_problem(rng, n=320)
    base = _scores(q8, sq, w, k8, sk, 320, "f8")
    perm = rng.permutation(5).astype(np.int32)
    pk8, psk = np.empty_like(k8), np.empty_like(sk)
    for lp in range(5):
        pk8[perm[lp] * 64:(perm[lp] + 1) * 64] = k8[lp * 64:(lp + 1) * 64]
        psk[perm[lp] * 64:(perm[lp] + 1) * 64] = sk[lp * 64:(lp + 1) * 64]
    paged = _scores(q8, sq, w, pk8, psk, 320, "f8", pt=perm[None, :])
    assert np.array_equal(base, paged)
    sperm = rng.permutation(320)
    moved = _scores(q8, sq, w, k8[sperm], sk[sperm], 320, "f8")
    assert np.array_equal(moved, base[:, sperm])


def test_indexer_rows_see_only_their_prefix_and_their_sequence():
    rng = np.random.default_rng(8)
    q8, sq, w, k8, sk = _rand_f8_problem(rng, R=2, n=256)
    # two sequences of 128 positions each in one pool; row 0 -> seq 1 with 100 visible, row 1 -> seq 0 with 128
    pt = np.array([[0, 1], [2, 3]], np.int32)
    sc = oracle.indexer_scores(q8, sq, w, k8, sk, np.array([1, 0], np.int32), np.array([100, 128], np.int32),
                               pt, 64, "f8", ld=128)
    alone1 = oracle.indexer_scores(q8[:1], sq[:1], w[:1], k8[128:], sk[128:], np.zeros(1, np.int32),
                                   np.array([100], np.int32), _contig_layout(128), 64, "f8", ld=128)
    assert np.array_equal(sc[0, :100], alone1[0, :100]) and np.isnan(sc[0, 100:]).all()
    alone0 = _scores(q8[1:], sq[1:], w[1:], k8[:128], sk[:128], 128, "f8")
    assert np.array_equal(sc[1], alone0[0])


def test_p1_sketch_special_case_same_selection():
    """The lizeman sketch scores one head as (k_I @ q_I)/sqrt(d_I) with no ReLU.  With one head, unit weight and
    every dot positive, the ReLU is inactive and a positive factor cannot change the order, so the selected set
    must equal torch.topk of the sketch's scores."""
    rng = np.random.default_rng(9)
    d_I, n, k = 64, 500, 37
    q = np.abs(rng.standard_normal((1, 1, d_I))).astype(np.float32)
    kk = np.abs(rng.standard_normal((-(-n // 64) * 64, d_I))).astype(np.float32)
    sc = _scores(q, None, np.ones((1, 1), np.float32), kk, None, n, "f32")
    idx, _ = oracle.topk(sc, [n], k)
    sketch = (torch.from_numpy(kk[:n]).double() @ torch.from_numpy(q[0, 0]).double()) / d_I ** 0.5
    assert set(idx[0].tolist()) == set(sketch.topk(k).indices.tolist())


# ----------------------------------------------------------------------------------------------- top-k

def _brute_force_selection(scores, k):
    """Definition by rank: position p is kept iff fewer than min(k, n) positions precede it in the order
    (higher score first, then lower position)."""
    n = len(scores)
    keff = min(k, n)
    rank = [sum(1 for s in range(n) if scores[s] > scores[p] or (scores[s] == scores[p] and s < p)) for p in range(n)]
    return [p for r in range(keff) for p in range(n) if rank[p] == r]


@settings(max_examples=300, deadline=None)
@given(st.lists(st.sampled_from([-2.0, -0.5, 0.0, 0.25, 1.0, 3.0, 7.5]), min_size=1, max_size=64),
       st.integers(min_value=1, max_value=66))
def test_topk_matches_rank_definition_with_ties(vals, k):
    sc = np.array([vals], np.float64)
    idx, kth = oracle.topk(sc, [len(vals)], k)
    expect = _brute_force_selection(vals, k)
    keff = min(k, len(vals))
    assert idx[0, :keff].tolist() == expect
    assert (idx[0, keff:] == -1).all()
    assert kth[0] == vals[expect[-1]]


def test_topk_matches_torch_topk_on_distinct_scores():
    rng = np.random.default_rng(10)
    sc = rng.standard_normal((3, 5000))
    for k in (1, 17, 2048, 4999, 5000, 6000):
        idx, kth = oracle.topk(sc, [5000, 5000, 5000], k)
        keff = min(k, 5000)
        for r in range(3):
            ref = torch.from_numpy(sc[r]).topk(keff)
            assert idx[r, :keff].tolist() == ref.indices.tolist()
            assert kth[r] == ref.values[-1].item()


def test_topk_short_row_reads_everything():
    sc = np.array([[3.0, 1.0, 2.0, np.nan, np.nan]])
    idx, kth = oracle.topk(sc, [3], 8)
    assert idx[0].tolist() == [0, 2, 1, -1, -1, -1, -1, -1] and kth[0] == 1.0


def test_topk_empty_row():
    idx, kth = oracle.topk(np.zeros((1, 4)), [0], 4)
    assert (idx == -1).all() and np.isnan(kth[0])


# ------------------------------------------------------------------------------------------- attention

def _attn_case(rng, n=200, H=4, d_c=64, dtype="f32"):
    c = rng.standard_normal((-(-n // 64) * 64, d_c)).astype(np.float32)
    q = (rng.standard_normal((1, H, d_c)) / math.sqrt(d_c)).astype(np.float32)
    if dtype == "bf16":
        c = torch.from_numpy(c).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        q = torch.from_numpy(q).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return q, c


def _as_f64(x, dtype):
    return oracle.decode(x, dtype)


def _attn(q, c, idx, n, dtype, scale, pt=None):
    pt = _contig_layout(n) if pt is None else pt
    return oracle.sparse_attn(q, c, np.asarray(idx, np.int32)[None], np.zeros(1, np.int32), pt, 64, dtype, scale)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("scale", [1.0, 1 / math.sqrt(64)])
def test_attention_full_selection_equals_dense_sdpa(dtype, scale):
    """k >= n selects every position, so the step must equal dense softmax attention (torch SDPA, fp64)."""
    rng = np.random.default_rng(11)
    n, H, d_c = 200, 4, 64
    q, c = _attn_case(rng, n, H, d_c, dtype)
    o, lse = _attn(q, c, np.arange(n), n, dtype, scale)
    Q = torch.from_numpy(_as_f64(q, dtype))[:, :, None, :]              # [1, H, 1, d]
    K = torch.from_numpy(_as_f64(c, dtype)[:n])[None, None].expand(1, H, n, d_c)
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, K, scale=scale)
    assert np.allclose(o, ref[:, :, 0, :].numpy(), rtol=1e-12, atol=1e-12)
    logits = (Q @ K.transpose(-1, -2))[:, :, 0, :] * scale
    assert np.allclose(lse, torch.logsumexp(logits, -1).numpy(), rtol=1e-12, atol=1e-12)


def test_attention_mask_form_equals_gather_form():
    """The selector's reference form: top-k then -inf outside the list, softmax over the whole row."""
    rng = np.random.default_rng(12)
    n, H, d_c = 300, 3, 32
    q, c = _attn_case(rng, n, H, d_c)
    sel = rng.choice(n, size=40, replace=False)
    o, lse = _attn(q, c, sel, n, "f32", 0.7)
    Q, K = torch.from_numpy(q.astype(np.float64))[0], torch.from_numpy(c[:n].astype(np.float64))
    logits = 0.7 * (Q @ K.T)
    mask = torch.full((n,), float("-inf"), dtype=torch.float64)
    mask[torch.from_numpy(sel)] = 0.0
    p = torch.softmax(logits + mask, dim=-1)
    assert np.allclose(o[0], (p @ K).numpy(), rtol=1e-12, atol=1e-13)


def test_attention_special_cases():
    rng = np.random.default_rng(13)
    n, H, d_c = 100, 2, 16
    q, c = _attn_case(rng, n, H, d_c)
    # one selected row: output is that row, lse is its logit
    o, lse = _attn(q, c, [37, -1, -1], n, "f32", 1.0)
    assert np.array_equal(o[0, 0], c[37].astype(np.float64))
    assert np.isclose(lse[0, 0], float(q[0, 0].astype(np.float64) @ c[37].astype(np.float64)), rtol=1e-14)
    # zero query: uniform weights, output is the mean of the selected rows, lse = log(count)
    sel = np.array([3, 9, 50, 77])
    o, lse = _attn(np.zeros_like(q), c, sel, n, "f32", 1.0)
    assert np.allclose(o[0, 1], c[sel].astype(np.float64).mean(0), rtol=1e-14, atol=1e-15)
    assert np.isclose(lse[0, 1], math.log(4))
    # empty selection
    o, lse = _attn(q, c, [-1, -1], n, "f32", 1.0)
    assert (o == 0).all() and np.isneginf(lse).all()


def test_attention_order_invariant_and_paged():
    rng = np.random.default_rng(14)
    n, H, d_c = 256, 3, 32
    q, c = _attn_case(rng, n, H, d_c)
    sel = rng.choice(n, size=50, replace=False)
    o1, l1 = _attn(q, c, sel, n, "f32", 1.0)
    o2, l2 = _attn(q, c, sel[::-1], n, "f32", 1.0)
    assert np.allclose(o1, o2, rtol=1e-13, atol=1e-14) and np.allclose(l1, l2, rtol=1e-14)
    perm = rng.permutation(4).astype(np.int32)
    pc = np.empty_like(c)
    for lp in range(4):
        pc[perm[lp] * 64:(perm[lp] + 1) * 64] = c[lp * 64:(lp + 1) * 64]
    o3, l3 = _attn(q, pc, sel, n, "f32", 1.0, pt=perm[None])
    assert np.array_equal(o1, o3) and np.array_equal(l1, l3)


def test_attention_heads_share_one_latent_row():
    """MQA: each head's output depends only on its own query and the shared rows."""
    rng = np.random.default_rng(15)
    n, H, d_c = 128, 4, 32
    q, c = _attn_case(rng, n, H, d_c)
    sel = rng.choice(n, size=20, replace=False)
    o_all, _ = _attn(q, c, sel, n, "f32", 1.0)
    for h in range(H):
        o_h, _ = _attn(q[:, h:h + 1], c, sel, n, "f32", 1.0)
        assert np.array_equal(o_all[0, h], o_h[0, 0])


# ------------------------------------------------------------------------------------ indexer-key append

def _e4m3_table():
    return oracle.decode(np.arange(256, dtype=np.uint8), "f8")


def test_e4m3_nearest_round_trips_every_finite_code():
    vals = _e4m3_table()
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert oracle.e4m3_nearest(np.float32(vals[c])) == c, hex(c)


def test_e4m3_nearest_midpoints_go_to_the_even_code():
    vals = _e4m3_table()
    for c in range(0x7E):
        mid = np.float32((vals[c] + vals[c + 1]) / 2)  # at most 5 significant bits: exact in fp32
        assert float(mid) == (vals[c] + vals[c + 1]) / 2
        even = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_nearest(mid) == even
        assert oracle.e4m3_nearest(np.nextafter(mid, np.float32(np.inf))) == c + 1
        assert oracle.e4m3_nearest(np.nextafter(mid, np.float32(-np.inf))) == c
        assert oracle.e4m3_nearest(-mid) == 0x80 | even


def test_e4m3_nearest_matches_torch_cast():
    # torch's float -> float8_e4m3fn conversion rounds to nearest even and keeps the sign bit
    rng = np.random.default_rng(11)
    mag = np.exp2(rng.uniform(-14, np.log2(448.0), 20000)).astype(np.float32)
    x = np.concatenate([mag * rng.choice([-1, 1], mag.size), np.float32([0.0, -0.0, 448.0, -448.0, 1e-30, -1e-30])])
    x = x.astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    mine = np.array([oracle.e4m3_nearest(v) for v in x], np.uint8)
    assert np.array_equal(mine, ref)
    assert oracle.e4m3_nearest(np.float32(1e6)) == 0x7E and oracle.e4m3_nearest(np.float32(-1e6)) == 0xFE


def test_quantize_key_closed_forms_and_error_bound():
    vals = _e4m3_table()
    # all-zero key: scale 1, zero codes
    codes, s = oracle.quantize_key(np.zeros(64, np.float32))
    assert s == 1.0 and not codes.any()
    # the largest magnitude takes the largest code, with its sign; a power-of-two amax gives an exact scale
    x = np.zeros(64, np.float32)
    x[5], x[9] = -7.0, 3.5
    codes, s = oracle.quantize_key(x)
    assert s == np.float32(7.0) / np.float32(448.0) and codes[5] == 0xFE and codes[9] == 0x76  # 3.5/7 * 448 = 224
    assert np.count_nonzero(codes) == 2
    # any key: every dequantised value lies within half an e4m3 step of the fp32 key
    rng = np.random.default_rng(5)
    for _ in range(50):
        x = (rng.standard_normal(128) * np.exp2(rng.uniform(-20, 20))).astype(np.float32)
        x[rng.integers(128)] *= 30  # one outlier: many small values fall in the subnormal range
        codes, s = oracle.quantize_key(x)
        assert s == np.float32(np.abs(x).max()) / np.float32(448.0)
        y = x.astype(np.float64) / s
        deq = vals[codes]
        normal = np.abs(y) >= 2.0 ** -6
        assert np.all(np.abs(deq - y)[normal] <= 2.0 ** -4 * np.abs(y)[normal] * (1 + 1e-6))
        assert np.all(np.abs(deq - y)[~normal] <= 2.0 ** -10 * (1 + 1e-6))
        assert np.array_equal(np.signbit(deq), np.signbit(y.astype(np.float32)))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_key_projection_exact_integer_matmul(dtype):
    # small integers: every product and partial sum is exact, so k = c W must equal the integer matmul; d_c != d_I
    # and an asymmetric W catch a transposed operand
    rng = np.random.default_rng(3)
    c = rng.integers(-8, 9, size=(5, 96)).astype(np.float32)
    w = rng.integers(-8, 9, size=(96, 40)).astype(np.float32)
    enc = (lambda a: torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)) \
        if dtype == "bf16" else (lambda a: a)
    k = oracle.key_projection(enc(c), enc(w), dtype)
    assert np.array_equal(k, c.astype(np.int64) @ w.astype(np.int64))


def test_key_projection_matches_library_matmul():
    rng = np.random.default_rng(4)
    c = rng.standard_normal((3, 512)).astype(np.float32)
    w = (rng.standard_normal((512, 128)) / 22).astype(np.float32)
    k = oracle.key_projection(c, w, "f32")
    assert np.allclose(k, c.astype(np.float64) @ w.astype(np.float64), rtol=1e-12, atol=1e-12)


def _enc_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy() \
        .view(np.uint16)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_query_projection_exact_integer_matmul_and_head_columns(dtype):
    # integer operands: q_I = h W_QI and w = h W_w are exact; head j must own columns j d_I .. j d_I + d_I - 1
    # (d_model, H_I, d_I all different so a transposed or mis-strided operand fails)
    rng = np.random.default_rng(11)
    R, d_model, H_I, d_I = 3, 80, 4, 16
    h = rng.integers(-6, 7, size=(R, d_model)).astype(np.float32)
    wq = rng.integers(-6, 7, size=(d_model, H_I * d_I)).astype(np.float32)
    ww = rng.integers(-6, 7, size=(d_model, H_I)).astype(np.float32)
    enc = _enc_bf16 if dtype == "bf16" else (lambda a: a)
    q, qs, w = oracle.query_projection(enc(h), enc(wq), enc(ww), H_I, dtype, "f32")
    exact_q = (h.astype(np.int64) @ wq.astype(np.int64)).reshape(R, H_I, d_I)
    assert qs is None and q.shape == (R, H_I, d_I)
    assert np.array_equal(q, exact_q) and np.array_equal(w, h.astype(np.int64) @ ww.astype(np.int64))


def test_query_projection_one_hot_state_gives_known_codes_and_per_head_scales():
    # h = e_d picks row d of W_QI; head j's slice is an e4m3-representable vector v_j (holding +-448) times 2^j, so
    # the scale is exactly 2^j and the codes are those of v_j
    vals = _e4m3_table()
    rng = np.random.default_rng(12)
    d_model, H_I, d_I, d = 24, 5, 32, 7
    wq = rng.standard_normal((d_model, H_I * d_I)).astype(np.float32)
    want = np.empty((H_I, d_I), np.uint8)
    for j in range(H_I):
        codes = rng.integers(0, 0x7F, d_I).astype(np.uint8) | (rng.integers(0, 2, d_I).astype(np.uint8) << 7)
        codes[rng.integers(d_I)] = 0x7E if j % 2 else 0xFE  # +448 or -448
        want[j] = codes
        wq[d, j * d_I:(j + 1) * d_I] = vals[codes] * 2.0 ** j
    ww = rng.standard_normal((d_model, H_I)).astype(np.float32)
    h = np.zeros((1, d_model), np.float32)
    h[0, d] = 1
    q, qs, w = oracle.query_projection(h, wq, ww, H_I, "f32", "f8")
    neg_zero = (want & 0x7F) == 0  # -0 in the weight is +0 after the sum
    assert np.array_equal(q[0][~neg_zero], want[~neg_zero]) and not (q[0][neg_zero] & 0x7F).any()
    assert np.array_equal(qs[0], 2.0 ** np.arange(H_I)) and np.array_equal(w[0], ww[d])


def test_query_projection_zero_state_power_of_two_scaling_and_empty():
    rng = np.random.default_rng(13)
    R, d_model, H_I, d_I = 4, 64, 8, 64
    h = rng.standard_normal((R, d_model)).astype(np.float32)
    wq = (rng.standard_normal((d_model, H_I * d_I)) / 8).astype(np.float32)
    ww = (rng.standard_normal((d_model, H_I)) / 8).astype(np.float32)
    q, qs, w = oracle.query_projection(np.zeros_like(h), wq, ww, H_I, "f32", "f8")
    assert not q.any() and (qs == 1).all() and not w.any()
    # scaling h by 2^m scales every sum exactly: codes unchanged, scales and head weights times 2^m
    q1, s1, w1 = oracle.query_projection(h, wq, ww, H_I, "f32", "f8")
    q2, s2, w2 = oracle.query_projection(h * 8, wq, ww, H_I, "f32", "f8")
    assert np.array_equal(q1, q2) and np.array_equal(s2, s1 * 8) and np.array_equal(w2, w1 * 8)
    # against a library fp64 matmul rounded to fp32 (both within one fp32 rounding of the exact sum)
    qf, _, wf = oracle.query_projection(h, wq, ww, H_I, "f32", "f32")
    ref_q = (h.astype(np.float64) @ wq.astype(np.float64)).reshape(R, H_I, d_I)
    assert np.allclose(qf, ref_q, rtol=2.0 ** -23, atol=1e-30)
    assert np.allclose(wf, h.astype(np.float64) @ ww.astype(np.float64), rtol=2.0 ** -23, atol=1e-30)
    # fp8 codes are the per-head quantisation of the fp32 projection
    for r in range(R):
        for j in range(H_I):
            c, sc = oracle.quantize_key(qf[r, j])
            assert np.array_equal(q1[r, j], c) and s1[r, j] == np.float32(sc)
    qe, se, we = oracle.query_projection(h[:0], wq, ww, H_I, "f32", "f8")
    assert qe.shape == (0, H_I, d_I) and se.shape == (0, H_I) and we.shape == (0, H_I)


def test_key_append_places_rows_through_the_page_table():
    page_size, d_I = 4, 8
    page_table = np.array([[2, 0, -1], [1, 3, -1]], np.int32)  # sequence 0: pages 2, 0; sequence 1: pages 1, 3
    pool = np.full((4 * page_size, d_I), 0xAA, np.uint8)
    scale = np.full(4 * page_size, -5.0, np.float32)
    k = np.arange(5 * d_I, dtype=np.float32).reshape(5, d_I) - 10
    positions = np.array([0, 5, -1, 7, 12], np.int32)  # 12 = 3 pages x 4: beyond the table, skipped
    row_seq = np.array([0, 0, 1, 1, 0], np.int32)
    out, sc = oracle.key_append(k, positions, row_seq, page_table, page_size, pool, scale)
    targets = {0: 2 * page_size + 0, 1: 0 * page_size + 1, 3: 3 * page_size + 3}  # row -> physical row
    for r, phys in targets.items():
        codes, s = oracle.quantize_key(k[r])
        assert np.array_equal(out[phys], codes) and sc[phys] == np.float32(s)
    untouched = np.setdiff1d(np.arange(4 * page_size), list(targets.values()))
    assert (out[untouched] == 0xAA).all() and (sc[untouched] == -5.0).all()
    # an fp32 pool stores the keys as they are
    fpool, none = oracle.key_append(k, positions, row_seq, page_table, page_size, np.zeros((16, d_I), np.float32))
    assert none is None and np.array_equal(fpool[targets[3]], k[3]) and not fpool[untouched].any()


# ------------------------------------------------------------------------- attention over the fp8 latent cache

def _bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy() \
        .view(np.uint16)


def _fp8_entries(rng, n, pow2_scales=False, rope_zero=False):
    codes = rng.integers(0, 256, size=(n, 512)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38  # no NaN codes
    if pow2_scales:
        scales = np.exp2(rng.integers(-8, 3, size=(n, 4))).astype(np.float32)
    else:
        scales = rng.uniform(0.001, 0.02, size=(n, 4)).astype(np.float32)
    rope = np.zeros((n, 64), np.float32) if rope_zero else rng.standard_normal((n, 64)).astype(np.float32)
    ent = np.zeros((n, 656), np.uint8)
    ent[:, :512] = codes
    ent[:, 512:528] = scales.view(np.uint8).reshape(n, 16)
    ent[:, 528:] = _bf16_bits(rope).view(np.uint8).reshape(n, 128)
    return ent


def test_fp8_entry_layout_by_hand():
    ent = np.zeros(656, np.uint8)
    ent[0], ent[130], ent[300], ent[511] = 0x38, 0xB8, 0x40, 0x7E  # 1.0, -1.0, 2.0, 448
    ent[512:528] = np.array([2.0, 0.5, 4.0, 0.25], np.float32).view(np.uint8)
    rope = np.zeros(64, np.float32)
    rope[5], rope[63] = 1.5, -3.0
    ent[528:] = _bf16_bits(rope).view(np.uint8)
    key = oracle.fp8_entry_key(ent)
    vals = oracle.decode(np.array([0x38, 0xB8, 0x40, 0x7E], np.uint8), "f8")
    assert vals[0] == 1.0 and vals[1] == -1.0 and vals[3] == 448.0
    assert key[0] == 2.0 and key[130] == -0.5 and key[300] == vals[2] * 4.0 and key[511] == 448.0 * 0.25
    assert key[512 + 5] == 1.5 and key[575] == -3.0
    assert np.count_nonzero(key) == 6


@pytest.mark.parametrize("scale", [1.0, 1 / math.sqrt(576)])
def test_fp8_attention_full_selection_equals_sdpa(scale):
    # the whole selection: softmax(scale * q [c; r]^T) c, with a 576-wide key and a 512-wide value
    rng = np.random.default_rng(21)
    n, H = 40, 6
    ent = _fp8_entries(rng, n)
    q = _bf16_bits(rng.standard_normal((1, H, 576)) * 0.05)
    page_table = np.arange(1, dtype=np.int32).reshape(1, 1)
    o, lse = oracle.sparse_attn_fp8(q, ent, np.arange(n, dtype=np.int32)[None], np.zeros(1, np.int32),
                                    page_table, 64, scale)
    keys = torch.from_numpy(np.stack([oracle.fp8_entry_key(e) for e in ent]))
    qf = torch.from_numpy(oracle.decode(q, "bf16")[0])
    ref = torch.nn.functional.scaled_dot_product_attention(qf[None], keys[None], keys[None, :, :512], scale=scale)[0]
    assert np.allclose(o[0], ref.numpy(), rtol=1e-10, atol=1e-12)
    logits = scale * (qf @ keys.T)
    assert np.allclose(lse[0], torch.logsumexp(logits, dim=1).numpy(), rtol=1e-12)


def test_fp8_attention_reduces_to_latent_attention_without_rope():
    # power-of-two scales make every dequantised value an exact fp32, and zero RoPE values leave only <q_c, c>: the
    # fp8 entry attention must equal the plain latent attention over an fp32 pool of those values
    rng = np.random.default_rng(22)
    n, H, page_size = 70, 4, 32
    ent = _fp8_entries(rng, n + 26, pow2_scales=True, rope_zero=True)
    f32_pool = np.stack([oracle.fp8_entry_key(e)[:512] for e in ent]).astype(np.float32)
    assert np.array_equal(f32_pool.astype(np.float64), np.stack([oracle.fp8_entry_key(e)[:512] for e in ent]))
    q = _bf16_bits(rng.standard_normal((2, H, 576)) * 0.05)
    page_table = np.array([[2, 0, 1], [1, 2, 0]], np.int32)
    sel = np.array([[5, 70, -1, 33, 0, 64], [1, 2, 3, 90, 95, -1]], np.int32)
    row_seq = np.array([0, 1], np.int32)
    o, lse = oracle.sparse_attn_fp8(q, ent, sel, row_seq, page_table, page_size, 0.7)
    qc = oracle.decode(q, "bf16")[:, :, :512].astype(np.float32)
    o2, lse2 = oracle.sparse_attn(qc, f32_pool, sel, row_seq, page_table, page_size, "f32", 0.7)
    assert np.allclose(o, o2, rtol=1e-12, atol=1e-14) and np.allclose(lse, lse2, rtol=1e-12)
    # an empty selection
    o3, lse3 = oracle.sparse_attn_fp8(q[:1], ent, np.full((1, 4), -1, np.int32), row_seq[:1], page_table, page_size,
                                      1.0)
    assert not o3.any() and np.isneginf(lse3).all()
