"""The seeded generator is deterministic and follows its stated recipe."""
import hashlib

import numpy as np

import oracle
import synth


def _digest(p):
    h = hashlib.sha256()
    for a in (p.q_idx, p.q_idx_scale, p.head_w, p.k_idx_pool, p.k_idx_scale, p.q, p.kv_pool, p.row_seq, p.row_len,
              p.page_table):
        if a is not None:
            h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def test_deterministic():
    cfg = synth.get("decode_128k", lengths=[3000], H=8)
    assert _digest(synth.make_problem(cfg)) == _digest(synth.make_problem(cfg))


def test_recipe_tiny():
    p = synth.make_problem(synth.get("tiny_fp32"))
    assert p.R == 1 and p.row_len[0] == 4095 and p.q_idx.dtype == np.float32 and p.q_idx_scale is None
    assert len(p.boosted[0]) == 32 and p.boosted[0].max() < 4095
    assert p.kv_pool.shape == (64 * 64, 512) and (p.kv_pool[4095:] == 0).all()
    # latent ~ N(0,1), queries ~ N(0, 1/512), w ~ U(0,1)
    assert abs(p.kv_pool[:4095].std() - 1) < 0.02 and abs(p.q.std() * np.sqrt(512) - 1) < 0.1
    assert 0 <= p.head_w.min() and p.head_w.max() <= 1


def test_recipe_fp8_boost_and_quantisation():
    cfg = synth.get("decode_128k", lengths=[6000], anchors=40, recent=64, H=8)
    p = synth.make_problem(cfg)
    b = p.boosted[0]
    assert len(b) == 104 and len(np.unique(b)) == 104
    assert (b[-64:] == np.arange(6000 - 64, 6000)).all()
    # every key row uses the full e4m3 range: its largest |code| is 448 (0x7E / 0xFE)
    dec = oracle.decode(p.k_idx_pool[:6000], "f8")
    assert np.allclose(np.abs(dec).max(axis=1), 448.0)
    assert (p.k_idx_scale[:6000] > 0).all()
    assert p.q.dtype == np.uint16 and p.kv_pool.dtype == np.uint16


def test_paged_layout_is_a_permutation_and_holds_the_same_rows():
    cfg = synth.get("batched_paged", batch=3, length_range=(100, 300), H=4, H_I=4)
    p = synth.make_problem(cfg)
    npg = [-(-int(n) // 64) for n in p.row_len]
    used = np.concatenate([p.page_table[b, :npg[b]] for b in range(3)])
    assert sorted(used.tolist()) == list(range(p.num_pages))
    flat = synth.make_problem(dict(cfg, paged=False))
    for b in range(3):
        n = int(p.row_len[b])
        rows = lambda q: q.page_table[b, np.arange(n) // 64].astype(np.int64) * 64 + np.arange(n) % 64
        assert np.array_equal(p.kv_pool[rows(p)], flat.kv_pool[rows(flat)])
        assert np.array_equal(p.k_idx_pool[rows(p)], flat.k_idx_pool[rows(flat)])


def test_prefill_reuses_the_decode_cache_and_query():
    d = synth.make_problem(synth.get("decode_128k", lengths=[5000], H=4))
    pf = synth.make_problem(synth.get("prefill_chunk", cache_len=5000, rows=6, H=4))
    assert np.array_equal(pf.kv_pool, d.kv_pool) and np.array_equal(pf.k_idx_pool, d.k_idx_pool)
    assert pf.row_len.tolist() == [4995, 4996, 4997, 4998, 4999, 5000]
    assert np.array_equal(pf.q_idx[-1], d.q_idx[0]) and np.array_equal(pf.q[-1], d.q[0])
    assert not np.array_equal(pf.q_idx[0], d.q_idx[0])


def test_prefill_of_several_sequences_groups_rows():
    p = synth.make_problem(synth.get("prefill_paged", rows=5, length_range=(300, 700), H=4))
    assert p.R == 15 and p.rows_per_seq == 5
    for b in range(3):
        rows = slice(5 * b, 5 * b + 5)
        assert (p.row_seq[rows] == b).all()
        n = int(p.row_len[5 * b + 4])
        assert p.row_len[rows].tolist() == list(range(n - 4, n + 1))
