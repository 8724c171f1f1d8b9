"""The C-ABI library loads, exports every symbol include/dsa.h declares, and rejects bad arguments on the host
before anything is enqueued.  No call here reaches a kernel launch (each one fails validation first), so the
file runs without a GPU."""
import ctypes
import os
import re

import pytest

import long_context_sparse_indexer_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 1 << 20          # a 256-byte-aligned non-NULL address that validation never dereferences
MISALIGNED = FAKE + 4


def _declared():
    text = open(os.path.join(ROOT, "include", "dsa.h")).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(dsa_\w+)\s*\(", text, re.M)))


def test_header_symbols_exported():
    names = _declared()
    assert {"dsa_indexer_scores", "dsa_topk", "dsa_sparse_mla_attn", "dsa_decode_step", "dsa_dense_mla_attn",
            "dsa_workspace_bytes", "dsa_status_str", "dsa_last_error", "dsa_abi_version"} <= set(names)
    L = dsa.lib()
    for n in names:
        assert hasattr(L, n), n
    assert dsa.dsa_abi_version() == 1


def _problem(**kw):
    base = dict(num_rows=2, num_seqs=1, idx_heads=64, idx_dim=64, attn_heads=128, latent_dim=512, topk=2048,
                page_size=64, max_pages=64, num_pages=64, max_row_len=4096, idx_dtype="f8", kv_dtype="bf16")
    base.update(kw)
    return dsa.make_problem(**base)


LAYOUT = dsa.dsa_layout_t(FAKE, FAKE, FAKE)


def _idx(p, layout=LAYOUT, q=FAKE, qs=FAKE, w=FAKE, k=FAKE, ks=FAKE, scores=FAKE, ld=4096):
    L = dsa.lib()
    return L.dsa_indexer_scores(ctypes.byref(p) if p is not None else None,
                                ctypes.byref(layout) if layout is not None else None, q, qs, w, k, ks, scores, ld, None)


def test_null_problem_and_layout():
    assert _idx(None) == dsa.DSA_EINVAL
    assert "problem is NULL" in dsa.dsa_last_error()
    assert _idx(_problem(), layout=None) == dsa.DSA_EINVAL
    assert _idx(_problem(), layout=dsa.dsa_layout_t(FAKE, None, FAKE)) == dsa.DSA_EINVAL


@pytest.mark.parametrize("kw, status, text", [
    (dict(num_rows=-1), dsa.DSA_EINVAL, "num_rows"),
    (dict(topk=0), dsa.DSA_EINVAL, "topk"),
    (dict(topk=20000), dsa.DSA_EINVAL, "topk"),
    (dict(page_size=48), dsa.DSA_EINVAL, "page_size"),
    (dict(page_size=16), dsa.DSA_EINVAL, "page_size"),
    (dict(max_row_len=4097), dsa.DSA_EINVAL, "max_row_len"),
    (dict(max_row_len=-5), dsa.DSA_EINVAL, "max_row_len"),
    (dict(rows_per_seq=0), dsa.DSA_EINVAL, "rows_per_seq"),
    (dict(idx_dim=96), dsa.DSA_EUNSUPPORTED, "idx_dim"),
    (dict(idx_heads=48), dsa.DSA_EUNSUPPORTED, "idx_heads"),
    (dict(idx_dtype=7), dsa.DSA_EINVAL, "idx_dtype"),
    (dict(num_pages=0), dsa.DSA_EINVAL, "num_pages"),
    (dict(num_rows=70000), dsa.DSA_EUNSUPPORTED, "num_rows"),
])
def test_indexer_problem_validation(kw, status, text):
    assert _idx(_problem(**kw)) == status
    assert text in dsa.dsa_last_error()


def test_indexer_pointer_validation():
    p = _problem()
    assert _idx(p, q=None) == dsa.DSA_EINVAL
    assert _idx(p, qs=None) == dsa.DSA_EINVAL and "scale" in dsa.dsa_last_error()
    assert _idx(p, k=MISALIGNED) == dsa.DSA_EINVAL and "aligned" in dsa.dsa_last_error()
    assert _idx(p, scores=None) == dsa.DSA_EINVAL
    assert _idx(p, ld=4000) == dsa.DSA_EINVAL and "scores_ld" in dsa.dsa_last_error()
    assert _idx(p, ld=4098) == dsa.DSA_EINVAL
    pf = _problem(idx_dtype="f32")
    assert _idx(pf) == dsa.DSA_EINVAL and "no scales" in dsa.dsa_last_error()


def test_topk_workspace_validation():
    p = _problem()
    L = dsa.lib()
    need = dsa.dsa_workspace_bytes(p, dsa.DSA_OP_TOPK)
    assert need > 0
    st = L.dsa_topk(ctypes.byref(p), ctypes.byref(LAYOUT), FAKE, 4096, FAKE, None, need, None)
    assert st == dsa.DSA_EWORKSPACE
    st = L.dsa_topk(ctypes.byref(p), ctypes.byref(LAYOUT), FAKE, 4096, FAKE, FAKE, need - 1, None)
    assert st == dsa.DSA_EWORKSPACE and "bytes" in dsa.dsa_last_error()
    st = L.dsa_topk(ctypes.byref(p), ctypes.byref(LAYOUT), FAKE, 4096, FAKE, FAKE + 16, need, None)
    assert st == dsa.DSA_EWORKSPACE and "aligned" in dsa.dsa_last_error()
    st = L.dsa_topk(ctypes.byref(p), ctypes.byref(LAYOUT), FAKE, 4096, None, FAKE, need, None)
    assert st == dsa.DSA_EINVAL


def test_attention_validation():
    L = dsa.lib()
    for kw, status in [(dict(latent_dim=576), dsa.DSA_EUNSUPPORTED), (dict(attn_heads=24), dsa.DSA_EUNSUPPORTED),
                       (dict(kv_dtype=9), dsa.DSA_EINVAL), (dict(kv_dtype="f32", topk=8192), dsa.DSA_EUNSUPPORTED),
                       (dict(softmax_scale=float("nan")), dsa.DSA_EINVAL)]:
        p = _problem(**kw)
        st = L.dsa_sparse_mla_attn(ctypes.byref(p), ctypes.byref(LAYOUT), FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                   1 << 30, None)
        assert st == status, (kw, dsa.dsa_last_error())
    p = _problem(num_rows=1)
    need = dsa.dsa_workspace_bytes(p, dsa.DSA_OP_ATTN)
    assert need > 0  # one row splits its selection over several blocks
    st = L.dsa_sparse_mla_attn(ctypes.byref(p), ctypes.byref(LAYOUT), FAKE, FAKE, FAKE, FAKE, None, None, 0, None)
    assert st == dsa.DSA_EWORKSPACE
    st = L.dsa_sparse_mla_attn(ctypes.byref(p), ctypes.byref(LAYOUT), FAKE, FAKE, None, FAKE, None, FAKE, need, None)
    assert st == dsa.DSA_EINVAL


def test_dense_attention_validation():
    # dense attention attends to every visible position: its selection width is the longest row, within what
    # the attention kernels split over (131072 bf16, 4096 fp32)
    L = dsa.lib()
    p = _problem(num_rows=1, max_row_len=60000, max_pages=1024, num_pages=1024)
    need = dsa.dsa_workspace_bytes(p, dsa.DSA_OP_DENSE)
    assert need > 0  # one row splits its 60000 positions over many blocks
    st = L.dsa_dense_mla_attn(ctypes.byref(p), ctypes.byref(LAYOUT), FAKE, FAKE, FAKE, None, FAKE, need - 1, None)
    assert st == dsa.DSA_EWORKSPACE
    st = L.dsa_dense_mla_attn(ctypes.byref(p), ctypes.byref(LAYOUT), None, FAKE, FAKE, None, FAKE, need, None)
    assert st == dsa.DSA_EINVAL
    for kw in (dict(max_row_len=131073, max_pages=4096, num_pages=4096),
               dict(kv_dtype="f32", latent_dim=64, max_row_len=4097, max_pages=128, num_pages=128)):
        p = _problem(num_rows=1, **kw)
        st = L.dsa_dense_mla_attn(ctypes.byref(p), ctypes.byref(LAYOUT), FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None)
        assert st == dsa.DSA_EUNSUPPORTED, (kw, dsa.dsa_last_error())
        assert "dense attention" in dsa.dsa_last_error()


def test_decode_step_validation():
    L = dsa.lib()
    p = _problem()
    need = dsa.dsa_workspace_bytes(p, dsa.DSA_OP_STEP)
    assert need >= dsa.dsa_workspace_bytes(p, dsa.DSA_OP_TOPK)
    args = [FAKE] * 5 + [FAKE, FAKE, None, FAKE, None]
    assert L.dsa_decode_step(ctypes.byref(p), ctypes.byref(LAYOUT), *args, FAKE, need - 256, None) == dsa.DSA_EWORKSPACE
    bad = list(args)
    bad[6] = MISALIGNED  # kv_pool
    assert L.dsa_decode_step(ctypes.byref(p), ctypes.byref(LAYOUT), *bad, FAKE, need, None) == dsa.DSA_EINVAL


def test_workspace_query_errors_and_strings():
    with pytest.raises(dsa.DsaError):
        dsa.dsa_workspace_bytes(_problem(topk=0), dsa.DSA_OP_TOPK)
    with pytest.raises(dsa.DsaError):
        dsa.dsa_workspace_bytes(_problem(), 99)
    # attention of enough rows to give every CU a block needs no split buffers: 0 bytes with no error
    assert dsa.dsa_workspace_bytes(_problem(num_rows=256), dsa.DSA_OP_ATTN) == 0
    assert dsa.dsa_workspace_bytes(_problem(num_rows=1), dsa.DSA_OP_ATTN) > 0
    for s in range(5):
        assert dsa.dsa_status_str(s).startswith("DSA_")
    assert "unknown" in dsa.dsa_status_str(42)


def test_binding_rejects_host_tensors():
    import torch
    p = _problem()
    lay = dsa.dsa_layout_t(FAKE, FAKE, FAKE)
    with pytest.raises(ValueError):
        dsa.dsa_indexer_scores(p, lay, torch.zeros(4), None, None, None, None, torch.zeros(4), 4096, stream=0)


def test_key_append_validation():
    L = dsa.lib()
    p = _problem(idx_dim=128)

    def call(p=p, positions=FAKE, src=FAKE, w=FAKE, pool=FAKE, scale=FAKE):
        return L.dsa_indexer_key_append(ctypes.byref(p), ctypes.byref(LAYOUT), positions, src, w, pool, scale, None)
    assert call(positions=None) == dsa.DSA_EINVAL and "non-NULL" in dsa.dsa_last_error()
    assert call(scale=None) == dsa.DSA_EINVAL and "k_idx_scale" in dsa.dsa_last_error()
    assert call(p=_problem(idx_dtype="f32")) == dsa.DSA_EINVAL and "no scales" in dsa.dsa_last_error()
    assert call(src=FAKE + 1) == dsa.DSA_EINVAL and "aligned" in dsa.dsa_last_error()
    assert call(p=_problem(kv_dtype=9)) == dsa.DSA_EINVAL and "kv_dtype" in dsa.dsa_last_error()
    assert call(p=_problem(latent_dim=1025, kv_dtype="f32")) == dsa.DSA_EUNSUPPORTED
    assert "latent_dim" in dsa.dsa_last_error()
    assert call(p=_problem(idx_dim=96)) == dsa.DSA_EUNSUPPORTED  # the fp8 cache widths of the indexer
    assert call(w=None, src=FAKE + 2) == dsa.DSA_EINVAL and "4-byte" in dsa.dsa_last_error()


def test_query_projection_validation():
    L = dsa.lib()

    def call(p=None, d_model=7168, h=FAKE, wq=FAKE, ww=FAKE, q=FAKE, qs=FAKE, hw=FAKE):
        p = p if p is not None else _problem()
        return L.dsa_indexer_query_proj(ctypes.byref(p), d_model, h, wq, ww, q, qs, hw, None)
    assert L.dsa_indexer_query_proj(None, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == dsa.DSA_EINVAL
    assert call(h=None) == dsa.DSA_EINVAL and "non-NULL" in dsa.dsa_last_error()
    assert call(qs=None) == dsa.DSA_EINVAL and "q_idx_scale" in dsa.dsa_last_error()
    assert call(p=_problem(idx_dtype="f32", kv_dtype="f32")) == dsa.DSA_EINVAL and "no scales" in dsa.dsa_last_error()
    assert call(p=_problem(kv_dtype="f8")) == dsa.DSA_EINVAL and "kv_dtype" in dsa.dsa_last_error()
    assert call(d_model=0) == dsa.DSA_EINVAL and "d_model" in dsa.dsa_last_error()
    assert call(d_model=7164) == dsa.DSA_EUNSUPPORTED and "d_model" in dsa.dsa_last_error()
    assert call(p=_problem(idx_dim=96)) == dsa.DSA_EUNSUPPORTED and "idx_dim" in dsa.dsa_last_error()
    assert call(p=_problem(idx_dim=256)) == dsa.DSA_EUNSUPPORTED and "idx_dim" in dsa.dsa_last_error()
    assert call(p=_problem(idx_heads=60)) == dsa.DSA_EUNSUPPORTED and "idx_heads" in dsa.dsa_last_error()
    assert call(p=_problem(idx_heads=136)) == dsa.DSA_EUNSUPPORTED and "idx_heads" in dsa.dsa_last_error()
    assert call(wq=FAKE + 8) == dsa.DSA_EINVAL and "16-byte" in dsa.dsa_last_error()
    assert call(hw=FAKE + 2) == dsa.DSA_EINVAL and "4-byte" in dsa.dsa_last_error()
    # R = 0 returns before any HIP call
    assert call(p=_problem(num_rows=0)) == dsa.DSA_OK


def test_prefill_step_workspace_holds_no_score_matrix():
    # a 4096-row chunk over 131072 positions: the step keeps candidate lists and samples, not R x n scores
    p = _problem(num_rows=4096, rows_per_seq=4096, max_row_len=131072, max_pages=2048, num_pages=2048)
    need = dsa.dsa_workspace_bytes(p, dsa.DSA_OP_STEP)
    assert 0 < need < 4096 * 131072 * 4 // 3
    # per-row decode rows still store their score rows
    d = _problem(num_rows=8, max_row_len=131072, max_pages=2048, num_pages=2048)
    assert dsa.dsa_workspace_bytes(d, dsa.DSA_OP_STEP) >= 8 * 131072 * 4


def test_zero_rows_enqueue_nothing():
    # R = 0 is valid everywhere and returns before any HIP call (no GPU needed)
    L = dsa.lib()
    p = _problem(num_rows=0, idx_dim=128)
    assert L.dsa_indexer_key_append(ctypes.byref(p), ctypes.byref(LAYOUT), FAKE, FAKE, FAKE, FAKE, FAKE, None) == 0
    assert L.dsa_indexer_key_append(ctypes.byref(p), ctypes.byref(LAYOUT), FAKE, FAKE, None, FAKE, FAKE, None) == 0
    pf = _problem(num_rows=0, kv_dtype="f8")
    assert dsa.dsa_workspace_bytes(pf, dsa.DSA_OP_DENSE) == 0
    assert L.dsa_dense_mla_attn(ctypes.byref(pf), ctypes.byref(LAYOUT), FAKE, FAKE, FAKE, None, None, 0, None) == 0


def test_static_scratch_step_rejects_oversized_problems():
    """The allocation-free step checks its problem against its fixed scratch before any device work."""
    P = _problem(num_rows=64, num_seqs=64, max_pages=16384, num_pages=16384 * 64, max_row_len=1048576)
    st = dsa.lib().dsa_decode_step_static(ctypes.byref(P), ctypes.byref(LAYOUT), *([FAKE] * 10), None)
    assert st == dsa.DSA_EUNSUPPORTED and "static scratch" in dsa.dsa_last_error()
    assert dsa.dsa_workspace_bytes(P, dsa.DSA_OP_STEP) > 64 << 20


def test_fp8_indexer_weights_must_be_aligned():
    p = _problem()
    assert _idx(p, w=MISALIGNED) == dsa.DSA_EINVAL and "16-byte aligned" in dsa.dsa_last_error()
    assert _idx(p, qs=MISALIGNED) == dsa.DSA_EINVAL and "16-byte aligned" in dsa.dsa_last_error()
