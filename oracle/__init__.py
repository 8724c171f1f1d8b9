"""ctypes wrapper of the fp64 CPU oracle (oracle/dsa_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's CPU-baseline leg are the only
callers.  The GPU library never imports, links or calls it, and it never imports the GPU library.

Every function takes the numpy arrays produced by the seeded generator (or hand-made ones) and returns fp64
results.  See dsa_oracle.c for the definitions and the passages of the pages each one follows.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

F32, BF16, F8E4M3 = 0, 1, 2
_DT = {"f32": F32, "bf16": BF16, "f8": F8E4M3}
_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        P, I32, I64, D = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        L.dsa_oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        L.dsa_oracle_e4m3_value.restype = D
        L.dsa_oracle_bf16_value.argtypes = [ctypes.c_uint16]
        L.dsa_oracle_bf16_value.restype = D
        L.dsa_oracle_threads.argtypes = []
        L.dsa_oracle_threads.restype = ctypes.c_int
        L.dsa_oracle_decode.argtypes = [P, I32, I64, P]
        L.dsa_oracle_decode.restype = None
        L.dsa_oracle_indexer_scores.argtypes = [I32, I32, I32, I32, P, P, P, P, P, P, P, P, I32, I32, P, I64]
        L.dsa_oracle_indexer_scores.restype = ctypes.c_int
        L.dsa_oracle_topk.argtypes = [I32, I32, P, P, I64, P, P]
        L.dsa_oracle_topk.restype = ctypes.c_int
        L.dsa_oracle_sparse_attn.argtypes = [I32, I32, I32, I32, P, P, P, I32, P, P, I32, I32, D, P, P]
        L.dsa_oracle_sparse_attn.restype = ctypes.c_int
        L.dsa_oracle_e4m3_nearest.argtypes = [ctypes.c_float]
        L.dsa_oracle_e4m3_nearest.restype = ctypes.c_uint8
        L.dsa_oracle_quantize_key.argtypes = [I32, P, P, P]
        L.dsa_oracle_quantize_key.restype = None
        L.dsa_oracle_key_projection.argtypes = [I32, I32, I32, I32, P, P, P]
        L.dsa_oracle_key_projection.restype = ctypes.c_int
        L.dsa_oracle_query_projection.argtypes = [I32, I32, I32, I32, I32, P, P, P, I32, P, P, P]
        L.dsa_oracle_query_projection.restype = ctypes.c_int
        L.dsa_oracle_key_append.argtypes = [I32, I32, P, P, P, P, I32, I32, I32, P, P]
        L.dsa_oracle_key_append.restype = ctypes.c_int
        L.dsa_oracle_fp8_entry_key.argtypes = [P, P]
        L.dsa_oracle_fp8_entry_key.restype = None
        L.dsa_oracle_sparse_attn_fp8.argtypes = [I32, I32, P, P, P, I32, P, P, I32, I32, D, P, P]
        L.dsa_oracle_sparse_attn_fp8.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def threads() -> int:
    """OpenMP threads the oracle runs on."""
    return int(lib().dsa_oracle_threads())


def decode(codes: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 value of every stored element ("f8" codes, "bf16" bit patterns or "f32")."""
    src = np.ascontiguousarray(codes)
    out = np.empty(src.shape, np.float64)
    lib().dsa_oracle_decode(_p(src), _DT[dtype], src.size, _p(out))
    return out


def indexer_scores(q_idx, q_idx_scale, head_w, k_idx_pool, k_idx_scale, row_seq, row_len, page_table,
                   page_size: int, idx_dtype: str, ld: int | None = None) -> np.ndarray:
    """I[r, s] for s < row_len[r] (fp64); entries at s >= row_len[r] are NaN."""
    R, H_I, d_I = q_idx.shape
    row_len = _c(row_len, np.int32)
    ld = int(ld if ld is not None else (row_len.max() if R else 0))
    out = np.full((R, max(ld, 1)), np.nan)
    code_t = np.uint8 if idx_dtype == "f8" else np.float32
    q_idx, k_idx_pool = _c(q_idx, code_t), _c(k_idx_pool, code_t)
    q_idx_scale, k_idx_scale = _c(q_idx_scale, np.float32), _c(k_idx_scale, np.float32)
    head_w, row_seq, page_table = _c(head_w, np.float32), _c(row_seq, np.int32), _c(page_table, np.int32)
    rc = lib().dsa_oracle_indexer_scores(
        R, H_I, d_I, _DT[idx_dtype], _p(q_idx), _p(q_idx_scale), _p(head_w), _p(k_idx_pool), _p(k_idx_scale),
        _p(row_seq), _p(row_len), _p(page_table), page_table.shape[1], page_size, _p(out), out.shape[1])
    if rc:
        raise ValueError(f"oracle indexer rejected its arguments (code {rc})")
    return out[:, :ld]


def topk(scores: np.ndarray, row_len, k: int):
    """(idx [R, k] int32 with -1 padding, k_eff-th score [R]); order: score desc, position asc."""
    scores = np.ascontiguousarray(scores, np.float64)
    R = scores.shape[0]
    row_len = _c(row_len, np.int32)
    idx = np.empty((R, k), np.int32)
    kth = np.empty(R, np.float64)
    rc = lib().dsa_oracle_topk(R, k, _p(row_len), _p(scores), scores.shape[1] if scores.ndim == 2 else 0,
                               _p(idx), _p(kth))
    if rc:
        raise ValueError(f"oracle top-k rejected its arguments (code {rc})")
    return idx, kth


def sparse_attn(q, kv_pool, topk_idx, row_seq, page_table, page_size: int, kv_dtype: str, scale: float):
    """(o [R, H, d_c] fp64, lse [R, H] fp64) over the selected rows (entries < 0 are ignored)."""
    R, H, d_c = q.shape
    code_t = np.uint16 if kv_dtype == "bf16" else np.float32
    q, kv_pool = _c(q, code_t), _c(kv_pool, code_t)
    topk_idx, row_seq, page_table = _c(topk_idx, np.int32), _c(row_seq, np.int32), _c(page_table, np.int32)
    k = topk_idx.shape[1]
    out = np.empty((R, H, d_c), np.float64)
    lse = np.empty((R, H), np.float64)
    rc = lib().dsa_oracle_sparse_attn(R, H, d_c, _DT[kv_dtype], _p(q), _p(kv_pool), _p(topk_idx), k, _p(row_seq),
                                      _p(page_table), page_table.shape[1], page_size, float(scale), _p(out), _p(lse))
    if rc:
        raise ValueError(f"oracle attention rejected its arguments (code {rc})")
    return out, lse


def decode_step(prob):
    """The whole step on a synth.Problem: (scores, idx, kth, o, lse)."""
    scores = indexer_scores(prob.q_idx, prob.q_idx_scale, prob.head_w, prob.k_idx_pool, prob.k_idx_scale,
                            prob.row_seq, prob.row_len, prob.page_table, prob.page_size, prob.idx_dtype)
    idx, kth = topk(scores, prob.row_len, prob.k)
    if prob.kv_dtype == "f8":
        o, lse = sparse_attn_fp8(prob.q, prob.kv_pool, idx, prob.row_seq, prob.page_table, prob.page_size,
                                 prob.softmax_scale)
    else:
        o, lse = sparse_attn(prob.q, prob.kv_pool, idx, prob.row_seq, prob.page_table, prob.page_size,
                             prob.kv_dtype, prob.softmax_scale)
    return scores, idx, kth, o, lse


def e4m3_nearest(y: float) -> int:
    """The e4m3 code nearest to the fp32 value y (ties to the even code, clamped to +-448, sign kept)."""
    return int(lib().dsa_oracle_e4m3_nearest(float(y)))


def quantize_key(x) -> tuple[np.ndarray, float]:
    """(codes uint8 [d], scale) of one fp32 key vector: scale = max|x| / 448, codes nearest x / scale."""
    x = _c(x, np.float32)
    codes = np.empty(x.shape[-1], np.uint8)
    scale = np.empty(1, np.float32)
    lib().dsa_oracle_quantize_key(x.shape[-1], _p(x), _p(codes), _p(scale))
    return codes, float(scale[0])


def key_projection(c, w, c_dtype: str) -> np.ndarray:
    """k = c W_KI in fp64 ([R, d_c] x [d_c, d_I], d ascending), from bf16 bit patterns or fp32 values."""
    code_t = np.uint16 if c_dtype == "bf16" else np.float32
    c, w = _c(c, code_t), _c(w, code_t)
    R, d_c = c.shape
    d_I = w.shape[1]
    if w.shape[0] != d_c:
        raise ValueError("c and w disagree on d_c")
    k = np.empty((R, d_I), np.float64)
    if lib().dsa_oracle_key_projection(R, d_c, d_I, _DT[c_dtype], _p(c), _p(w), _p(k)):
        raise ValueError("oracle key projection rejected its arguments")
    return k


def query_projection(h, w_q, w_w, H_I: int, h_dtype: str, idx_dtype: str):
    """(q [R, H_I, d_I], q_scale [R, H_I] or None, head_w [R, H_I]) of hidden states h [R, d_model] through
    W_QI [d_model, H_I d_I] and W_w [d_model, H_I]; q holds e4m3 codes ("f8") or fp32 values ("f32")."""
    code_t = np.uint16 if h_dtype == "bf16" else np.float32
    h, w_q, w_w = _c(h, code_t), _c(w_q, code_t), _c(w_w, code_t)
    R, d_model = h.shape
    if w_q.shape[0] != d_model or w_w.shape != (d_model, H_I) or w_q.shape[1] % H_I:
        raise ValueError("h, w_q and w_w disagree on their shapes")
    d_I = w_q.shape[1] // H_I
    f8 = idx_dtype == "f8"
    q = np.empty((R, H_I, d_I), np.uint8 if f8 else np.float32)
    q_scale = np.empty((R, H_I), np.float32) if f8 else None
    head_w = np.empty((R, H_I), np.float32)
    rc = lib().dsa_oracle_query_projection(R, d_model, H_I, d_I, _DT[h_dtype], _p(h), _p(w_q), _p(w_w),
                                           _DT[idx_dtype], _p(q), _p(q_scale), _p(head_w))
    if rc:
        raise ValueError(f"oracle query projection rejected its arguments (code {rc})")
    return q, q_scale, head_w


def key_append(k32, positions, row_seq, page_table, page_size: int, pool, pool_scale=None):
    """Writes fp32 keys k32 [R, d_I] into copies of the pool (uint8 codes + scales, or fp32 with no scales)
    at each row's position; returns (pool, pool_scale)."""
    k32 = _c(k32, np.float32)
    R, d_I = k32.shape
    f8 = pool.dtype == np.uint8
    pool = np.array(pool, copy=True)
    pool_scale = np.array(pool_scale, np.float32, copy=True) if f8 else None
    positions, row_seq, page_table = _c(positions, np.int32), _c(row_seq, np.int32), _c(page_table, np.int32)
    rc = lib().dsa_oracle_key_append(R, d_I, _p(k32), _p(positions), _p(row_seq), _p(page_table),
                                     page_table.shape[1], page_size, F8E4M3 if f8 else F32, _p(pool), _p(pool_scale))
    if rc:
        raise ValueError("oracle key append rejected its arguments")
    return pool, pool_scale


FP8_ENTRY_BYTES = 656


def fp8_entry_key(entry) -> np.ndarray:
    """The 576-wide fp64 key of one 656-byte latent cache entry (512 dequantised latent values, 64 RoPE values)."""
    entry = _c(entry, np.uint8)
    if entry.size != FP8_ENTRY_BYTES:
        raise ValueError("an fp8 latent entry has 656 bytes")
    key = np.empty(576, np.float64)
    lib().dsa_oracle_fp8_entry_key(_p(entry), _p(key))
    return key


def sparse_attn_fp8(q, pool, topk_idx, row_seq, page_table, page_size: int, scale: float):
    """(o [R, H, 512], lse [R, H]) in fp64 over the selected 656-byte entries; q [R, H, 576] bf16 bit patterns."""
    q = _c(q, np.uint16)
    R, H, width = q.shape
    if width != 576:
        raise ValueError("the fp8-latent query is 576 wide")
    pool = _c(pool, np.uint8)
    topk_idx, row_seq, page_table = _c(topk_idx, np.int32), _c(row_seq, np.int32), _c(page_table, np.int32)
    k = topk_idx.shape[1]
    out = np.empty((R, H, 512), np.float64)
    lse = np.empty((R, H), np.float64)
    rc = lib().dsa_oracle_sparse_attn_fp8(R, H, _p(q), _p(pool), _p(topk_idx), k, _p(row_seq), _p(page_table),
                                          page_table.shape[1], page_size, float(scale), _p(out), _p(lse))
    if rc:
        raise ValueError(f"oracle fp8 attention rejected its arguments (code {rc})")
    return out, lse
