"""Python binding of libdsa, the gfx950 DeepSeek Sparse Attention decode-step library.

Argument marshalling only: every step of the path runs in the HIP kernels behind include/dsa.h.  PyTorch
supplies device memory (tensor data pointers) and the stream (the current HIP stream unless one is given).
The functions carry the C names and raise DsaError on any non-OK status.  There is no CPU fallback: if
libdsa.so cannot be built or loaded, the first call raises.
"""
from __future__ import annotations

import ctypes
import os

from . import _build

DSA_OK, DSA_EINVAL, DSA_EUNSUPPORTED, DSA_EWORKSPACE, DSA_EHIP = range(5)
DSA_F32, DSA_BF16, DSA_F8E4M3 = 0, 1, 2
DSA_OP_TOPK, DSA_OP_ATTN, DSA_OP_STEP, DSA_OP_DENSE = 1, 2, 3, 4
DTYPES = {"f32": DSA_F32, "bf16": DSA_BF16, "f8": DSA_F8E4M3}


class dsa_problem_t(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in (
        "num_rows", "num_seqs", "idx_heads", "idx_dim", "attn_heads", "latent_dim", "topk", "page_size",
        "max_pages", "num_pages", "max_row_len", "rows_per_seq", "idx_dtype", "kv_dtype")] + [
        ("softmax_scale", ctypes.c_float)]


class dsa_layout_t(ctypes.Structure):
    _fields_ = [("row_seq", ctypes.c_void_p), ("row_len", ctypes.c_void_p), ("page_table", ctypes.c_void_p)]


class DsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libdsa.so (built in-tree on first use if absent)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        P, I64, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
        PP, PL = ctypes.POINTER(dsa_problem_t), ctypes.POINTER(dsa_layout_t)
        L.dsa_indexer_scores.argtypes = [PP, PL, P, P, P, P, P, P, I64, P]
        L.dsa_topk.argtypes = [PP, PL, P, I64, P, P, SZ, P]
        L.dsa_sparse_mla_attn.argtypes = [PP, PL, P, P, P, P, P, P, SZ, P]
        L.dsa_decode_step.argtypes = [PP, PL, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
        L.dsa_decode_step_static.argtypes = [PP, PL, P, P, P, P, P, P, P, P, P, P, P]
        L.dsa_dense_mla_attn.argtypes = [PP, PL, P, P, P, P, P, SZ, P]
        L.dsa_indexer_key_append.argtypes = [PP, PL, P, P, P, P, P, P]
        L.dsa_indexer_query_proj.argtypes = [PP, ctypes.c_int32, P, P, P, P, P, P, P]
        for f in ("dsa_indexer_scores", "dsa_topk", "dsa_sparse_mla_attn", "dsa_decode_step", "dsa_dense_mla_attn",
                  "dsa_indexer_key_append", "dsa_decode_step_static", "dsa_indexer_query_proj"):
            getattr(L, f).restype = ctypes.c_int
        L.dsa_workspace_bytes.argtypes = [PP, ctypes.c_int32]
        L.dsa_workspace_bytes.restype = SZ
        L.dsa_status_str.argtypes = [ctypes.c_int]
        L.dsa_status_str.restype = ctypes.c_char_p
        L.dsa_last_error.argtypes = []
        L.dsa_last_error.restype = ctypes.c_char_p
        L.dsa_abi_version.argtypes = []
        L.dsa_abi_version.restype = ctypes.c_int32
        _lib = L
    return _lib


def make_problem(**fields) -> dsa_problem_t:
    """dsa_problem_t from keyword fields; dtype fields accept "f32" / "bf16" / "f8" or the enum value."""
    p = dsa_problem_t()
    defaults = dict(num_seqs=1, page_size=64, rows_per_seq=1, softmax_scale=1.0, idx_heads=64, idx_dim=64,
                    attn_heads=128, latent_dim=512, idx_dtype=DSA_F8E4M3, kv_dtype=DSA_BF16)
    for key, val in {**defaults, **fields}.items():
        if key in ("idx_dtype", "kv_dtype") and isinstance(val, str):
            val = DTYPES[val]
        setattr(p, key, val)
    return p


def make_layout(row_seq, row_len, page_table) -> dsa_layout_t:
    """dsa_layout_t over three int32 device tensors (the caller keeps them alive)."""
    return dsa_layout_t(_ptr(row_seq, "row_seq"), _ptr(row_len, "row_len"), _ptr(page_table, "page_table"))


def _ptr(t, name):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _check(status: int):
    if status != DSA_OK:
        raise DsaError(status, lib().dsa_last_error().decode())


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def dsa_indexer_scores(problem, layout, q_idx, q_idx_scale, head_w, k_idx_pool, k_idx_scale, scores,
                       scores_ld=None, stream=None):
    ld = scores.shape[-1] if scores_ld is None else scores_ld
    _check(lib().dsa_indexer_scores(
        ctypes.byref(problem), ctypes.byref(layout), _ptr(q_idx, "q_idx"), _ptr(q_idx_scale, "q_idx_scale"),
        _ptr(head_w, "head_w"), _ptr(k_idx_pool, "k_idx_pool"), _ptr(k_idx_scale, "k_idx_scale"),
        _ptr(scores, "scores"), ld, _stream(stream)))


def dsa_topk(problem, layout, scores, topk_idx, workspace, scores_ld=None, stream=None):
    ld = scores.shape[-1] if scores_ld is None else scores_ld
    _check(lib().dsa_topk(ctypes.byref(problem), ctypes.byref(layout), _ptr(scores, "scores"), ld,
                          _ptr(topk_idx, "topk_idx"), _ptr(workspace, "workspace"), _nbytes(workspace),
                          _stream(stream)))


def dsa_sparse_mla_attn(problem, layout, q, kv_pool, topk_idx, out, lse, workspace, stream=None):
    _check(lib().dsa_sparse_mla_attn(ctypes.byref(problem), ctypes.byref(layout), _ptr(q, "q"),
                                     _ptr(kv_pool, "kv_pool"), _ptr(topk_idx, "topk_idx"), _ptr(out, "out"),
                                     _ptr(lse, "lse"), _ptr(workspace, "workspace"), _nbytes(workspace),
                                     _stream(stream)))


def dsa_dense_mla_attn(problem, layout, q, kv_pool, out, lse, workspace, stream=None):
    _check(lib().dsa_dense_mla_attn(ctypes.byref(problem), ctypes.byref(layout), _ptr(q, "q"),
                                    _ptr(kv_pool, "kv_pool"), _ptr(out, "out"), _ptr(lse, "lse"),
                                    _ptr(workspace, "workspace"), _nbytes(workspace), _stream(stream)))


def dsa_indexer_key_append(problem, layout, positions, src, w_k, k_idx_pool, k_idx_scale, stream=None):
    _check(lib().dsa_indexer_key_append(ctypes.byref(problem), ctypes.byref(layout), _ptr(positions, "positions"),
                                        _ptr(src, "src"), _ptr(w_k, "w_k"), _ptr(k_idx_pool, "k_idx_pool"),
                                        _ptr(k_idx_scale, "k_idx_scale"), _stream(stream)))


def dsa_indexer_query_proj(problem, d_model, h, w_q, w_w, q_idx, q_idx_scale, head_w, stream=None):
    _check(lib().dsa_indexer_query_proj(ctypes.byref(problem), d_model, _ptr(h, "h"), _ptr(w_q, "w_q"),
                                        _ptr(w_w, "w_w"), _ptr(q_idx, "q_idx"), _ptr(q_idx_scale, "q_idx_scale"),
                                        _ptr(head_w, "head_w"), _stream(stream)))


def dsa_decode_step(problem, layout, q_idx, q_idx_scale, head_w, k_idx_pool, k_idx_scale, q, kv_pool, topk_idx,
                    out, lse, workspace, stream=None):
    _check(lib().dsa_decode_step(
        ctypes.byref(problem), ctypes.byref(layout), _ptr(q_idx, "q_idx"), _ptr(q_idx_scale, "q_idx_scale"),
        _ptr(head_w, "head_w"), _ptr(k_idx_pool, "k_idx_pool"), _ptr(k_idx_scale, "k_idx_scale"), _ptr(q, "q"),
        _ptr(kv_pool, "kv_pool"), _ptr(topk_idx, "topk_idx"), _ptr(out, "out"), _ptr(lse, "lse"),
        _ptr(workspace, "workspace"), _nbytes(workspace), _stream(stream)))


def dsa_decode_step_static(problem, layout, q_idx, q_idx_scale, head_w, k_idx_pool, k_idx_scale, q, kv_pool,
                           topk_idx, out, lse, stream=None):
    _check(lib().dsa_decode_step_static(
        ctypes.byref(problem), ctypes.byref(layout), _ptr(q_idx, "q_idx"), _ptr(q_idx_scale, "q_idx_scale"),
        _ptr(head_w, "head_w"), _ptr(k_idx_pool, "k_idx_pool"), _ptr(k_idx_scale, "k_idx_scale"), _ptr(q, "q"),
        _ptr(kv_pool, "kv_pool"), _ptr(topk_idx, "topk_idx"), _ptr(out, "out"), _ptr(lse, "lse"), _stream(stream)))


def dsa_workspace_bytes(problem, op: int) -> int:
    n = lib().dsa_workspace_bytes(ctypes.byref(problem), op)
    if n == 0 and lib().dsa_last_error():
        msg = lib().dsa_last_error().decode()
        if msg:
            raise DsaError(DSA_EINVAL, msg)
    return n


def dsa_status_str(status: int) -> str:
    return lib().dsa_status_str(status).decode()


def dsa_last_error() -> str:
    return lib().dsa_last_error().decode()


def dsa_abi_version() -> int:
    return lib().dsa_abi_version()
