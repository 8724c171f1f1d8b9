"""Move a generated workload into device memory (plumbing only: copies, no arithmetic)."""
from __future__ import annotations

import types

import numpy as np
import torch

from .gen import Problem


def _t(a, device, dtype=None):
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(device)


def upload(p: Problem, device="cuda") -> types.SimpleNamespace:
    """Device tensors of every input plus the problem fields of the C ABI (as a dict)."""
    f8 = p.idx_dtype == "f8"
    kv_t = torch.int16 if p.kv_dtype in ("bf16", "f8") else None  # f8 latents: bf16 queries, byte entries
    d = types.SimpleNamespace()
    d.q_idx = _t(p.q_idx, device)
    d.q_idx_scale = _t(p.q_idx_scale, device)
    d.head_w = _t(p.head_w, device)
    d.k_idx_pool = _t(p.k_idx_pool, device)
    d.k_idx_scale = _t(p.k_idx_scale, device)
    d.q = _t(p.q.view(np.int16) if kv_t else p.q, device, kv_t and torch.bfloat16)
    d.kv_pool = _t(p.kv_pool.view(np.int16) if p.kv_dtype == "bf16" else p.kv_pool, device,
                   torch.bfloat16 if p.kv_dtype == "bf16" else None)
    d.row_seq = _t(p.row_seq, device)
    d.row_len = _t(p.row_len, device)
    d.page_table = _t(p.page_table, device)
    d.fields = dict(num_rows=p.R, num_seqs=p.S, idx_heads=p.H_I, idx_dim=p.d_I, attn_heads=p.H, latent_dim=p.d_c,
                    topk=p.k, page_size=p.page_size, max_pages=p.max_pages, num_pages=p.num_pages,
                    max_row_len=p.max_row_len, rows_per_seq=p.rows_per_seq, idx_dtype=p.idx_dtype,
                    kv_dtype=p.kv_dtype, softmax_scale=p.softmax_scale)
    d.f8 = f8
    return d
