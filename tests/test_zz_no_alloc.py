"""The allocation-free step (dsa_decode_step_static, scratch in the library's device code) against the step with a
caller workspace, through the C ABI: bit-identical selections, outputs and lse on two calls in a row, the second
with a smaller input, so that the second call runs over scratch the first one left behind."""
import ctypes

import numpy as np
import pytest
import torch

import long_context_sparse_indexer_amd as dsa
import synth
from synth.device import upload

pytestmark = pytest.mark.gpu


def _run(prob):
    d = upload(prob)
    P = dsa.make_problem(**d.fields)
    L = dsa.make_layout(d.row_seq, d.row_len, d.page_table)
    dev = d.q_idx.device
    res = {}
    for mode in ("workspace", "static"):
        idx = torch.full((prob.R, prob.k), -7, dtype=torch.int32, device=dev)
        out = torch.full((prob.R, prob.H, prob.d_c), 3.0, dtype=torch.bfloat16, device=dev)
        lse = torch.full((prob.R, prob.H), 5.0, dtype=torch.float32, device=dev)
        if mode == "workspace":
            ws = torch.empty(max(256, dsa.dsa_workspace_bytes(P, dsa.DSA_OP_STEP)), dtype=torch.uint8, device=dev)
            dsa.dsa_decode_step(P, L, d.q_idx, d.q_idx_scale, d.head_w, d.k_idx_pool, d.k_idx_scale, d.q, d.kv_pool,
                                idx, out, lse, ws)
        else:
            st = dsa.lib().dsa_decode_step_static(
                ctypes.byref(P), ctypes.byref(L), d.q_idx.data_ptr(), d.q_idx_scale.data_ptr(), d.head_w.data_ptr(),
                d.k_idx_pool.data_ptr(), d.k_idx_scale.data_ptr(), d.q.data_ptr(), d.kv_pool.data_ptr(),
                idx.data_ptr(), out.data_ptr(), lse.data_ptr(), torch.cuda.current_stream().cuda_stream)
            assert st == dsa.DSA_OK, dsa.dsa_last_error()
        torch.cuda.synchronize()
        res[mode] = (idx.cpu().numpy(), out.float().cpu().numpy(), lse.cpu().numpy())
    return res


def test_static_scratch_step_matches_workspace_step_twice():
    # a 128K row with split partials, then a smaller batch of short rows (one shorter than the budget)
    first = synth.make_problem(synth.get("decode_128k", seed=31))
    second = synth.make_problem(synth.get("batched_paged", batch=3, length_range=(1000, 9000), seed=32, H=32))
    for prob in (first, second):
        r = _run(prob)
        for a, b in zip(r["workspace"], r["static"]):
            assert np.array_equal(a, b, equal_nan=True)
        assert (r["static"][0][:, :1] >= 0).all()

