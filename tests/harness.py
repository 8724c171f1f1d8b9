"""Shared GPU-test plumbing: run the HIP path on a generated workload and compare it with the oracle.

Acceptance (from the step's definition and the stated tolerances):
  * indexer scores: within the forward error bound of fp32 summation, |I_gpu - I| <= gamma_n * B with
    n = 2 (d_I + H_I + 3), gamma_n = n u / (1 - n u), u = 2^-24 and B = sum_j |w_j| sum_d |q_I[j,d] k_I[s,d]|
    (the absolute-value form of the score: every product is exact or rounded once, every sum is fp32);
  * top-k: the selected set is k_eff distinct in-range positions; every position in the symmetric difference
    with the oracle's set has an oracle score within 1e-3 relative of the oracle's k_eff-th score; given the
    same scores, the selection is bit-exact against the oracle's selection rule;
  * attention: max abs error <= 2e-2 for bf16 latents and <= 1e-4 for fp32, on the GPU's own index set
    against the oracle's attention over that same set, and end to end against the oracle's own set.
"""
from __future__ import annotations

import sys
import types

import numpy as np
import torch

import long_context_sparse_indexer_amd as dsa
import oracle
from synth.device import upload

U32 = 2.0 ** -24
TIE_BAND = 1e-3
ATOL = {"bf16": 2e-2, "f32": 1e-4}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gpu_step(prob, stream=None, fields=None):
    """Run the indexer, top-k and attention as separate calls and as the fused step; returns host arrays."""
    d = upload(prob)
    f = dict(d.fields)
    if fields:
        f.update(fields)
    P = dsa.make_problem(**f)
    L = dsa.make_layout(d.row_seq, d.row_len, d.page_table)
    R, ld = prob.R, max(4, -(-max(prob.max_row_len, 1) // 4) * 4)
    dev = d.q_idx.device
    scores = torch.full((R, ld), float("nan"), device=dev)
    dsa.dsa_indexer_scores(P, L, d.q_idx, d.q_idx_scale, d.head_w, d.k_idx_pool, d.k_idx_scale, scores, ld, stream)
    idx = torch.empty((R, prob.k), dtype=torch.int32, device=dev)
    ws = torch.empty(max(dsa.dsa_workspace_bytes(P, dsa.DSA_OP_STEP), 256), dtype=torch.uint8, device=dev)
    dsa.dsa_topk(P, L, scores, idx, ws, ld, stream)
    out_dt = torch.bfloat16 if prob.kv_dtype == "bf16" else torch.float32
    out = torch.empty((R, prob.H, prob.d_c), dtype=out_dt, device=dev)
    lse = torch.empty((R, prob.H), dtype=torch.float32, device=dev)
    dsa.dsa_sparse_mla_attn(P, L, d.q, d.kv_pool, idx, out, lse, ws, stream)
    # fused step on the same inputs
    idx2 = torch.empty_like(idx)
    out2 = torch.empty_like(out)
    lse2 = torch.empty_like(lse)
    dsa.dsa_decode_step(P, L, d.q_idx, d.q_idx_scale, d.head_w, d.k_idx_pool, d.k_idx_scale, d.q, d.kv_pool, idx2,
                        out2, lse2, ws, stream)
    torch.cuda.synchronize()
    res = types.SimpleNamespace(
        scores=scores.cpu().numpy().astype(np.float64), idx=idx.cpu().numpy(), out=out.float().cpu().numpy(),
        lse=lse.cpu().numpy(), idx_step=idx2.cpu().numpy(), out_step=out2.float().cpu().numpy(),
        lse_step=lse2.cpu().numpy())
    del d, scores, ws
    return res


def score_bound(prob, r):
    """B[s] = sum_j |w_j| sum_d |q_I[j,d]| |k_I[s,d]| for the visible positions of row r (fp64)."""
    n = int(prob.row_len[r])
    q = np.abs(oracle.decode(prob.q_idx[r], prob.idx_dtype))                      # [H_I, d_I]
    if prob.q_idx_scale is not None:
        q = q * prob.q_idx_scale[r][:, None].astype(np.float64)
    s = np.arange(n)
    phys = prob.page_table[prob.row_seq[r], s // prob.page_size].astype(np.int64) * prob.page_size + s % prob.page_size
    k = np.abs(oracle.decode(prob.k_idx_pool[phys], prob.idx_dtype))              # [n, d_I]
    if prob.k_idx_scale is not None:
        k = k * prob.k_idx_scale[phys][:, None].astype(np.float64)
    return (k @ q.T) @ np.abs(prob.head_w[r].astype(np.float64))


def check_scores(prob, gpu_scores, ref_scores):
    nops = 2 * (prob.d_I + prob.H_I + 3)
    gamma = nops * U32 / (1 - nops * U32)
    worst = 0.0
    for r in range(prob.R):
        n = int(prob.row_len[r])
        if n == 0:
            continue
        g, o = gpu_scores[r, :n], ref_scores[r, :n]
        assert np.isfinite(g).all(), f"row {r}: non-finite GPU scores"
        bound = gamma * score_bound(prob, r) + 1e-30
        ratio = np.abs(g - o) / bound
        worst = max(worst, float(ratio.max()))
        assert (ratio <= 1.0).all(), f"row {r}: score error {float(ratio.max()):.2f}x the fp32 bound"
    return worst


def check_topk_set(prob, gpu_idx, ref_scores, ref_idx, ref_kth):
    for r in range(prob.R):
        n = int(prob.row_len[r])
        keff = min(prob.k, n)
        g = gpu_idx[r]
        assert (g[keff:] == -1).all(), f"row {r}: padding"
        sel = g[:keff]
        assert ((sel >= 0) & (sel < n)).all(), f"row {r}: out-of-range index"
        assert len(np.unique(sel)) == keff, f"row {r}: duplicate indices"
        assert (np.diff(sel) > 0).all(), f"row {r}: selection not in increasing position order"
        diff = set(sel.tolist()) ^ set(ref_idx[r, :keff].tolist())
        if diff:
            kth = ref_kth[r]
            band = TIE_BAND * abs(kth)
            worst = max(abs(ref_scores[r, p] - kth) for p in diff)
            assert worst <= band, f"row {r}: {len(diff)} differing positions, worst |I - I_k| = {worst:.3e} > {band:.3e}"


def check_topk_exact(prob, gpu_scores, gpu_idx):
    """Given the GPU's own fp32 scores, the selection must be exactly the oracle rule's selection."""
    idx, _ = oracle.topk(np.where(np.isnan(gpu_scores), 0.0, gpu_scores), prob.row_len, prob.k)
    for r in range(prob.R):
        keff = min(prob.k, int(prob.row_len[r]))
        assert np.array_equal(np.sort(idx[r, :keff]), gpu_idx[r, :keff]), f"row {r}: selection differs"


def check_attention(prob, out, lse, idx):
    ref_o, ref_lse = oracle.sparse_attn(prob.q, prob.kv_pool, idx, prob.row_seq, prob.page_table, prob.page_size,
                                        prob.kv_dtype, prob.softmax_scale)
    tol = ATOL[prob.kv_dtype]
    err = float(np.abs(out - ref_o).max()) if out.size else 0.0
    assert err <= tol, f"attention max abs error {err:.3e} > {tol}"
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(lse), fin), "lse finiteness differs"
    if fin.any():
        lerr = float(np.abs(lse[fin] - ref_lse[fin]).max())
        assert lerr <= 1e-3, f"lse error {lerr:.3e}"
    return err


def full_check(prob, fields=None):
    res = gpu_step(prob, fields=fields)
    ref_scores, ref_idx, ref_kth, ref_o, _ = oracle.decode_step(prob)
    score_ratio = check_scores(prob, res.scores, ref_scores)
    check_topk_exact(prob, res.scores, res.idx)
    check_topk_set(prob, res.idx, ref_scores, ref_idx, ref_kth)
    e_own = check_attention(prob, res.out, res.lse, res.idx)
    tol = ATOL[prob.kv_dtype]
    e2e = float(np.abs(res.out - ref_o).max())
    assert e2e <= tol, f"end-to-end error {e2e:.3e} against the oracle's own selection"
    # the fused step equals the separate calls bit for bit
    assert np.array_equal(res.idx_step, res.idx)
    assert np.array_equal(res.out_step, res.out) and np.array_equal(res.lse_step, res.lse, equal_nan=True)
    return res, dict(attn_err=e_own, e2e_err=e2e, score_ratio=score_ratio)
