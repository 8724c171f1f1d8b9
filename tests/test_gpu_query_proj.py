"""GPU parity of the indexer-query projection (dsa_indexer_query_proj) against the oracle.

Codes, scales and head weights are decided in a fixed order on both sides (exact fp64 products summed over d
ascending, one rounding to fp32, IEEE fp32 divisions), so every output must match the oracle's bit for bit.
The cases cover the decode shape (d_model 7168, 64 heads of 64), a 128-wide head (one quantisation group over two
waves), narrow heads (groups inside a wave), a d_model that leaves a partial chunk, the many-rows launch (four
chains per thread) and the fp32 tiny configuration.
"""
import numpy as np
import pytest
import torch

import long_context_sparse_indexer_amd as dsa
import oracle
import synth
from harness import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsa.lib()


def _run(R, d_model, H_I, d_I, act, idx, seed):
    say(f"query projection case R={R} d_model={d_model} H_I={H_I} d_I={d_I} act={act} idx={idx} seed={seed}")
    inp = synth.query_proj_inputs(R, d_model, H_I, d_I, act, seed)
    dev = "cuda:0"
    up = {k: torch.from_numpy(v.view(np.int16) if act == "bf16" else v).to(dev) for k, v in inp.items()}
    f8 = idx == "f8"
    q = torch.full((R, H_I, d_I), 0xAA if f8 else -5.0, dtype=torch.uint8 if f8 else torch.float32, device=dev)
    qs = torch.full((R, H_I), -5.0, dtype=torch.float32, device=dev) if f8 else None
    hw = torch.full((R, H_I), -5.0, dtype=torch.float32, device=dev)
    P = dsa.make_problem(num_rows=R, idx_heads=H_I, idx_dim=d_I, idx_dtype=idx, kv_dtype=act, topk=1,
                         max_pages=1, num_pages=1, max_row_len=0)
    dsa.dsa_indexer_query_proj(P, d_model, up["h"], up["w_q"], up["w_w"], q, qs, hw)
    torch.cuda.synchronize()
    rq, rs, rw = oracle.query_projection(inp["h"], inp["w_q"], inp["w_w"], H_I, act, idx)
    gq = q.cpu().numpy()
    if f8:
        bad = np.argwhere(gq != rq)
        assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[:4].tolist()}"
        assert np.array_equal(qs.cpu().numpy().view(np.uint32), rs.view(np.uint32)), "scales differ"
        if R > 1:
            assert (rs[0] == 1).all() and not rq[0].any(), "row 0 is a zero state"
        if H_I > 1:
            assert (rs[:, -1] == 1).all() and not rq[:, -1].any(), "the last head is a zero head"
    else:
        assert np.array_equal(gq.view(np.uint32), rq.view(np.uint32)), "fp32 queries differ"
    assert np.array_equal(hw.cpu().numpy().view(np.uint32), rw.view(np.uint32)), "head weights differ"
    say("  ok: codes, scales and head weights bit-exact")


def test_query_projection_decode_shape_one_token():
    _run(1, 7168, 64, 64, "bf16", "f8", 1)


def test_query_projection_wide_heads_several_tokens():
    _run(7, 7168, 64, 128, "bf16", "f8", 2)


def test_query_projection_narrow_heads_partial_chunk():
    # d_model 1000: the last 128-row chunk of W is partial; heads of 16 share a wave; 8 heads fill two tiles
    _run(9, 1000, 8, 16, "bf16", "f8", 3)


def test_query_projection_many_rows():
    # 64 tokens x 65 column tiles is past the one-chain-per-thread grid, so each thread runs four chains
    _run(64, 1024, 64, 64, "bf16", "f8", 4)


def test_query_projection_fp32_tiny_config():
    _run(3, 256, 4, 64, "f32", "f32", 5)
    _run(5, 512, 8, 32, "f32", "f8", 6)
