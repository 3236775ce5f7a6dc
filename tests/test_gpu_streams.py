"""Calls on a stream other than torch's current one, with no workspace or
outputs passed: the binding must allocate them on the launch stream, so that
allocations made meanwhile on the current stream never receive the memory of
a workspace that the launched kernels still use. Every result must equal the
same call made on the current stream, bit for bit."""
from __future__ import annotations

import pytest
import torch

import workloads
from parity_util import say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _step(dsa, inp, s, **kw):
    return dsa.dsa_decode_step(inp["q_idx"], inp["k_idx"], inp["w"], inp["q"], inp["kv_cmp"],
                               inp["kv_win"], s.k, s.scale, return_idx=True, **kw)


@pytest.mark.parametrize("raw_handle", [False, True])
def test_side_stream_without_workspace(raw_handle):
    import indexer_top_gathered_amd as dsa
    s = workloads.StepShape(B=4, N=20000, H_I=64, D_I=128, k=1024, W=128, H_q=128, D=512)
    say(f"[streams] side stream, raw handle={raw_handle}")
    inp = workloads.step_inputs(s, 4343, device=DEV)
    ref_out, ref_idx = _step(dsa, inp, s)
    ref_scores = dsa.dsa_indexer_score(inp["q_idx"], inp["k_idx"], inp["w"])
    ref_tk = dsa.dsa_topk(ref_scores, s.k)
    torch.cuda.synchronize()
    dims = dsa.make_dims(s.B, s.N, s.H_I, s.D_I, s.k, s.W, s.H_q, s.D, s.scale)
    nb = dsa.dsa_decode_step_workspace_bytes(dims)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    st = side.cuda_stream if raw_handle else side
    results = []
    for rep in range(4):
        o, i = _step(dsa, inp, s, stream=st)
        sc = dsa.dsa_indexer_score(inp["q_idx"], inp["k_idx"], inp["w"], stream=st)
        tk = dsa.dsa_topk(sc, s.k, stream=st)
        # Meanwhile, on the current stream: blocks of the workspace's size,
        # filled at once (they would overwrite a workspace still in use if
        # the allocator handed its memory out here).
        junk = [torch.full((nb,), 0xA5, dtype=torch.uint8, device=DEV) for _ in range(3)]
        results.append((o, i, tk))
        del junk
    side.synchronize()
    torch.cuda.synchronize()
    for o, i, tk in results:
        assert torch.equal(o.view(torch.int16), ref_out.view(torch.int16))
        assert torch.equal(i, ref_idx)
        assert torch.equal(tk, ref_tk)
