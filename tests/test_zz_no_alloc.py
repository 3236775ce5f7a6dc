"""The allocation-free step (dsa_decode_step_noalloc, for callers that
cannot allocate device memory) against dsa_decode_step, called through the C
ABI: the same kernels run on the library's static workspace, so the output
and the indices must equal those of dsa_decode_step bit for bit. Two calls in
a row, the second on a smaller input, so the second runs on the scratch the
first left behind."""
from __future__ import annotations

import pytest
import torch

import workloads
from parity_util import say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run(dsa, s, seed):
    inp = workloads.step_inputs(s, seed, device=DEV)
    ref_out, ref_idx = dsa.dsa_decode_step(inp["q_idx"], inp["k_idx"], inp["w"], inp["q"],
                                           inp["kv_cmp"], inp["kv_win"], s.k, s.scale,
                                           return_idx=True)
    out = torch.empty_like(ref_out)
    idx = torch.empty_like(ref_idx)
    torch.cuda.synchronize()
    dsa.dsa_decode_step_noalloc(inp["q_idx"], inp["k_idx"], inp["w"], inp["q"], inp["kv_cmp"],
                                inp["kv_win"], s.k, s.scale, out, out_idx=idx)
    torch.cuda.synchronize()
    return ref_out, ref_idx, out, idx


def test_noalloc_step_equals_the_step_twice_in_a_row():
    import indexer_top_gathered_amd as dsa
    shapes = [workloads.C4,
              workloads.StepShape(B=3, N=5000, H_I=8, D_I=128, k=300, W=16, H_q=32, D=128)]
    for n, s in enumerate(shapes):
        say(f"[noalloc] call {n}: B={s.B} N={s.N} k={s.k} H_q={s.H_q} D={s.D}")
        ref_out, ref_idx, out, idx = _run(dsa, s, 61000 + n)
        assert torch.equal(idx, ref_idx), f"call {n}: indices differ"
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), \
            f"call {n}: output differs"


def test_noalloc_rejects_a_shape_beyond_the_scratch():
    import indexer_top_gathered_amd as dsa
    s = workloads.StepShape(B=64, N=262144, H_I=8, D_I=128, k=64, W=0, H_q=16, D=128)
    dims = dsa.make_dims(s.B, s.N, s.H_I, s.D_I, s.k, s.W, s.H_q, s.D, s.scale)
    assert dsa.dsa_decode_step_workspace_bytes(dims) > dsa.NOALLOC_SCRATCH_BYTES
    q_idx = torch.zeros((s.B, s.H_I, 128), dtype=torch.bfloat16, device=DEV)
    # only the host checks run: nothing is launched
    with pytest.raises(dsa.DsaError, match="SCRATCH_LIMIT"):
        dsa.dsa_decode_step_noalloc(
            q_idx, torch.zeros((s.B, s.N, 128), dtype=torch.bfloat16, device=DEV),
            torch.zeros((s.B, s.H_I), dtype=torch.float32, device=DEV),
            torch.zeros((s.B, s.H_q, s.D), dtype=torch.bfloat16, device=DEV),
            torch.zeros((s.B, s.N, s.D), dtype=torch.bfloat16, device=DEV), None, s.k, s.scale,
            torch.empty((s.B, s.H_q, s.D), dtype=torch.bfloat16, device=DEV))
