"""GPU parity of dsa_indexer_qproj against the CPU oracle.

Bar: |q_gpu - q_ref| <= 2^-8 |q_ref| + 2 d_in 2^-24 sum_i |x_i w_i| + 2^-133:
half a bf16 ulp for the final rounding (with a factor 2 of slack) plus the
forward-error bound of a float32 sum of d_in exact products (Higham,
Accuracy and Stability of Numerical Algorithms, section 3.1) with a factor 2
of slack; the last term covers subnormal results."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_util import host, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_case(B, d_in, H_I, seed, where=""):
    import indexer_top_gathered_amd as dsa
    say(f"[qproj] {where} B={B} d_in={d_in} H_I={H_I}")
    inp = workloads.qproj_inputs(B, d_in, H_I, seed, device=DEV)
    got = dsa.dsa_indexer_qproj(inp["x"], inp["w_q"], H_I)
    torch.cuda.synchronize()
    xb, wb = host(inp["x"]), host(inp["w_q"])
    ref = oracle.qproj(xb, wb).reshape(B, H_I, 128)
    mag = (np.abs(oracle.bf16_decode(xb)) @ np.abs(oracle.bf16_decode(wb)).T).reshape(B, H_I, 128)
    bound = 2.0 ** -8 * np.abs(ref) + 2 * d_in * 2.0 ** -24 * mag + 2.0 ** -133
    g = got.float().cpu().numpy().astype(np.float64)
    err = np.abs(g - ref)
    assert np.all(err <= bound), f"{where}: {int((err > bound).sum())} outputs outside the bound"
    return got


@pytest.mark.parametrize("B,d_in,H_I", [(1, 512, 1), (3, 1536, 8), (16, 4096, 64), (17, 2048, 13),
                                        (40, 7168, 64)])
def test_qproj_random(B, d_in, H_I):
    run_case(B, d_in, H_I, 51000 + B + d_in, f"random")


def test_qproj_deterministic_and_one_hot_exact():
    import indexer_top_gathered_amd as dsa
    B, d_in, H_I = 16, 1024, 8
    inp = workloads.qproj_inputs(B, d_in, H_I, 52000, device=DEV)
    a = dsa.dsa_indexer_qproj(inp["x"], inp["w_q"], H_I)
    b = dsa.dsa_indexer_qproj(inp["x"], inp["w_q"], H_I)
    x = torch.zeros((B, d_in), dtype=torch.bfloat16, device=DEV)
    cols = torch.arange(B, device=DEV) * 61 % d_in
    x[torch.arange(B, device=DEV), cols] = 1.0
    c = dsa.dsa_indexer_qproj(x, inp["w_q"], H_I)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    # a one-hot row selects one column of w_q exactly (one exact product, zeros elsewhere)
    ref = inp["w_q"][:, cols].T.reshape(B, H_I, 128)
    assert torch.equal(c.view(torch.int16), ref.contiguous().view(torch.int16))
