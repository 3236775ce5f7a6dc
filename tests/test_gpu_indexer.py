"""GPU parity of dsa_indexer_score against the CPU oracle (float32 forward-error
bound; bit-exact where the exact score is representable)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_util import assert_scores_close, host, indexer_bound, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_case(q, k, w, where):
    import indexer_top_gathered_amd as dsa
    say(f"[indexer] {where} q={tuple(q.shape)} k={tuple(k.shape)}")
    s = dsa.dsa_indexer_score(q, k, w)
    torch.cuda.synchronize()
    qb, kb, wb = host(q), host(k), host(w)
    ref = oracle.indexer(qb, kb, wb)
    assert_scores_close(s.cpu().numpy(), ref, indexer_bound(qb, kb, wb), where)
    return s, ref


@pytest.mark.parametrize("H", [1, 8, 13, 16, 33, 64])
@pytest.mark.parametrize("N", [1, 17, 1000, 4099])
def test_random(H, N):
    s = workloads.StepShape(B=2, N=N, H_I=H, D_I=128, k=1, W=0, H_q=16, D=128)
    inp = workloads.step_inputs(s, 10000 + 100 * H + N, device=DEV)
    run_case(inp["q_idx"], inp["k_idx"], inp["w"], f"H={H} N={N}")


def test_exact_when_representable():
    """Integer-valued inputs small enough that every partial sum is exact in
    float32: the GPU must reproduce the oracle bit for bit."""
    g = torch.Generator(device=DEV).manual_seed(3)
    B, N, H = 3, 5000, 64
    q = torch.randint(-3, 4, (B, H, 128), generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randint(-3, 4, (B, N, 128), generator=g, device=DEV).to(torch.bfloat16)
    w = (torch.randint(0, 8, (B, H), generator=g, device=DEV).float() / 8)
    s, ref = run_case(q, k, w, "exact integer inputs")
    assert np.array_equal(s.cpu().numpy(), ref)


def test_negative_weights_relu_then_weight():
    g = torch.Generator(device=DEV).manual_seed(4)
    B, N, H = 2, 700, 8
    q = torch.randn((B, H, 128), generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn((B, N, 128), generator=g, device=DEV).to(torch.bfloat16)
    w = torch.randn((B, H), generator=g, device=DEV)
    run_case(q, k, w, "negative weights")


def test_tiny_step_workload_full():
    s = workloads.C1
    inp = workloads.step_inputs(s, 1000, device=DEV)
    run_case(inp["q_idx"], inp["k_idx"], inp["w"], "tiny step workload")


def test_production_step_workload_full():
    s = workloads.C4
    inp = workloads.step_inputs(s, 4000, device=DEV)
    run_case(inp["q_idx"], inp["k_idx"], inp["w"], "production step workload B=16 N=32768 H=64")


def test_stress_workload_sampled_positions_exact():
    """The stress construction makes every score exact: the GPU scores equal
    the quantised rows bit for bit at every position of every row."""
    import indexer_top_gathered_amd as dsa
    s = workloads.C5
    say("[indexer] stress workload B=64 N=262144 H=64 (exact construction)")
    inp = workloads.stress_step_inputs(s, 5000, device=DEV)
    out = dsa.dsa_indexer_score(inp["q_idx"], inp["k_idx"], inp["w"])
    torch.cuda.synchronize()
    assert torch.equal(out, inp["stress_scores"].float())
    # and the oracle agrees on a sample of positions of two rows
    cols = torch.randperm(s.N, generator=torch.Generator().manual_seed(0))[:4096].sort().values
    for b in (0, 63):
        kb = host(inp["k_idx"][b:b + 1, cols.to(DEV)].contiguous())
        ref = oracle.indexer(host(inp["q_idx"][b:b + 1]), kb, host(inp["w"][b:b + 1]))
        assert np.array_equal(out[b, cols.to(DEV)].cpu().numpy(), ref[0])
    del inp, out
    torch.cuda.empty_cache()


def test_deterministic():
    import indexer_top_gathered_amd as dsa
    s = workloads.StepShape(B=4, N=20000, H_I=64, D_I=128, k=1, W=0, H_q=16, D=128)
    inp = workloads.step_inputs(s, 777, device=DEV)
    a = dsa.dsa_indexer_score(inp["q_idx"], inp["k_idx"], inp["w"])
    b = dsa.dsa_indexer_score(inp["q_idx"], inp["k_idx"], inp["w"])
    torch.cuda.synchronize()
    assert torch.equal(a, b)
