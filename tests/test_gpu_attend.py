"""GPU parity of dsa_sparse_attend against the CPU oracle on the same indices:
max|out - ref| <= 1e-2 max|ref| + 1e-3."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_util import assert_attention_close, host, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_case(q, kv, idx, win, scale, where):
    import indexer_top_gathered_amd as dsa
    say(f"[attend] {where} q={tuple(q.shape)} kv={tuple(kv.shape)} k={idx.shape[1]} "
        f"W={0 if win is None else win.shape[1]}")
    out = dsa.dsa_sparse_attend(q, kv, idx, win, scale)
    torch.cuda.synchronize()
    ref = oracle.attend(host(q), host(kv), host(idx), None if win is None else host(win), scale)
    err = assert_attention_close(out, ref, where)
    say(f"    max|diff| = {err:.3e}")
    return out


def _inputs(B, N, k, W, Hq, D, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    q = torch.randn((B, Hq, D), generator=g, device=DEV).to(torch.bfloat16)
    kv = torch.randn((B, N, D), generator=g, device=DEV).to(torch.bfloat16)
    win = torch.randn((B, W, D), generator=g, device=DEV).to(torch.bfloat16) if W else None
    keys = torch.rand((B, N), generator=g, device=DEV)
    idx = keys.argsort(dim=1)[:, :k].to(torch.int32).contiguous()
    return q, kv, idx, win


@pytest.mark.parametrize("D", [128, 512])
@pytest.mark.parametrize("Hq", [16, 32, 48, 128])
@pytest.mark.parametrize("k,W", [(1, 0), (5, 3), (40, 7), (100, 0), (300, 128)])
def test_random(D, Hq, k, W):
    B, N = 2, 777
    q, kv, idx, win = _inputs(B, N, k, W, Hq, D, 100 + D + Hq + k + W)
    run_case(q, kv, idx, win, 1 / np.sqrt(D), f"D={D} Hq={Hq} k={k} W={W}")


def test_large_logits_and_duplicate_rows():
    B, N, k, W, Hq, D = 3, 4000, 1000, 64, 128, 512
    q, kv, idx, win = _inputs(B, N, k, W, Hq, D, 7)
    idx[:, 1::3] = idx[:, 0:1]  # the same row selected many times
    run_case(q, kv, idx.contiguous(), win, 0.5, "sharp softmax, duplicated rows")


def test_tiny_step_workload_full():
    s = workloads.C1
    inp = workloads.step_inputs(s, 1000, device=DEV)
    ref_idx = oracle.topk(oracle.indexer(host(inp["q_idx"]), host(inp["k_idx"]), host(inp["w"])), s.k)
    idx = torch.from_numpy(ref_idx).to(DEV)
    run_case(inp["q"], inp["kv_cmp"], idx, inp["kv_win"], s.scale, "tiny step workload")


def test_production_step_workload_full():
    s = workloads.C4
    inp = workloads.step_inputs(s, 4000, device=DEV)
    ref_idx = oracle.topk(oracle.indexer(host(inp["q_idx"]), host(inp["k_idx"]), host(inp["w"])), s.k)
    idx = torch.from_numpy(ref_idx).to(DEV)
    run_case(inp["q"], inp["kv_cmp"], idx, inp["kv_win"], s.scale, "production step workload")


def test_row_order_does_not_matter():
    import indexer_top_gathered_amd as dsa
    B, N, k, W, Hq, D = 2, 3000, 512, 32, 64, 512
    q, kv, idx, win = _inputs(B, N, k, W, Hq, D, 9)
    a = dsa.dsa_sparse_attend(q, kv, idx, win, 0.05)
    perm = torch.randperm(k, generator=torch.Generator().manual_seed(1)).to(DEV)
    b = dsa.dsa_sparse_attend(q, kv, idx[:, perm].contiguous(), win, 0.05)
    torch.cuda.synchronize()
    diff = (a.float() - b.float()).abs().max().item()
    assert diff <= 1e-2 * a.float().abs().max().item() + 1e-3
