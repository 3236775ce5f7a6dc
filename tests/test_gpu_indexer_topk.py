"""GPU parity of dsa_indexer_topk, the indexer fused with the top-k.

Its scores must equal dsa_indexer_score's bit for bit, and its index set the
oracle's top-k of those scores exactly. Rows are built through the exact
construction of the stress workload (indexer query e_0, weights 1/H_I, key
channel 0 = the wanted score, non-negative, exact in float32) when a given score pattern
is wanted: sorted and reversed rows, ties, and rows whose top scores all
sit in chunk 0 (group g = j / 32 belongs to chunk (g - g / C) mod C), which the chunk cut
cannot settle and the merge must select again from the score row.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_util import assert_topk_equal, host, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def exact_inputs(scores_bf16: torch.Tensor, H: int, seed: int) -> dict:
    """Indexer inputs whose float32 scores equal the given bf16 rows exactly."""
    B, N = scores_bf16.shape
    g = torch.Generator(device=DEV).manual_seed(seed)
    k_idx = torch.randn(B, N, 128, generator=g, device=DEV).to(torch.bfloat16)
    k_idx[:, :, 0] = scores_bf16
    q_idx = torch.zeros((B, H, 128), dtype=torch.bfloat16, device=DEV)
    q_idx[:, :, 0] = 1.0
    w = torch.full((B, H), 1.0 / H, dtype=torch.float32, device=DEV)
    return {"q_idx": q_idx, "k_idx": k_idx, "w": w}


def check(inp: dict, k: int, where: str, want_scores=None):
    import indexer_top_gathered_amd as dsa
    B, N = inp["k_idx"].shape[:2]
    C = dsa.dsa_indexer_topk_chunks(B, N, k)
    say(f"[indexer_topk] {where}: B={B} N={N} k={k} H_I={inp['q_idx'].shape[1]} chunks={C}")
    idx, sc = dsa.dsa_indexer_topk(inp["q_idx"], inp["k_idx"], inp["w"], k, return_scores=True)
    idx_ws = dsa.dsa_indexer_topk(inp["q_idx"], inp["k_idx"], inp["w"], k)  # scores kept inside
    ref_sc = dsa.dsa_indexer_score(inp["q_idx"], inp["k_idx"], inp["w"])
    torch.cuda.synchronize()
    assert torch.equal(sc.view(torch.int32), ref_sc.view(torch.int32)), f"{where}: scores differ"
    assert torch.equal(idx, idx_ws), f"{where}: result depends on where the scores go"
    if want_scores is not None:
        assert torch.equal(sc, want_scores.float()), f"{where}: the construction is not exact"
    g = idx.cpu().numpy()
    for b in range(B):
        assert len(np.unique(g[b])) == k and g[b].min() >= 0 and g[b].max() < N, where
    assert_topk_equal(g, oracle.topk(host(sc), k), False, where)
    return idx, C


@pytest.mark.parametrize("B,N,H,k", [
    (16, 32768, 64, 1024),      # the production shape
    (1, 4096, 8, 256),          # the tiny step
    (3, 1001, 13, 77),          # N not a multiple of 32
    (2, 5000, 64, 4096),        # the largest k
    (200, 700, 8, 64),          # many rows, one chunk each
    (3, 257, 1, 256),           # one head
    (1, 40, 8, 40),             # k = N
    (2, 9000, 64, 1),           # k = 1
    (1, 600000, 8, 2048),       # one long row: more chunks than the merge holds (unfused)
    # Chunk-cut shapes (rows longer than one top-k workgroup takes whole):
    (3, 8193, 13, 77),          # one position past the whole-row path, ragged tail
    (2, 12000, 64, 4096),       # the largest k over few chunk keys
    (200, 9000, 8, 64),         # many rows of two chunks
    (3, 10001, 1, 1),           # one head, k = 1
])
def test_random_rows(B, N, H, k):
    s = workloads.StepShape(B=B, N=N, H_I=H, D_I=128, k=k, W=0, H_q=16, D=128)
    inp = workloads.step_inputs(s, 81000 + N + k, device=DEV)
    check({x: inp[x] for x in ("q_idx", "k_idx", "w")}, k, "random")


@pytest.mark.parametrize("order", ["ascending", "descending", "stress levels", "all equal"])
def test_patterned_rows(order):
    B, N, k = 4, 32768, 1024
    g = torch.Generator(device=DEV).manual_seed(82000)
    x = torch.randn(B, N, generator=g, device=DEV) + 8.0  # the construction passes a ReLU
    if order == "ascending":
        sc = x.sort(dim=1).values
    elif order == "descending":
        sc = x.sort(dim=1, descending=True).values
    elif order == "stress levels":  # 256 levels, heavy ties; odd rows sorted
        sc = torch.clamp(torch.floor((x - 4) * 32), 0, 255) / 32
        sc[1::2] = sc[1::2].sort(dim=1).values
    else:
        sc = torch.zeros_like(x)
    sc = sc.to(torch.bfloat16)
    check(exact_inputs(sc, 16, 82100), k, order, want_scores=sc)


@pytest.mark.parametrize("B,N,k,levels", [(4, 32768, 1024, False), (3, 9000, 300, False),
                                          (2, 20000, 2048, True), (1, 12288, 256, False)])
def test_rows_the_cut_cannot_settle(B, N, k, levels):
    """The top scores of rows 0, 2, ... all sit in chunk 0's positions (group
    g = j / 32 belongs to chunk (g - g / C) mod C): that chunk keeps only its
    top few, so the merge must select those rows again from their score
    rows; odd rows are random and settle normally."""
    import indexer_top_gathered_amd as dsa
    C = dsa.dsa_indexer_topk_chunks(B, N, k)
    assert C >= 2, "the shape must take the chunk cut"
    g = torch.Generator(device=DEV).manual_seed(83000 + N)
    x = torch.randn(B, N, generator=g, device=DEV) + 8.0  # the construction passes a ReLU
    if levels:
        x = torch.clamp(torch.floor((x - 4) * 8), 0, 63) / 8     # ties at every level
    pos = torch.arange(N, device=DEV)
    grp = pos // 32
    in_chunk0 = ((grp - grp // C) % C) == 0
    # More of the row's top k sit in chunk 0 than it can keep (a chunk keeps
    # at most about twice its share k / C plus four standard deviations).
    share = k / C
    assert min(k, int(in_chunk0.sum())) > 2 * (share + 4 * share ** 0.5 + 17) + 8
    x[0::2, in_chunk0] += 16.0
    sc = x.to(torch.bfloat16)
    check(exact_inputs(sc, 8, 83100), k, f"piled into chunk 0 (C={C})", want_scores=sc)
