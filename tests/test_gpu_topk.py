"""GPU parity of dsa_topk against the CPU oracle: given an identical score row
the GPU index set, and the values when returned, must equal the oracle's
exactly (order too when sorted_index is set)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_util import assert_topk_equal, assert_values_are_copies, host, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_case(scores: torch.Tensor, k: int, sorted_index=False, values=False, where=""):
    say(f"[topk] {where} dtype={scores.dtype} shape={tuple(scores.shape)} k={k} "
        f"sorted={sorted_index} values={values}")
    import indexer_top_gathered_amd as dsa
    res = dsa.dsa_topk(scores, k, return_values=values, sorted_index=sorted_index)
    idx, val = (res if values else (res, None))
    torch.cuda.synchronize()
    ref = oracle.topk(host(scores), k, index_order=False)
    assert_topk_equal(idx.cpu().numpy(), ref, sorted_index, where)
    if values:
        assert_values_are_copies(val, scores, idx, where)
    return idx


def _ties(B, N, levels, seed, dtype):
    g = torch.Generator(device=DEV).manual_seed(seed)
    x = torch.randint(0, levels, (B, N), generator=g, device=DEV).float() / 4 - levels / 8
    return x.to(dtype)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("N,k", [(1, 1), (5, 5), (7, 3), (100, 1), (4096, 4096), (4097, 100),
                                 (10001, 1000), (40000, 333), (131072, 512), (300000, 2048),
                                 (50000, 4096), (8193, 1024), (16385, 4096), (32769, 777),
                                 (65536, 2048), (8000, 4000)])
def test_random_rows(dtype, N, k):
    B = 3 if N < 200000 else 2
    x = workloads.normal_rows(B, N, "bf16" if dtype == torch.bfloat16 else "f32", 1234 + N,
                              device=DEV)
    run_case(x, k, where=f"normal N={N}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("levels", [1, 2, 7, 256])
def test_heavy_ties(dtype, levels):
    x = _ties(4, 20011, levels, 77 + levels, dtype)
    run_case(x, 1500, values=True, where=f"ties levels={levels}")
    run_case(x, 1500, sorted_index=True, where=f"ties levels={levels} sorted")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("k", [1, 37, 2048])
def test_special_rows(dtype, k):
    N = 70000
    ar = torch.arange(N, device=DEV, dtype=torch.float32)
    rows = torch.stack([
        torch.full((N,), 0.5, device=DEV),      # all equal
        ar / 64,                                 # ascending (ties in bf16)
        ar.flip(0) / 64,                         # descending
        (ar % 1000) / 10,                        # saw-tooth
    ]).to(dtype)
    idx = run_case(rows, k, sorted_index=True, values=True, where="special rows").cpu().numpy()
    assert idx[0].tolist() == list(range(k))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_rising_and_falling_long_rows(dtype):
    # Segments of several register blocks: a rising row beats the running
    # bound in every later block (each block then takes its own threshold and
    # the list is compacted); a falling row is settled by its first block.
    N = 262144
    ar = torch.arange(N, device=DEV, dtype=torch.float32)
    rows = torch.stack([ar, ar.flip(0), (ar % 4096) + ar / N]).to(dtype)
    run_case(rows, 2048, values=True, where="rising/falling long rows")
    run_case(rows, 777, sorted_index=True, where="rising/falling long rows sorted")


@pytest.mark.parametrize("lift", [0.75, 10.0])
def test_segments_outgrowing_their_first_threshold(lift):
    # float32 rows of 262144 with k = 2048 take the quota form in 4 segments
    # of 4 register blocks. A random first three blocks set the threshold
    # and predict a list that fits the segment's slots, so the threshold is
    # kept for the last block; lifting the last quarter of the row (most of
    # each segment's last block) makes that block overflow the prediction
    # (0.75: the final cut to the slots) or the whole LDS list (10: the
    # block takes its own threshold).
    N = 262144
    g = torch.Generator(device=DEV).manual_seed(61)
    x = torch.randn((3, N), generator=g, device=DEV)
    x[:, 3 * N // 4:] += lift
    x[2] = x[2].round(decimals=1)  # ties across the lifted and plain parts
    run_case(x, 2048, values=True, where=f"last quarter lifted by {lift}")
    run_case(x, 2048, sorted_index=True, where=f"last quarter lifted by {lift}, sorted")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_heavy_bucket_of_several_values(dtype):
    # A few huge scores stretch the candidates' range, so one histogram
    # bucket holds the whole cluster below them: more than 512 entries of
    # several distinct values, with the k-th inside. Low background elsewhere.
    N = 65536
    g = torch.Generator(device=DEV).manual_seed(8)
    x = -1.0e6 - torch.rand((2, N), generator=g, device=DEV)
    pos = torch.randperm(N, generator=g, device=DEV)
    huge, clus = pos[:10], pos[10:3010]
    x[:, huge] = 1.0e30 * (1 + torch.arange(10, device=DEV, dtype=torch.float32))
    if dtype == torch.float32:
        base = torch.tensor(1.0, dtype=torch.float32, device=DEV).view(torch.int32)
        vals = (base + torch.arange(3000, device=DEV, dtype=torch.int32) % 1000).view(torch.float32)
    else:  # eight adjacent bf16 values above 1.0
        vals = 1.0 + (torch.arange(3000, device=DEV, dtype=torch.float32) % 8) / 128
    x[:, clus] = vals
    x = x.to(dtype)
    run_case(x, 1510, values=True, where="heavy multi-value bucket")
    run_case(x, 1510, sorted_index=True, where="heavy multi-value bucket sorted")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_signed_zero_infinity_and_subnormal(dtype):
    N = 9000
    g = torch.Generator(device=DEV).manual_seed(5)
    x = torch.randn((2, N), generator=g, device=DEV) * 1e-3
    x[:, ::7] = 0.0
    x[:, 3::7] = -0.0
    x[0, 100] = float("inf")
    x[0, 200] = float("-inf")
    x[1, 5:50] = float("-inf")
    x[1, 60:70] = float("inf")
    x[1, 80] = 1e-40  # subnormal in float32 (flushed to a bf16 subnormal/zero after rounding)
    x = x.to(dtype)
    # about 3200 scores are positive, so k reaches into the zeros: -0.0 and
    # +0.0 must tie and go by index
    run_case(x, 4000, values=True, where="signed zeros")
    run_case(x, 4000, sorted_index=True, values=True, where="signed zeros sorted")


def test_negative_rows_and_wide_range():
    g = torch.Generator(device=DEV).manual_seed(6)
    x = -torch.rand((3, 65536), generator=g, device=DEV) * torch.logspace(-30, 30, 65536, device=DEV)
    run_case(x, 777, values=True, where="negative wide range")


def test_sampling_workload_full():
    s = workloads.C3
    x = workloads.sampling_rows(s.B, s.N, 3006, device=DEV)
    run_case(x, s.k, values=True, where="sampling workload 128x129280 k=1024")


def test_indexer_topk_workload_full():
    s = workloads.C2
    x = workloads.normal_rows(s.B, s.N, "bf16", 2006, device=DEV)
    run_case(x, s.k, where="indexer-shaped workload 64x131072 bf16 k=512")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_stress_levels_full(dtype):
    s = workloads.C5_TOPK
    x = workloads.stress_levels(s.B, s.N, 5008, device=DEV, dtype=dtype)
    run_case(x, s.k, where=f"stress levels 64x262144 k=2048 {dtype}")
    run_case(x, s.k, sorted_index=True, values=True, where=f"stress levels {dtype} sorted")


def test_deterministic_and_workspace_contents_do_not_matter():
    import indexer_top_gathered_amd as dsa
    x = workloads.normal_rows(8, 100003, "f32", 99, device=DEV)
    k = 1024
    nb = dsa.dsa_topk_workspace_bytes(8, 100003, k, torch.float32)
    ws1 = torch.zeros(nb, dtype=torch.uint8, device=DEV)
    ws2 = torch.full((nb,), 0xFF, dtype=torch.uint8, device=DEV)
    a, av = dsa.dsa_topk(x, k, return_values=True, ws=ws1)
    b, bv = dsa.dsa_topk(x, k, return_values=True, ws=ws2)
    c, cv = dsa.dsa_topk(x, k, return_values=True, ws=ws2)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(b, c)
    assert torch.equal(av, bv)


def _segment_zero_positions(N: int, segs: int, piece: int) -> torch.Tensor:
    """Positions of the pieces that the rotating interleave gives segment 0:
    piece g (of `piece` scores) sits in run g // segs at slot g % segs, and
    segment s owns slot (s + run) mod segs."""
    g = torch.arange((N + piece - 1) // piece, device=DEV)
    mine = g[(g % segs - g // segs) % segs == 0]
    pos = (mine[:, None] * piece + torch.arange(piece, device=DEV)[None, :]).reshape(-1)
    return pos[pos < N]


# (N, k, segments, quota) of full rows split for the quota form at B = 3:
# 8 one-block segments keeping 113 each of k = 512, and 2 segments of
# several blocks keeping 2246 each of k = 4096.
QUOTA_SHAPES = [(131072, 512, 8, 113), (131072, 4096, 2, 2246)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("N,k,segs,quota", QUOTA_SHAPES)
def test_rows_whose_top_k_sits_in_one_segment(dtype, N, k, segs, quota):
    # Full rows split into a power-of-two number of segments keep only about
    # their share of the top k each. Rows 0 and 2 put every large score into
    # the pieces of one segment, so that segment drops scores of the row's top
    # k: the merge must see it through the cuts and select those rows again
    # from their scores. Row 1 is random (settled by the segments' quotas).
    B = 3
    piece = 64 if dtype == torch.bfloat16 else 32
    g = torch.Generator(device=DEV).manual_seed(41)
    x = torch.randn((B, N), generator=g, device=DEV)
    pos = _segment_zero_positions(N, segs, piece)
    x[0, pos] += 100.0
    # row 2: ties on the boosted level, so the fallback also breaks ties
    x[2, pos] = 7.0
    x = x.to(dtype)
    run_case(x, k, where=f"top k in one segment N={N}")
    run_case(x, k, values=True, where=f"top k in one segment N={N}, values")
    idx = run_case(x, k, sorted_index=True, values=True, where=f"top k in one segment N={N}, sorted")
    assert idx[2].cpu().tolist() == pos[:k].cpu().tolist()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("N,k,segs,quota", QUOTA_SHAPES)
def test_segment_quota_edges(dtype, N, k, segs, quota):
    # quota, quota + 1 and 3.5 quota boosted scores in one segment's pieces,
    # the rest of the row random: with its random share the segment holds
    # more of the row's top k than its quota in every row, by a little or a
    # lot; the results must be exact either way.
    B = 3
    piece = 64 if dtype == torch.bfloat16 else 32
    g = torch.Generator(device=DEV).manual_seed(43)
    x = torch.randn((B, N), generator=g, device=DEV)
    pos = _segment_zero_positions(N, segs, piece)
    for row, n in ((0, quota), (1, quota + 1), (2, min(k, 7 * quota // 2))):
        x[row, pos[:n]] += 50.0
    x = x.to(dtype)
    run_case(x, k, values=True, where=f"segment quota edges N={N}")
    run_case(x, k, sorted_index=True, where=f"segment quota edges N={N} sorted")
