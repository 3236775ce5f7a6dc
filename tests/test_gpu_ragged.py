"""GPU parity of the ragged-row calls against the CPU oracle.

- dsa_topk_ragged: on an identical score row, the first min(k, lengths[b])
  slots hold exactly the oracle's selection from the row's valid prefix (in
  ascending order with sorted_index), every later slot holds -1, and the
  values are bit copies of the scores there and -inf in the empty slots.
- dsa_sparse_attend with empty slots (-1): within the attention tolerance of
  the oracle, which leaves those slots out; a row with no rows at all is 0.
- dsa_decode_step_ragged: equals the composition of the single calls bit for
  bit, its indices are the oracle's ragged top-k of the GPU's own scores, its
  index sets differ from the all-oracle chain only in the near-tie band, and
  its output matches the oracle on the GPU's indices."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_util import assert_attention_close, host, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _clamped(lengths: np.ndarray, N: int) -> np.ndarray:
    return np.clip(lengths, 0, N).astype(np.int32)


def check_ragged_topk(idx: np.ndarray, ref: np.ndarray, lengths: np.ndarray, k: int,
                      sorted_index: bool, where: str):
    assert idx.shape == ref.shape, where
    for b in range(idx.shape[0]):
        m = min(k, int(lengths[b]))
        assert np.all(idx[b, m:] == -1), f"{where}: row {b} (length {lengths[b]}) pads are not -1"
        if sorted_index:
            ok = np.array_equal(idx[b, :m], ref[b, :m])
        else:
            ok = np.array_equal(np.sort(idx[b, :m]), np.sort(ref[b, :m]))
        assert ok, f"{where}: row {b} (length {lengths[b]}) selection differs"


def run_topk(scores: torch.Tensor, lengths: np.ndarray, k: int, sorted_index=False,
             values=False, where=""):
    import indexer_top_gathered_amd as dsa
    B, N = scores.shape
    say(f"[ragged topk] {where} dtype={scores.dtype} shape={(B, N)} k={k} sorted={sorted_index} "
        f"values={values} lengths={lengths.tolist()[:12]}")
    lens = torch.from_numpy(lengths).to(DEV)
    res = dsa.dsa_topk_ragged(scores, lens, k, return_values=values, sorted_index=sorted_index)
    idx, val = (res if values else (res, None))
    torch.cuda.synchronize()
    cl = _clamped(lengths, N)
    ref = oracle.topk_ragged(host(scores), cl, k, index_order=sorted_index)
    gidx = idx.cpu().numpy()
    check_ragged_topk(gidx, ref, cl, k, sorted_index, where)
    if values:
        valid = idx >= 0
        got = torch.where(valid, val, torch.full_like(val, 0))
        want = torch.gather(scores, 1, idx.clamp(min=0).long())
        want = torch.where(valid, want, torch.full_like(want, 0))
        bits = torch.int16 if val.dtype == torch.bfloat16 else torch.int32
        assert torch.equal(got.view(bits), want.view(bits)), f"{where}: values are not bit copies"
        pads = val[~valid]
        assert bool(torch.all(torch.isneginf(pads))), f"{where}: empty slots' values are not -inf"
    return idx


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("N,k", [(5, 5), (100, 7), (5000, 100), (4096, 4096), (70000, 1),
                                 (70000, 2048), (300000, 2048)])
def test_ragged_topk_random_rows(dtype, N, k):
    B = 10
    x = workloads.normal_rows(B, N, "bf16" if dtype == torch.bfloat16 else "f32", 500 + N + k,
                              device=DEV)
    lengths = workloads.ragged_lengths(B, N, k, 600 + N)
    run_topk(x, lengths, k, where=f"normal N={N}")
    run_topk(x, lengths, k, sorted_index=True, values=True, where=f"normal N={N} sorted")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_ragged_topk_ties_and_tail_spikes(dtype):
    """Quantised rows whose tail, past each length, holds the row's largest
    values: none of them may be selected."""
    B, N, k = 8, 40000, 1500
    g = torch.Generator(device=DEV).manual_seed(91)
    x = (torch.randint(0, 7, (B, N), generator=g, device=DEV).float() / 4).to(dtype)
    lengths = workloads.ragged_lengths(B, N, k, 92)
    for b in range(B):
        x[b, int(lengths[b]):] = 1000.0
    run_topk(x, lengths, k, values=True, where="ties, spikes past the length")
    run_topk(x, lengths, k, sorted_index=True, where="ties, spikes past the length, sorted")


def test_ragged_topk_lengths_out_of_range_are_clamped():
    B, N, k = 4, 3000, 200
    x = workloads.normal_rows(B, N, "f32", 93, device=DEV)
    lengths = np.array([-5, N + 100, 150, 2 ** 31 - 1], dtype=np.int32)
    run_topk(x, lengths, k, values=True, where="lengths outside [0, N]")


def test_ragged_topk_full_lengths_equal_dsa_topk():
    import indexer_top_gathered_amd as dsa
    B, N, k = 6, 50000, 2048
    x = workloads.normal_rows(B, N, "bf16", 94, device=DEV)
    lens = torch.full((B,), N, dtype=torch.int32, device=DEV)
    for sorted_index in (False, True):
        a = dsa.dsa_topk(x, k, sorted_index=sorted_index)
        b = dsa.dsa_topk_ragged(x, lens, k, sorted_index=sorted_index)
        torch.cuda.synchronize()
        if sorted_index:
            assert torch.equal(a, b)
        else:
            assert torch.equal(a.sort(dim=1).values, b.sort(dim=1).values)


def _attend_inputs(B, N, k, W, Hq, D, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    q = torch.randn((B, Hq, D), generator=g, device=DEV).to(torch.bfloat16)
    kv = torch.randn((B, N, D), generator=g, device=DEV).to(torch.bfloat16)
    win = torch.randn((B, W, D), generator=g, device=DEV).to(torch.bfloat16) if W else None
    keys = torch.rand((B, N), generator=g, device=DEV)
    idx = keys.argsort(dim=1)[:, :k].to(torch.int32).contiguous()
    return q, kv, idx, win


@pytest.mark.parametrize("k,W,Hq,D", [(40, 0, 16, 128), (40, 7, 32, 512), (300, 128, 128, 512),
                                      (2048, 0, 64, 512), (2048, 128, 128, 512)])
def test_attend_with_empty_slots(k, W, Hq, D):
    """Empty slots as a ragged top-k leaves them (a -1 tail after the
    row's length), scattered ones, and rows with no selected rows at all."""
    import indexer_top_gathered_amd as dsa
    B, N = 6, 5000
    q, kv, idx, win = _attend_inputs(B, N, k, W, Hq, D, 700 + k + W + Hq)
    lengths = workloads.ragged_lengths(B, N, k, 701)
    for b in range(B):
        idx[b, min(k, int(lengths[b])):] = -1
    g = torch.Generator(device=DEV).manual_seed(702)
    scatter = torch.rand((B, k), generator=g, device=DEV) < 0.3
    idx[3] = torch.where(scatter[3], torch.full_like(idx[3], -1), idx[3])
    idx[5] = -1
    idx = idx.contiguous()
    say(f"[attend empty slots] k={k} W={W} Hq={Hq} D={D} lengths={lengths.tolist()}")
    out = dsa.dsa_sparse_attend(q, kv, idx, win, 1 / np.sqrt(D))
    torch.cuda.synchronize()
    ref = oracle.attend(host(q), host(kv), host(idx), None if win is None else host(win),
                        1 / np.sqrt(D))
    err = assert_attention_close(out, ref, f"empty slots k={k} W={W}")
    say(f"    max|diff| = {err:.3e}")
    if W == 0:
        assert bool(torch.all(out[0] == 0)) and bool(torch.all(out[5] == 0)), \
            "a row with no selected rows must output zeros"


def test_attend_empty_slots_equal_dropping_them():
    """A row whose slots are half empty gives what the same row with those
    slots pointing at nothing would: the softmax over the others only."""
    import indexer_top_gathered_amd as dsa
    B, N, k, W, Hq, D = 2, 4000, 1024, 64, 64, 512
    q, kv, idx, win = _attend_inputs(B, N, k, W, Hq, D, 710)
    holes = idx.clone()
    holes[:, 1::2] = -1
    a = dsa.dsa_sparse_attend(q, kv, holes.contiguous(), win, 0.05)
    b = dsa.dsa_sparse_attend(q, kv, idx[:, 0::2].contiguous(), win, 0.05)
    torch.cuda.synchronize()
    diff = (a.float() - b.float()).abs().max().item()
    assert diff <= 1e-2 * b.float().abs().max().item() + 1e-3, diff


def run_ragged_step(s: workloads.StepShape, inp: dict, lengths: np.ndarray, where: str):
    import indexer_top_gathered_amd as dsa
    say(f"[ragged step] {where} B={s.B} N={s.N} H_I={s.H_I} k={s.k} W={s.W} H_q={s.H_q} "
        f"D={s.D} lengths={lengths.tolist()[:12]}")
    lens = torch.from_numpy(lengths).to(DEV)
    out, idx = dsa.dsa_decode_step_ragged(inp["q_idx"], inp["k_idx"], inp["w"], inp["q"],
                                          inp["kv_cmp"], inp["kv_win"], lens, s.k, s.scale,
                                          return_idx=True)
    scores = dsa.dsa_indexer_score(inp["q_idx"], inp["k_idx"], inp["w"])
    idx2 = dsa.dsa_topk_ragged(scores, lens, s.k)
    out2 = dsa.dsa_sparse_attend(inp["q"], inp["kv_cmp"], idx2, inp["kv_win"], s.scale)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2), f"{where}: fused indices differ from the composition"
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)), f"{where}: fused output differs"
    cl = _clamped(lengths, s.N)
    gidx = idx.cpu().numpy()
    gscores = scores.cpu().numpy()
    check_ragged_topk(gidx, oracle.topk_ragged(gscores, cl, s.k), cl, s.k, False,
                      where + " (top-k of GPU scores)")
    # index sets against the all-oracle chain, inside each row's prefix
    ref_scores = oracle.indexer(host(inp["q_idx"]), host(inp["k_idx"]), host(inp["w"]))
    ref_idx = oracle.topk_ragged(ref_scores, cl, s.k)
    for b in range(s.B):
        m = min(s.k, int(cl[b]))
        g, r = gidx[b, :m], ref_idx[b, :m]
        if m == 0:
            continue
        assert len(np.unique(g)) == m and g.max() < cl[b], f"{where}: row {b} is not a valid set"
        tau = float(ref_scores[b, r[-1]])
        scale = abs(tau) if tau != 0 else float(np.max(ref_scores[b, :cl[b]]))
        diff = np.setxor1d(g, r)
        if diff.size:
            dev = np.abs(ref_scores[b, diff].astype(np.float64) - tau)
            assert np.all(dev <= 1e-3 * scale), f"{where}: row {b} beyond the near-tie band"
    win = None if s.W == 0 else host(inp["kv_win"])
    ref = oracle.attend(host(inp["q"]), host(inp["kv_cmp"]), gidx, win, s.scale)
    err = assert_attention_close(out, ref, where)
    say(f"    max|diff| = {err:.3e}")
    return out, idx


@pytest.mark.parametrize("shape", [
    workloads.StepShape(B=6, N=1001, H_I=13, D_I=128, k=77, W=5, H_q=32, D=128),
    workloads.StepShape(B=6, N=9000, H_I=64, D_I=128, k=1024, W=0, H_q=64, D=512),
    workloads.StepShape(B=8, N=33333, H_I=64, D_I=128, k=2048, W=128, H_q=128, D=512),
])
def test_ragged_steps(shape):
    inp = workloads.step_inputs(shape, 32000 + shape.N, device=DEV)
    lengths = workloads.ragged_lengths(shape.B, shape.N, shape.k, 33000 + shape.N)
    run_ragged_step(shape, inp, lengths, "ragged")


def test_ragged_step_full_lengths_equal_dsa_decode_step():
    import indexer_top_gathered_amd as dsa
    s = workloads.StepShape(B=4, N=20000, H_I=64, D_I=128, k=2048, W=128, H_q=128, D=512)
    inp = workloads.step_inputs(s, 34000, device=DEV)
    lens = torch.full((s.B,), s.N, dtype=torch.int32, device=DEV)
    a, ia = dsa.dsa_decode_step(inp["q_idx"], inp["k_idx"], inp["w"], inp["q"], inp["kv_cmp"],
                                inp["kv_win"], s.k, s.scale, return_idx=True)
    b, ib = dsa.dsa_decode_step_ragged(inp["q_idx"], inp["k_idx"], inp["w"], inp["q"],
                                       inp["kv_cmp"], inp["kv_win"], lens, s.k, s.scale,
                                       return_idx=True)
    ra = dsa.dsa_sparse_attend(inp["q"], inp["kv_cmp"], ia, inp["kv_win"], s.scale)
    rb = dsa.dsa_sparse_attend(inp["q"], inp["kv_cmp"], ib, inp["kv_win"], s.scale)
    torch.cuda.synchronize()
    # the same selection (the plain step's indexer and top-k are fused, so
    # its order differs), each step's output its own indices' attention
    assert torch.equal(ia.sort(dim=1).values, ib.sort(dim=1).values)
    assert torch.equal(a.view(torch.int16), ra.view(torch.int16))
    assert torch.equal(b.view(torch.int16), rb.view(torch.int16))
    lim = 1e-2 * float(b.float().abs().max()) + 1e-3
    assert float((a.float() - b.float()).abs().max()) <= lim


@pytest.mark.parametrize("B,N,zero_frac", [(150, 3000, 0.3), (200, 777, 0.9), (70, 40000, 0.0)])
def test_ragged_step_many_rows(B, N, zero_frac):
    """More than 64 rows: the indexer walks its share of the valid rounds
    across several 64-row chunks, over rows of length 0 and shares that
    start and end inside rows."""
    s = workloads.StepShape(B=B, N=N, H_I=8, D_I=128, k=min(64, N), W=0, H_q=16, D=128)
    inp = workloads.step_inputs(s, 35000 + B, device=DEV)
    rng = np.random.default_rng(B + N)
    lengths = rng.integers(1, N + 1, size=B).astype(np.int32)
    lengths[rng.random(B) < zero_frac] = 0
    lengths[-1] = N
    run_ragged_step(s, inp, lengths, f"{B} rows")


def test_ragged_step_workload_full():
    """The ragged-step bench configuration at full size: the production
    shape over lengths uniform on [1, N]."""
    s = workloads.C4
    inp = workloads.step_inputs(s, 6000, device=DEV)
    run_ragged_step(s, inp, workloads.serving_lengths(s.B, s.N, 6000), "ragged-step workload")
