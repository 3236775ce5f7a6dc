"""GPU parity of the fused dsa_decode_step against the CPU oracle.

Checked for every case: (1) the fused step's indices equal the oracle's
top-k of the GPU's own indexer scores exactly (the indexer is
deterministic, so the step's internal scores are those bits); (2) the index
set differs from the all-oracle set only inside the near-tie band; (3) the
attention output is within tolerance of the oracle evaluated on the GPU's
indices; (4) the step equals the composition of its calls: its indices are
dsa_indexer_topk's bit for bit and, as a set, dsa_topk's of
dsa_indexer_score's scores, and its output is dsa_sparse_attend's on those
indices bit for bit."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_util import (assert_attention_close, assert_index_sets_close, assert_topk_equal,
                         host, say)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_step(s: workloads.StepShape, inp: dict, where: str, rows=None):
    import indexer_top_gathered_amd as dsa
    say(f"[step] {where} B={s.B} N={s.N} H_I={s.H_I} k={s.k} W={s.W} H_q={s.H_q} D={s.D}")
    out, idx = dsa.dsa_decode_step(inp["q_idx"], inp["k_idx"], inp["w"], inp["q"],
                                   inp["kv_cmp"], inp["kv_win"], s.k, s.scale, return_idx=True)
    scores = dsa.dsa_indexer_score(inp["q_idx"], inp["k_idx"], inp["w"])
    idx1, scores1 = dsa.dsa_indexer_topk(inp["q_idx"], inp["k_idx"], inp["w"], s.k,
                                         return_scores=True)
    idx2 = dsa.dsa_topk(scores, s.k)
    out2 = dsa.dsa_sparse_attend(inp["q"], inp["kv_cmp"], idx, inp["kv_win"], s.scale)
    torch.cuda.synchronize()
    # (4) the fused step is the composition
    assert torch.equal(idx, idx1), f"{where}: step indices differ from dsa_indexer_topk's"
    assert torch.equal(scores1.view(torch.int32), scores.view(torch.int32)), \
        f"{where}: dsa_indexer_topk's scores differ from dsa_indexer_score's"
    assert torch.equal(idx.sort(dim=1).values, idx2.sort(dim=1).values), \
        f"{where}: fused index sets differ from dsa_topk's"
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)), f"{where}: fused output differs"
    gidx = idx.cpu().numpy()
    # (1) exact top-k of the GPU's own scores
    gscores = scores.cpu().numpy()
    assert_topk_equal(gidx, oracle.topk(gscores, s.k), False, where + " (top-k of GPU scores)")
    rows = list(range(s.B)) if rows is None else rows
    sel = torch.tensor(rows, device=DEV)
    # (2) index sets against the all-oracle chain
    ref_scores = oracle.indexer(host(inp["q_idx"][sel]), host(inp["k_idx"][sel]),
                                host(inp["w"][sel]))
    ref_idx = oracle.topk(ref_scores, s.k)
    assert_index_sets_close(gidx[rows], ref_scores, ref_idx, where)
    # (3) attention on the GPU's indices
    win = None if s.W == 0 else host(inp["kv_win"][sel])
    ref = oracle.attend(host(inp["q"][sel]), host(inp["kv_cmp"][sel]), gidx[rows], win,
                        s.scale)
    err = assert_attention_close(out[sel], ref, where)
    say(f"    max|diff| = {err:.3e}")
    return out, idx


@pytest.mark.parametrize("shape", [
    workloads.StepShape(B=1, N=40, H_I=8, D_I=128, k=40, W=0, H_q=16, D=128),      # k = N
    workloads.StepShape(B=3, N=1001, H_I=13, D_I=128, k=77, W=5, H_q=32, D=128),
    workloads.StepShape(B=2, N=9000, H_I=64, D_I=128, k=1024, W=128, H_q=128, D=512),
    workloads.StepShape(B=5, N=33333, H_I=64, D_I=128, k=2048, W=0, H_q=64, D=512),
    workloads.StepShape(B=2, N=5000, H_I=64, D_I=128, k=4096, W=128, H_q=128, D=512),  # largest k
    workloads.StepShape(B=200, N=700, H_I=8, D_I=128, k=64, W=16, H_q=16, D=128),     # many rows
    workloads.StepShape(B=3, N=257, H_I=1, D_I=128, k=256, W=1, H_q=16, D=512),       # one head
])
def test_small_steps(shape):
    inp = workloads.step_inputs(shape, 31000 + shape.N, device=DEV)
    run_step(shape, inp, "small")


# Shapes whose step lets the attention kernel select its rows from the chunk
# cut's candidates (D = 512, 64 heads per attention workgroup, at most 4096
# candidates per row), the cut merge's launch folded in: 8 and 4 candidate
# slots per thread, a ragged N, no window, 64 and 128 query heads, few rows
# per split, and the largest candidate count.
@pytest.mark.parametrize("shape", [
    workloads.StepShape(B=3, N=12345, H_I=64, D_I=128, k=256, W=128, H_q=128, D=512),
    workloads.StepShape(B=16, N=16384, H_I=64, D_I=128, k=256, W=0, H_q=64, D=512),
    workloads.StepShape(B=3, N=16000, H_I=16, D_I=128, k=64, W=5, H_q=128, D=512),
    workloads.StepShape(B=12, N=16384, H_I=64, D_I=128, k=1024, W=128, H_q=128, D=512),
    # two window tiles on every split (both copied before the selection)
    workloads.StepShape(B=16, N=16384, H_I=64, D_I=128, k=1024, W=512, H_q=128, D=512),
    # a last window tile of 4 rows (the rest empty slots)
    workloads.StepShape(B=16, N=16384, H_I=64, D_I=128, k=1024, W=100, H_q=128, D=512),
    # 16 splits of 64 selected rows, the last holding 40; window tiles on splits 0 and 1
    workloads.StepShape(B=8, N=16384, H_I=64, D_I=128, k=1000, W=40, H_q=128, D=512),
])
def test_steps_selecting_inside_attention(shape):
    inp = workloads.step_inputs(shape, 32000 + shape.N + shape.k, device=DEV)
    run_step(shape, inp, "selection inside attention")


def test_step_rows_the_cut_cannot_settle():
    """Rows 0 and 2 pile their top scores into chunk 0 (group g = j / 32
    belongs to chunk (g - g / C) mod C), so the selection inside attention
    takes the row again from its scores; the scores are exact (indexer query
    e_0, weights 1/H_I, key channel 0 = the wanted score)."""
    import indexer_top_gathered_amd as dsa
    s = workloads.StepShape(B=4, N=16384, H_I=16, D_I=128, k=256, W=16, H_q=128, D=512)
    C = dsa.dsa_indexer_topk_chunks(s.B, s.N, s.k)
    assert C >= 2
    inp = workloads.step_inputs(s, 33000, device=DEV)
    g = torch.Generator(device=DEV).manual_seed(33100)
    x = torch.randn(s.B, s.N, generator=g, device=DEV) + 8.0  # non-negative after rounding
    grp = torch.arange(s.N, device=DEV) // 32
    x[0::2, ((grp - grp // C) % C) == 0] += 16.0
    sc = x.to(torch.bfloat16)
    k_idx = inp["k_idx"].clone()
    k_idx[:, :, 0] = sc
    q_idx = torch.zeros_like(inp["q_idx"])
    q_idx[:, :, 0] = 1.0
    w = torch.full_like(inp["w"], 1.0 / s.H_I)
    inp = dict(inp, q_idx=q_idx, k_idx=k_idx, w=w)
    _, idx = run_step(s, inp, "rows piled into chunk 0")
    ref = oracle.topk(host(sc), s.k)
    assert_topk_equal(idx.cpu().numpy(), ref, False, "rows piled into chunk 0")


def test_tiny_step_workload_full():
    s = workloads.C1
    run_step(s, workloads.step_inputs(s, 1000, device=DEV), "tiny step workload")


def test_production_step_workload_full():
    s = workloads.C4
    run_step(s, workloads.step_inputs(s, 4000, device=DEV), "production step workload")


def test_stress_step_workload_full():
    """Stress step at full size. The indexer construction makes the scores
    exact, so the selected sets must equal the oracle's top-k of the
    quantised rows exactly. Attention is compared with the oracle on every
    batch row: each chunk of rows has its selected kv_cmp rows gathered on
    the device into a compact [rows, k, D] tensor, with the indices remapped
    to 0..k-1, so the host never holds the 17 GB cache. The fused step also
    equals the composition of the three single calls bit for bit."""
    import indexer_top_gathered_amd as dsa
    s = workloads.C5
    say("[step] stress workload: generating 21 GB of inputs")
    inp = workloads.stress_step_inputs(s, 5000, device=DEV)
    out, idx = dsa.dsa_decode_step(inp["q_idx"], inp["k_idx"], inp["w"], inp["q"],
                                   inp["kv_cmp"], inp["kv_win"], s.k, s.scale, return_idx=True)
    torch.cuda.synchronize()
    say("    fused step done; composition of the three calls")
    scores = dsa.dsa_indexer_score(inp["q_idx"], inp["k_idx"], inp["w"])
    idx2 = dsa.dsa_topk(scores, s.k)
    out2 = dsa.dsa_sparse_attend(inp["q"], inp["kv_cmp"], idx, inp["kv_win"], s.scale)
    torch.cuda.synchronize()
    assert torch.equal(idx.sort(dim=1).values, idx2.sort(dim=1).values), \
        "stress step: fused index sets differ from the composition"
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)), \
        "stress step: fused output differs from the composition"
    assert torch.equal(scores.view(torch.int32),
                       inp["stress_scores"].float().view(torch.int32)), "stress scores not exact"
    del scores, idx2, out2
    ref_idx = oracle.topk(host(inp["stress_scores"]), s.k)
    assert_topk_equal(idx.cpu().numpy(), ref_idx, False, "stress step indices")
    worst = 0.0
    chunk = 16
    for b0 in range(0, s.B, chunk):
        rows = torch.arange(b0, min(s.B, b0 + chunk), device=DEV)
        sel = idx[rows].long()                                               # [r, k]
        compact = torch.stack([inp["kv_cmp"][b][sel[i]] for i, b in enumerate(rows.tolist())])
        local = np.broadcast_to(np.arange(s.k, dtype=np.int32), (len(rows), s.k)).copy()
        ref = oracle.attend(host(inp["q"][rows]), host(compact), local,
                            host(inp["kv_win"][rows]), s.scale)
        err = assert_attention_close(out[rows], ref, f"stress step attention rows {b0}..")
        worst = max(worst, err)
        del compact
    say(f"    all {s.B} rows: max|diff| = {worst:.3e}")
    del inp, out, idx
    torch.cuda.empty_cache()


def test_deterministic_and_poisoned_workspace():
    import indexer_top_gathered_amd as dsa
    s = workloads.StepShape(B=4, N=20000, H_I=64, D_I=128, k=1024, W=128, H_q=128, D=512)
    inp = workloads.step_inputs(s, 4242, device=DEV)
    dims = dsa.make_dims(s.B, s.N, s.H_I, s.D_I, s.k, s.W, s.H_q, s.D, s.scale)
    nb = dsa.dsa_decode_step_workspace_bytes(dims)
    outs = []
    for fill in (0x00, 0xFF, 0xFF):
        ws = torch.full((nb,), fill, dtype=torch.uint8, device=DEV)
        o, i = dsa.dsa_decode_step(inp["q_idx"], inp["k_idx"], inp["w"], inp["q"], inp["kv_cmp"],
                                   inp["kv_win"], s.k, s.scale, ws=ws, return_idx=True)
        outs.append((o.clone(), i.clone()))
    torch.cuda.synchronize()
    for o, i in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0][0].view(torch.int16))
        assert torch.equal(i, outs[0][1])
