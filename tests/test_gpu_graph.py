"""HIP-graph capture of the fused steps.

The enqueue sequence of dsa_decode_step (and of its ragged and multi-token
forms) holds no host synchronisation, no allocation and no memset, so a
caller can capture it into a graph. Each replay is compared bit for bit with
an eager call on the same inputs. Between replays the captured input buffers
are rewritten in place (the graph must read the live buffers) and eager work
and synchronisations run.
"""
from __future__ import annotations

import pytest
import torch

import workloads
from parity_util import say

pytestmark = pytest.mark.gpu
DEV = "cuda"

SHAPES = [
    workloads.StepShape(B=1, N=4096, H_I=8, D_I=128, k=256, W=64, H_q=16, D=128),
    workloads.StepShape(B=4, N=20000, H_I=64, D_I=128, k=1024, W=128, H_q=128, D=512),
    # the attention kernel selects its rows from the chunk cut (no merge launch)
    workloads.StepShape(B=3, N=12345, H_I=64, D_I=128, k=256, W=128, H_q=128, D=512),
]


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm-up call outside the graph
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a, b)


@pytest.mark.parametrize("variant", ["step", "ragged", "tokens"])
@pytest.mark.parametrize("si", range(len(SHAPES)))
def test_captured_step_replays_equal_eager(variant, si):
    import indexer_top_gathered_amd as dsa
    s = SHAPES[si]
    T = 2 if variant == "tokens" else 1
    say(f"[graph] {variant} B={s.B} N={s.N} k={s.k} H_q={s.H_q} D={s.D} T={T}")

    def make_inputs(seed):
        if variant == "tokens":
            return workloads.mt_step_inputs(s, T, seed, device=DEV)
        return workloads.step_inputs(s, seed, device=DEV)

    def make_lengths(seed):
        if variant == "step":
            return None
        n = s.B * T
        ln = torch.tensor(workloads.serving_lengths(n, s.N, seed), dtype=torch.int32, device=DEV)
        ln[0] = min(s.k - 1, s.N)  # one row shorter than k: -1 slots
        return ln.view(s.B, T) if variant == "tokens" else ln

    inp = make_inputs(9100 + si)
    lengths = make_lengths(9200 + si)
    rows = s.B * T
    out = torch.empty((rows, s.H_q, s.D), dtype=torch.bfloat16, device=DEV)
    idx = torch.empty((rows, s.k), dtype=torch.int32, device=DEV)
    dims = dsa.make_dims(s.B, s.N, s.H_I, s.D_I, s.k, s.W, s.H_q, s.D, s.scale)
    nb = (dsa.dsa_decode_step_mt_workspace_bytes(dims, T) if variant == "tokens"
          else dsa.dsa_decode_step_workspace_bytes(dims))
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=DEV)

    def call(c, ln, o, i, w):
        if variant == "step":
            dsa.dsa_decode_step(c["q_idx"], c["k_idx"], c["w"], c["q"], c["kv_cmp"], c["kv_win"],
                                s.k, s.scale, out=o, out_idx=i, ws=w)
        elif variant == "ragged":
            dsa.dsa_decode_step_ragged(c["q_idx"], c["k_idx"], c["w"], c["q"], c["kv_cmp"],
                                       c["kv_win"], ln, s.k, s.scale, out=o, out_idx=i, ws=w)
        else:
            dsa.dsa_decode_step_mt(c["q_idx"], c["k_idx"], c["w"], c["q"], c["kv_cmp"],
                                   c["kv_win"], s.k, s.scale, lengths=ln,
                                   out=o.view(s.B, T, s.H_q, s.D), out_idx=i.view(s.B, T, s.k),
                                   ws=w)

    g = _capture(lambda: call(inp, lengths, out, idx, ws))

    ref_out = torch.empty_like(out)
    ref_idx = torch.empty_like(idx)
    ref_ws = torch.empty_like(ws)
    for rep in range(3):
        fresh = make_inputs(9300 + 10 * si + rep)
        for name, t in inp.items():
            t.copy_(fresh[name])
        if lengths is not None:
            lengths.copy_(make_lengths(9400 + 10 * si + rep))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        call(inp, lengths, ref_out, ref_idx, ref_ws)  # eager, on the same inputs
        torch.cuda.synchronize()
        assert _same(idx, ref_idx), f"replay {rep}: indices differ from the eager call"
        assert _same(out, ref_out), f"replay {rep}: output differs from the eager call"
        say(f"    replay {rep}: equal to eager")
    del g


# Full rows of these shapes take the top-k's quota form (segment cuts in the
# workspace, checked by the merge).
TOPK_SHAPES = [(16, 131072, 512, torch.bfloat16, False, False),
               (8, 129280, 1024, torch.float32, True, True)]


@pytest.mark.parametrize("ti", range(len(TOPK_SHAPES)))
def test_captured_topk_replays_equal_eager(ti):
    import indexer_top_gathered_amd as dsa
    B, N, k, dt, values, sorted_index = TOPK_SHAPES[ti]
    say(f"[graph] topk B={B} N={N} k={k} dtype={dt} values={values} sorted={sorted_index}")
    tag = "bf16" if dt == torch.bfloat16 else "f32"
    x = workloads.normal_rows(B, N, tag, 9500 + ti, device=DEV)
    idx = torch.empty((B, k), dtype=torch.int32, device=DEV)
    val = torch.empty((B, k), dtype=dt, device=DEV) if values else None
    ws = torch.empty(max(dsa.dsa_topk_workspace_bytes(B, N, k, dt), 256), dtype=torch.uint8, device=DEV)

    def call(o, v, w):
        dsa.dsa_topk(x, k, return_values=values, sorted_index=sorted_index, out_idx=o, out_val=v, ws=w)

    g = _capture(lambda: call(idx, val, ws))
    ref_idx = torch.empty_like(idx)
    ref_val = torch.empty_like(val) if values else None
    ref_ws = torch.empty_like(ws)
    for rep in range(3):
        fresh = workloads.normal_rows(B, N, tag, 9600 + 10 * ti + rep, device=DEV)
        if rep == 2:  # a row whose top k sits in few segments: the merge's fallback
            fresh[0, : 4 * k] += 50.0
        x.copy_(fresh)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        call(ref_idx, ref_val, ref_ws)  # eager, on the same inputs
        torch.cuda.synchronize()
        assert _same(idx, ref_idx), f"replay {rep}: indices differ from the eager call"
        if values:
            assert _same(val, ref_val), f"replay {rep}: values differ from the eager call"
        say(f"    replay {rep}: equal to eager")
    del g
