"""GPU parity of the attention sink and the compressor against the oracle.

Attention with a sink (one logit per query head that joins the softmax
normalisation with no value vector) is held to the attention bar,
max|out - ref| <= 1e-2 max|ref| + 1e-3, with the oracle evaluated on the
same indices; a sink of -inf on every head must reproduce dsa_sparse_attend
bit for bit; the fused step with a sink must equal its composition bit for
bit. The compressor is compared element by element with the oracle's
double-precision value c under a bound derived from its float32
arithmetic: the gate sums of D products carry at most about (D/64 + 6)
roundings each, which moves each softmax weight by a relative 2 dz + 8 u at
most (u = 2^-24, dz the gate sums' error bound), and the bf16 rounding of
the result adds at most half an ulp:
  |out - c| <= 2^-8 |c| + sum_i a_i |x_i| (2 dz + 2^-20) + 2^-126.
A gate that leaves one row with all the weight must give that row exactly.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_util import assert_attention_close, host, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _sinks(Hq, g):
    s = torch.linspace(-6.0, 9.0, Hq)
    s = s[torch.randperm(Hq, generator=g)]
    s[0] = -math.inf                      # one head without a sink
    return s.float()


@pytest.mark.parametrize("shape", [
    # (B, N, k, W, H_q, D): one split and several splits, both head dims
    (2, 300, 40, 8, 16, 128),
    (3, 5000, 512, 64, 32, 128),
    (2, 9000, 1024, 128, 128, 512),
    (1, 4096, 2048, 0, 64, 512),
])
def test_sparse_attend_sink_matches_oracle(shape):
    import indexer_top_gathered_amd as dsa
    B, N, k, W, Hq, D = shape
    say(f"[sink] attend B={B} N={N} k={k} W={W} H_q={Hq} D={D}")
    g = torch.Generator().manual_seed(7000 + N)
    s = workloads.StepShape(B=B, N=N, H_I=8, D_I=128, k=k, W=W, H_q=Hq, D=D)
    inp = workloads.step_inputs(s, 71000 + N, device=DEV)
    idx = torch.stack([torch.randperm(N, generator=g)[:k] for _ in range(B)]).int().to(DEV)
    sink = _sinks(Hq, g).to(DEV)
    win = inp["kv_win"] if W else None
    out = dsa.dsa_sparse_attend_sink(inp["q"], inp["kv_cmp"], idx, win, sink, s.scale)
    plain = dsa.dsa_sparse_attend(inp["q"], inp["kv_cmp"], idx, win, s.scale)
    none = dsa.dsa_sparse_attend_sink(inp["q"], inp["kv_cmp"], idx, win,
                                      torch.full((Hq,), -math.inf, device=DEV), s.scale)
    torch.cuda.synchronize()
    assert torch.equal(none.view(torch.int16), plain.view(torch.int16)), "sink -inf != no sink"
    ref = oracle.attend(host(inp["q"]), host(inp["kv_cmp"]), idx.cpu().numpy(),
                        None if win is None else host(win), s.scale,
                        sink=sink.double().cpu().numpy())
    err = assert_attention_close(out, ref, f"sink attention {shape}")
    assert float((out.float() - plain.float()).abs().max()) > 1e-3, "the sink had no effect"
    say(f"    max|diff| = {err:.3e}")


def test_sparse_attend_sink_with_empty_slots():
    import indexer_top_gathered_amd as dsa
    B, N, k, W, Hq, D = 3, 2000, 200, 0, 32, 512
    g = torch.Generator().manual_seed(7100)
    s = workloads.StepShape(B=B, N=N, H_I=8, D_I=128, k=k, W=W, H_q=Hq, D=D)
    inp = workloads.step_inputs(s, 71100, device=DEV)
    idx = torch.stack([torch.randperm(N, generator=g)[:k] for _ in range(B)]).int()
    idx[0, 150:] = -1          # a ragged tail
    idx[1, ::3] = -1           # scattered empty slots
    idx[2, :] = -1             # a batch row with no rows at all: zeros
    idx = idx.to(DEV)
    sink = _sinks(Hq, g).to(DEV)
    out = dsa.dsa_sparse_attend_sink(inp["q"], inp["kv_cmp"], idx, None, sink, s.scale)
    torch.cuda.synchronize()
    ref = oracle.attend(host(inp["q"]), host(inp["kv_cmp"]), idx.cpu().numpy(), None, s.scale,
                        sink=sink.double().cpu().numpy())
    assert_attention_close(out, ref, "sink attention with empty slots")
    assert torch.equal(out[2].float(), torch.zeros_like(out[2].float()))


@pytest.mark.parametrize("shape", [
    workloads.StepShape(B=2, N=3000, H_I=8, D_I=128, k=256, W=16, H_q=16, D=128),
    workloads.C4,
])
def test_decode_step_sink_is_the_composition_and_matches_oracle(shape):
    import indexer_top_gathered_amd as dsa
    s = shape
    say(f"[sink] step B={s.B} N={s.N} k={s.k} H_q={s.H_q} D={s.D}")
    inp = workloads.step_inputs(s, 72000 + s.N, device=DEV)
    sink = _sinks(s.H_q, torch.Generator().manual_seed(s.N)).to(DEV)
    out, idx = dsa.dsa_decode_step_sink(inp["q_idx"], inp["k_idx"], inp["w"], inp["q"],
                                        inp["kv_cmp"], inp["kv_win"], sink, s.k, s.scale,
                                        return_idx=True)
    scores = dsa.dsa_indexer_score(inp["q_idx"], inp["k_idx"], inp["w"])
    idx2 = dsa.dsa_topk(scores, s.k)
    out2 = dsa.dsa_sparse_attend_sink(inp["q"], inp["kv_cmp"], idx, inp["kv_win"], sink,
                                      s.scale)
    torch.cuda.synchronize()
    assert torch.equal(idx.sort(dim=1).values, idx2.sort(dim=1).values)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    ref = oracle.attend(host(inp["q"]), host(inp["kv_cmp"]), idx.cpu().numpy(),
                        host(inp["kv_win"]), s.scale, sink=sink.double().cpu().numpy())
    err = assert_attention_close(out, ref, "step with sink")
    say(f"    max|diff| = {err:.3e}")


def _compress_bound(x_bits: np.ndarray, wg: np.ndarray, c: np.ndarray) -> np.ndarray:
    """Right-hand side of the compressor bound, float64 [B, G, D]."""
    x = torch.from_numpy(x_bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    B, R, D = x.shape
    xg = x.reshape(B, R // 4, 4, D)
    z = np.einsum("bgid,d->bgi", xg, wg.astype(np.float64))
    S = np.einsum("bgid,d->bgi", np.abs(xg), np.abs(wg.astype(np.float64)))
    a = np.exp(z - z.max(-1, keepdims=True))
    a /= a.sum(-1, keepdims=True)
    dz = (D / 64 + 8) * 2.0 ** -24 * S.max(-1)                                  # [B, G]
    spread = np.einsum("bgi,bgid->bgd", a, np.abs(xg))
    return 2.0 ** -8 * np.abs(c) + spread * (2 * dz[..., None] + 2.0 ** -20) + 2.0 ** -126


@pytest.mark.parametrize("B,G,D", [(1, 1, 512), (16, 1, 512), (3, 37, 128), (2, 5, 1024),
                                   (4, 9, 264), (1, 200, 512)])
def test_compress_matches_oracle(B, G, D):
    import indexer_top_gathered_amd as dsa
    say(f"[compress] B={B} G={G} D={D}")
    g = torch.Generator(device=DEV).manual_seed(73000 + B * G + D)
    x = torch.randn(B, 4 * G, D, generator=g, device=DEV).to(torch.bfloat16)
    wg = (torch.randn(D, generator=g, device=DEV) * (3.0 / math.sqrt(D))).float()
    out = dsa.dsa_compress(x, wg)
    torch.cuda.synchronize()
    xb, wgh = host(x), wg.cpu().numpy()
    c = oracle.compress(xb, wgh)
    got = out.float().cpu().numpy().astype(np.float64)
    bound = _compress_bound(xb, wgh, c)
    err = np.abs(got - c)
    assert np.all(err <= bound), f"{int((err > bound).sum())} values outside the bound"
    say(f"    max|diff| = {err.max():.3e}")


def test_compress_dominant_gate_gives_that_row_exactly():
    import indexer_top_gathered_amd as dsa
    B, G, D = 4, 6, 512
    g = torch.Generator(device=DEV).manual_seed(74000)
    x = torch.randn(B, G, 4, D, generator=g, device=DEV)
    x[..., 0] = 0.0
    winner = torch.randint(0, 4, (B, G), generator=g, device=DEV)
    x = x.to(torch.bfloat16)
    # row `winner` of each group gets gate score 200, the others 0
    x[torch.arange(B, device=DEV)[:, None], torch.arange(G, device=DEV)[None, :], winner, 0] = 200.0
    picked = x[torch.arange(B, device=DEV)[:, None], torch.arange(G, device=DEV)[None, :], winner]
    wg = torch.zeros(D, device=DEV)
    wg[0] = 1.0
    out = dsa.dsa_compress(x.view(B, 4 * G, D).contiguous(), wg)
    torch.cuda.synchronize()
    # exp(-200) underflows float32: every other weight is exactly 0
    assert torch.equal(out.view(torch.int16), picked.view(torch.int16))
