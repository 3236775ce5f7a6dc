"""GPU parity of the calls that take several query tokens per batch row
(T tokens sharing the row's keys) against the CPU oracle and against the
one-token calls.

- dsa_indexer_score_mt: each token's scores equal dsa_indexer_score on that
  token's query and weights bit for bit (the same arithmetic in the same
  order), and lie within the indexer bound of the oracle.
- dsa_sparse_attend_mt: equals dsa_sparse_attend on the flattened query rows
  with each row's compressed rows repeated per token, bit for bit, and is
  within the attention tolerance of the oracle.
- dsa_decode_step_mt (with and without per-token lengths): equals the
  composition of the single calls bit for bit, its indices are the oracle's
  top-k of the GPU's own scores, its index sets differ from the all-oracle
  chain only in the near-tie band, and its output matches the oracle on the
  GPU's indices."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_util import (assert_attention_close, assert_scores_close, host, indexer_bound,
                         say)

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("T,H,N", [(2, 8, 1000), (3, 13, 4099), (4, 64, 9001), (2, 64, 40000),
                                   (4, 33, 777)])
def test_indexer_mt(T, H, N):
    import indexer_top_gathered_amd as dsa
    B = 3
    s = workloads.StepShape(B=B, N=N, H_I=H, D_I=128, k=1, W=0, H_q=16, D=128)
    inp = workloads.mt_step_inputs(s, T, 41000 + 10 * T + H, device=DEV)
    say(f"[indexer mt] B={B} T={T} H={H} N={N}")
    got = dsa.dsa_indexer_score_mt(inp["q_idx"], inp["k_idx"], inp["w"])
    one = [dsa.dsa_indexer_score(inp["q_idx"][:, t].contiguous(), inp["k_idx"],
                                 inp["w"][:, t].contiguous()) for t in range(T)]
    torch.cuda.synchronize()
    for t in range(T):
        assert torch.equal(got[:, t].view(torch.int32), one[t].view(torch.int32)), \
            f"token {t}: differs from the one-token indexer"
    qb, kb, wn = host(inp["q_idx"]), host(inp["k_idx"]), host(inp["w"])
    ref = oracle.indexer_mt(qb, kb, wn)
    g = got.cpu().numpy()
    for t in range(T):
        assert_scores_close(g[:, t], ref[:, t], indexer_bound(qb[:, t], kb, wn[:, t]),
                            f"indexer mt T={T} token {t}")


def _attend_mt_inputs(B, T, N, k, W, Hq, D, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    q = torch.randn((B, T, Hq, D), generator=g, device=DEV).to(torch.bfloat16)
    kv = torch.randn((B, N, D), generator=g, device=DEV).to(torch.bfloat16)
    win = torch.randn((B, T, W, D), generator=g, device=DEV).to(torch.bfloat16) if W else None
    keys = torch.rand((B, T, N), generator=g, device=DEV)
    idx = keys.argsort(dim=2)[:, :, :k].to(torch.int32).contiguous()
    return q, kv, idx, win


@pytest.mark.parametrize("T,k,W,Hq,D", [(2, 40, 7, 16, 128), (3, 300, 128, 128, 512),
                                        (4, 2048, 128, 64, 512), (2, 1024, 0, 128, 512)])
def test_attend_mt(T, k, W, Hq, D):
    import indexer_top_gathered_amd as dsa
    B, N = 3, 5000
    q, kv, idx, win = _attend_mt_inputs(B, T, N, k, W, Hq, D, 42000 + T + k)
    idx[1, T - 1, k // 2:] = -1   # a token with a short selection
    say(f"[attend mt] B={B} T={T} k={k} W={W} Hq={Hq} D={D}")
    scale = 1 / np.sqrt(D)
    out = dsa.dsa_sparse_attend_mt(q, kv, idx, win, scale)
    flat = dsa.dsa_sparse_attend(q.reshape(B * T, Hq, D), kv.repeat_interleave(T, dim=0),
                                 idx.reshape(B * T, k),
                                 None if win is None else win.reshape(B * T, W, D), scale)
    torch.cuda.synchronize()
    assert torch.equal(out.reshape(B * T, Hq, D).view(torch.int16), flat.view(torch.int16)), \
        "differs from the one-token call on flattened rows"
    ref = oracle.attend_mt(host(q), host(kv), host(idx), None if win is None else host(win), scale)
    err = assert_attention_close(out, ref, f"attend mt T={T} k={k}")
    say(f"    max|diff| = {err:.3e}")


def run_step_mt(s: workloads.StepShape, T: int, inp: dict, lengths, where: str):
    import indexer_top_gathered_amd as dsa
    B, N, k = s.B, s.N, s.k
    say(f"[step mt] {where} B={B} T={T} N={N} H_I={s.H_I} k={k} W={s.W} H_q={s.H_q} D={s.D} "
        f"lengths={'none' if lengths is None else lengths.reshape(-1).tolist()[:12]}")
    lens = None if lengths is None else torch.from_numpy(lengths).to(DEV)
    out, idx = dsa.dsa_decode_step_mt(inp["q_idx"], inp["k_idx"], inp["w"], inp["q"],
                                      inp["kv_cmp"], inp["kv_win"], k, s.scale, lengths=lens,
                                      return_idx=True)
    scores = dsa.dsa_indexer_score_mt(inp["q_idx"], inp["k_idx"], inp["w"])
    flat = scores.reshape(B * T, N)
    if lens is None:
        idx2 = dsa.dsa_topk(flat, k)
    else:
        idx2 = dsa.dsa_topk_ragged(flat, lens.reshape(-1), k)
    out2 = dsa.dsa_sparse_attend_mt(inp["q"], inp["kv_cmp"], idx2.reshape(B, T, k), inp["kv_win"],
                                    s.scale)
    torch.cuda.synchronize()
    assert torch.equal(idx.reshape(B * T, k), idx2), f"{where}: fused indices differ"
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)), f"{where}: fused output differs"
    gidx = idx.cpu().numpy().reshape(B * T, k)
    gs = flat.cpu().numpy()
    cl = None if lengths is None else np.clip(lengths.reshape(-1), 0, N).astype(np.int32)
    ref_g = oracle.topk(gs, k) if cl is None else oracle.topk_ragged(gs, cl, k)
    for r in range(B * T):
        m = k if cl is None else min(k, int(cl[r]))
        assert np.all(gidx[r, m:] == -1), f"{where}: row {r} pads"
        assert np.array_equal(np.sort(gidx[r, :m]), np.sort(ref_g[r, :m])), \
            f"{where}: row {r} is not the top-k of the GPU's scores"
    # index sets against the all-oracle chain, inside each row's prefix
    ref_s = oracle.indexer_mt(host(inp["q_idx"]), host(inp["k_idx"]), host(inp["w"])).reshape(B * T, N)
    ref_i = oracle.topk(ref_s, k) if cl is None else oracle.topk_ragged(ref_s, cl, k)
    for r in range(B * T):
        m = k if cl is None else min(k, int(cl[r]))
        if m == 0:
            continue
        tau = float(ref_s[r, ref_i[r, m - 1]])
        valid = N if cl is None else int(cl[r])
        scale = abs(tau) if tau != 0 else float(np.max(ref_s[r, :valid]))
        diff = np.setxor1d(gidx[r, :m], ref_i[r, :m])
        if diff.size:
            dev = np.abs(ref_s[r, diff].astype(np.float64) - tau)
            assert np.all(dev <= 1e-3 * scale), f"{where}: row {r} beyond the near-tie band"
    win = None if s.W == 0 else host(inp["kv_win"])
    ref = oracle.attend_mt(host(inp["q"]), host(inp["kv_cmp"]), gidx.reshape(B, T, k), win, s.scale)
    err = assert_attention_close(out, ref, where)
    say(f"    max|diff| = {err:.3e}")


@pytest.mark.parametrize("shape,T", [
    (workloads.StepShape(B=2, N=1001, H_I=13, D_I=128, k=77, W=5, H_q=32, D=128), 3),
    (workloads.StepShape(B=3, N=9000, H_I=64, D_I=128, k=1024, W=128, H_q=128, D=512), 2),
    (workloads.StepShape(B=2, N=33333, H_I=64, D_I=128, k=2048, W=0, H_q=64, D=512), 4),
])
def test_step_mt(shape, T):
    inp = workloads.mt_step_inputs(shape, T, 43000 + shape.N + T, device=DEV)
    run_step_mt(shape, T, inp, None, "full rows")
    rng = np.random.default_rng(shape.N)
    lengths = rng.integers(0, shape.N + 1, size=(shape.B, T)).astype(np.int32)
    lengths[0, 0] = 0
    lengths[-1, -1] = min(shape.k, shape.N) - 1
    run_step_mt(shape, T, inp, lengths, "per-token lengths")


def test_one_token_mt_calls_equal_the_one_token_calls():
    import indexer_top_gathered_amd as dsa
    s = workloads.StepShape(B=4, N=20000, H_I=64, D_I=128, k=1024, W=128, H_q=128, D=512)
    inp = workloads.step_inputs(s, 44000, device=DEV)
    a, ia = dsa.dsa_decode_step(inp["q_idx"], inp["k_idx"], inp["w"], inp["q"], inp["kv_cmp"],
                                inp["kv_win"], s.k, s.scale, return_idx=True)
    b, ib = dsa.dsa_decode_step_mt(inp["q_idx"][:, None], inp["k_idx"], inp["w"][:, None],
                                   inp["q"][:, None], inp["kv_cmp"], inp["kv_win"][:, None], s.k,
                                   s.scale, return_idx=True)
    torch.cuda.synchronize()
    assert torch.equal(ia, ib[:, 0])
    assert torch.equal(a.view(torch.int16), b[:, 0].view(torch.int16))


def test_mtp_step_workload_full():
    """The mtp-step bench configuration at full size: the production shape
    with 2 query tokens per row."""
    s = workloads.C4
    inp = workloads.mt_step_inputs(s, 2, 7000, device=DEV)
    run_step_mt(s, 2, inp, None, "mtp-step workload")
