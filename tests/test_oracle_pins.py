"""Pins for the CPU oracle (no GPU).

Each test checks the oracle against something other than itself: a library
routine (torch's bf16 conversion, torch.matmul, torch.topk,
scaled_dot_product_attention), a closed form, an invariant, or the O(N^2)
rank definition of top-k in oracle/brute.py. Cases are chosen so that a
dropped term, a wrong sign, a wrong index or a transposed operand in the
oracle fails at least one of them.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
import workloads


def bf16_bits(x: torch.Tensor) -> np.ndarray:
    return workloads.bits16(x.to(torch.bfloat16))


# ---------------------------------------------------------------- decoding

def test_bf16_decode_matches_torch_on_every_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    exp = (bits >> 7) & 0xFF
    man = bits & 0x7F
    keep = ~((exp == 0xFF) & (man != 0))  # drop NaNs
    bits = bits[keep]
    got = oracle.bf16_decode(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64)
    assert np.array_equal(got, ref.numpy())


# ---------------------------------------------------------------- indexer

def test_indexer_single_head_is_relu_of_matmul():
    """H=1, w=1: the score is ReLU(K q), checked against torch.matmul in fp64."""
    g = torch.Generator().manual_seed(11)
    B, N, D = 3, 257, 128
    q = torch.randn(B, 1, D, generator=g).to(torch.bfloat16)
    k = torch.randn(B, N, D, generator=g).to(torch.bfloat16)
    w = np.ones((B, 1), np.float32)
    got = oracle.indexer(bf16_bits(q), bf16_bits(k), w)
    ref = torch.relu(torch.matmul(k.double(), q.double().transpose(1, 2)))[..., 0]
    ref32 = ref.float().numpy()
    # The fp64 sums may differ in order; after rounding to fp32 at most 1 ulp apart.
    assert np.all(np.abs(got - ref32) <= np.spacing(np.abs(ref32)) + 0.0)
    assert (ref32 == 0).sum() > 100  # ReLU actually clipped many scores


def _dyadic_bf16(g, shape, lo=-16, hi=16, denom=8):
    """Values m/denom with integer m in [lo, hi): exact in bf16."""
    m = torch.randint(lo, hi, shape, generator=g)
    return (m.double() / denom)


def test_indexer_one_hot_closed_form_exact():
    """One-hot indexer queries q[b,h] = c_h * e_{d_h}: the score is
    sum_h w[b,h] * max(0, c_h * K[b,j,d_h]), evaluated exactly with Fractions.
    Distinct channels, signs and weights per (b,h) catch transposed or shifted
    indices, a missing ReLU and a wrong head weight."""
    g = torch.Generator().manual_seed(5)
    B, N, H, D = 2, 33, 5, 16
    K = _dyadic_bf16(g, (B, N, D))
    chans = [[(3 * h + 7 * b + 1) % D for h in range(H)] for b in range(B)]
    coefs = [[[1.0, -1.0, 0.5, 2.0, -0.25][(h + b) % 5] for h in range(H)] for b in range(B)]
    Q = torch.zeros(B, H, D, dtype=torch.float64)
    for b in range(B):
        for h in range(H):
            Q[b, h, chans[b][h]] = coefs[b][h]
    wv = np.array([[(h + 1) / 8 + b / 4 for h in range(H)] for b in range(B)], np.float32)
    got = oracle.indexer(bf16_bits(Q), bf16_bits(K), wv)
    for b in range(B):
        for j in range(N):
            s = Fraction(0)
            for h in range(H):
                prod = Fraction(coefs[b][h]) * Fraction(float(K[b, j, chans[b][h]]))
                s += Fraction(float(wv[b, h])) * max(Fraction(0), prod)
            assert got[b, j] == float(s), (b, j)


def test_indexer_relu_before_weight():
    """The ReLU acts on q.k, then the weight multiplies: with a negative
    weight the score is -ReLU(q.k), never ReLU(-q.k)."""
    q = torch.zeros(1, 1, 8, dtype=torch.float64)
    q[0, 0, 2] = 1.0
    k = torch.zeros(1, 2, 8, dtype=torch.float64)
    k[0, 0, 2] = 3.0
    k[0, 1, 2] = -3.0
    w = np.array([[-0.5]], np.float32)
    got = oracle.indexer(bf16_bits(q), bf16_bits(k), w)
    assert got.tolist() == [[-1.5, 0.0]]


def test_indexer_weight_scaling_and_head_permutation():
    g = torch.Generator().manual_seed(9)
    B, N, H, D = 2, 129, 8, 128
    q = torch.randn(B, H, D, generator=g).to(torch.bfloat16)
    k = torch.randn(B, N, D, generator=g).to(torch.bfloat16)
    w = torch.rand(B, H, generator=g).numpy().astype(np.float32)
    s1 = oracle.indexer(bf16_bits(q), bf16_bits(k), w)
    s2 = oracle.indexer(bf16_bits(q), bf16_bits(k), 2 * w)
    assert np.array_equal(s2, 2 * s1)  # power-of-two scaling is exact
    perm = torch.randperm(H, generator=g)
    s3 = oracle.indexer(bf16_bits(q[:, perm]), bf16_bits(k), np.ascontiguousarray(w[:, perm]))
    assert np.all(np.abs(s3 - s1) <= np.spacing(np.abs(s1)))
    # Batch rows are independent: swapping batches swaps score rows.
    s4 = oracle.indexer(bf16_bits(q.flip(0)), bf16_bits(k.flip(0)), np.ascontiguousarray(w[::-1]))
    assert np.array_equal(s4, s1[::-1])


def test_indexer_stress_construction_is_exact():
    """The stress workload's indexer inputs reproduce its quantised score rows
    exactly (first unit vector queries, weights 1/H)."""
    s = workloads.StepShape(B=2, N=3000, H_I=64, D_I=128, k=16, W=0, H_q=16, D=128)
    inp = workloads.stress_step_inputs(s, 5000)
    got = oracle.indexer(bf16_bits(inp["q_idx"]), bf16_bits(inp["k_idx"]), inp["w"].numpy())
    assert np.array_equal(got, inp["stress_scores"].float().numpy())


# ---------------------------------------------------------------- top-k

def _rows_with_ties(g, B, N, levels):
    return (torch.randint(0, levels, (B, N), generator=g).float() - levels / 2) / 4


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_rank_definition(seed):
    g = torch.Generator().manual_seed(100 + seed)
    N = [1, 7, 64, 130, 250, 300][seed]
    k = max(1, [1, 3, 17, 64, 250, 150][seed])
    k = min(k, N)
    x = _rows_with_ties(g, 3, N, levels=[2, 3, 5, 9, 40, 1000][seed])
    # sprinkle signed zeros and infinities
    if N > 4:
        x[0, 0] = -0.0
        x[0, 1] = 0.0
        x[1, 2] = float("inf")
        x[2, 3] = float("-inf")
    got = oracle.topk(x.numpy(), k)
    for b in range(x.shape[0]):
        assert got[b].tolist() == brute.rank_select(x[b].tolist(), k)


def test_topk_bf16_input_equals_decoded_input():
    g = torch.Generator().manual_seed(3)
    x = torch.randn(4, 2000, generator=g).to(torch.bfloat16)
    a = oracle.topk(bf16_bits(x), 100)
    b = oracle.topk(x.float().numpy(), 100)
    assert np.array_equal(a, b)


def test_topk_invariants_and_torch_values():
    g = torch.Generator().manual_seed(4)
    x = torch.randn(5, 20000, generator=g).to(torch.bfloat16).float()  # many ties
    k = 333
    idx = oracle.topk(x.numpy(), k)
    for b in range(5):
        sel = idx[b]
        assert len(set(sel.tolist())) == k and sel.min() >= 0 and sel.max() < 20000
        mask = np.zeros(20000, bool)
        mask[sel] = True
        vals = x[b].numpy()
        mn = vals[mask].min()
        assert vals[~mask].max() <= mn
        # tied values at the boundary: selected ones have the smaller indices
        tied_sel = np.nonzero(mask & (vals == mn))[0]
        tied_out = np.nonzero(~mask & (vals == mn))[0]
        if tied_out.size:
            assert tied_sel.max() < tied_out.min()
        ref = torch.topk(x[b], k).values.numpy()
        assert np.array_equal(np.sort(vals[sel]), np.sort(ref))
    # the default order is value desc, index asc
    v = x[0].numpy()[idx[0]]
    assert np.all(np.diff(v) <= 0)


def test_topk_special_rows():
    N, k = 1000, 37
    rows = np.stack([
        np.full(N, 0.5, np.float32),                   # all equal
        np.arange(N, dtype=np.float32),                # ascending
        np.arange(N, 0, -1).astype(np.float32),        # descending
    ])
    idx = oracle.topk(rows, k, index_order=True)
    assert idx[0].tolist() == list(range(k))
    assert idx[1].tolist() == list(range(N - k, N))
    assert idx[2].tolist() == list(range(k))
    full = oracle.topk(rows, N, index_order=True)
    assert all(full[b].tolist() == list(range(N)) for b in range(3))


def test_topk_index_order_is_sorted_same_set():
    g = torch.Generator().manual_seed(8)
    x = torch.randn(3, 5000, generator=g)
    a = oracle.topk(x.numpy(), 200, index_order=False)
    b = oracle.topk(x.numpy(), 200, index_order=True)
    assert np.array_equal(np.sort(a, axis=1), b)


def test_topk_rejects_bad_k():
    with pytest.raises(ValueError):
        oracle.topk(np.zeros((1, 4), np.float32), 5)


# ---------------------------------------------------------------- attention

def _sdpa_ref(q, rows, scale):
    """torch scaled_dot_product_attention in fp64; q [B,Hq,D], rows [B,R,D]."""
    B, Hq, D = q.shape
    qq = q.double().unsqueeze(2)                        # [B,Hq,1,D]
    kk = rows.double().unsqueeze(1).expand(B, Hq, rows.shape[1], D)
    out = torch.nn.functional.scaled_dot_product_attention(qq, kk, kk, scale=scale)
    return out[:, :, 0, :].numpy()


def test_attend_dense_equals_sdpa():
    """k = N and W = 0 select every row: the result is dense MQA."""
    g = torch.Generator().manual_seed(21)
    B, N, Hq, D = 2, 96, 16, 128
    q = torch.randn(B, Hq, D, generator=g).to(torch.bfloat16)
    kv = torch.randn(B, N, D, generator=g).to(torch.bfloat16)
    idx = torch.stack([torch.randperm(N, generator=g) for _ in range(B)]).int()
    scale = 1 / math.sqrt(D)
    got = oracle.attend(bf16_bits(q), bf16_bits(kv), idx.numpy(), None, scale)
    ref = _sdpa_ref(q, kv, scale)
    assert np.max(np.abs(got - ref)) < 1e-12


def test_attend_sparse_with_window_equals_sdpa_on_gathered_rows():
    g = torch.Generator().manual_seed(22)
    B, N, k, W, Hq, D = 3, 200, 40, 9, 16, 128
    q = torch.randn(B, Hq, D, generator=g).to(torch.bfloat16)
    kv = torch.randn(B, N, D, generator=g).to(torch.bfloat16)
    win = torch.randn(B, W, D, generator=g).to(torch.bfloat16)
    idx = torch.stack([torch.randperm(N, generator=g)[:k] for _ in range(B)]).int()
    scale = 0.07
    got = oracle.attend(bf16_bits(q), bf16_bits(kv), idx.numpy(), bf16_bits(win), scale)
    rows = torch.cat([torch.stack([kv[b, idx[b].long()] for b in range(B)]), win], dim=1)
    ref = _sdpa_ref(q, rows, scale)
    assert np.max(np.abs(got - ref)) < 1e-12


def test_attend_closed_forms():
    g = torch.Generator().manual_seed(23)
    B, N, Hq, D = 1, 10, 16, 128
    q = torch.randn(B, Hq, D, generator=g).to(torch.bfloat16)
    kv = torch.randn(B, N, D, generator=g).to(torch.bfloat16)
    kvd = kv.double().numpy()
    # one row: the output is that row, for every head
    out = oracle.attend(bf16_bits(q), bf16_bits(kv), np.array([[6]], np.int32), None, 0.3)
    assert np.array_equal(out[0], np.broadcast_to(kvd[0, 6], (Hq, D)))
    # zero query: uniform weights, the mean of the rows
    z = torch.zeros_like(q)
    idx = np.array([[1, 4, 9]], np.int32)
    out = oracle.attend(bf16_bits(z), bf16_bits(kv), idx, None, 0.3)
    assert np.max(np.abs(out[0] - kvd[0, [1, 4, 9]].mean(0))) < 1e-15
    # two rows: logistic weights of the logit gap
    idx = np.array([[2, 5]], np.int32)
    scale = 0.11
    out = oracle.attend(bf16_bits(q), bf16_bits(kv), idx, None, scale)
    qd = q.double().numpy()[0]
    for h in range(Hq):
        z1 = scale * float(np.dot(qd[h], kvd[0, 2]))
        z2 = scale * float(np.dot(qd[h], kvd[0, 5]))
        a, b = brute.softmax_weights_two_rows(z1, z2)
        assert np.max(np.abs(out[0, h] - (a * kvd[0, 2] + b * kvd[0, 5]))) < 1e-12


def test_attend_window_rows_equal_selected_rows_and_permutation():
    g = torch.Generator().manual_seed(24)
    B, N, Hq, D = 2, 50, 16, 128
    q = torch.randn(B, Hq, D, generator=g).to(torch.bfloat16)
    kv = torch.randn(B, N, D, generator=g).to(torch.bfloat16)
    sel = torch.tensor([[3, 17, 40, 41, 8], [0, 1, 2, 49, 30]], dtype=torch.int32)
    a = oracle.attend(bf16_bits(q), bf16_bits(kv), sel.numpy(), None, 0.2)
    # the same rows handed over as the window (plus one selected row)
    win = torch.stack([kv[b, sel[b, 1:].long()] for b in range(B)])
    b_ = oracle.attend(bf16_bits(q), bf16_bits(kv), sel[:, :1].contiguous().numpy(),
                       bf16_bits(win), 0.2)
    assert np.max(np.abs(a - b_)) < 1e-13
    perm = sel[:, torch.tensor([4, 2, 0, 3, 1])].contiguous()
    c = oracle.attend(bf16_bits(q), bf16_bits(kv), perm.numpy(), None, 0.2)
    assert np.max(np.abs(a - c)) < 1e-13


def test_attend_rejects_out_of_range_index():
    q = np.zeros((1, 16, 128), np.uint16)
    kv = np.zeros((1, 4, 128), np.uint16)
    with pytest.raises(ValueError):
        oracle.attend(q, kv, np.array([[4]], np.int32), None, 1.0)


# ---------------------------------------------------------------- step

def test_step_is_the_composition():
    s = workloads.StepShape(B=2, N=300, H_I=8, D_I=128, k=20, W=5, H_q=16, D=128)
    inp = workloads.step_inputs(s, 77000)
    b = {k_: (bf16_bits(v) if v.dtype == torch.bfloat16 else v.numpy()) for k_, v in inp.items()}
    scores, idx, out = oracle.step(b["q_idx"], b["k_idx"], b["w"], b["q"], b["kv_cmp"],
                                   b["kv_win"], s.k, s.scale)
    assert np.array_equal(scores, oracle.indexer(b["q_idx"], b["k_idx"], b["w"]))
    assert np.array_equal(idx, oracle.topk(scores, s.k))
    assert np.array_equal(out, oracle.attend(b["q"], b["kv_cmp"], idx, b["kv_win"], s.scale))


def test_oracle_threads_do_not_change_results():
    g = torch.Generator().manual_seed(31)
    x = torch.randn(16, 3000, generator=g)
    oracle.set_threads(1)
    a = oracle.topk(x.numpy(), 50)
    oracle.set_threads(4)
    b = oracle.topk(x.numpy(), 50)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------- ragged rows

@pytest.mark.parametrize("seed", range(4))
def test_topk_ragged_matches_rank_definition_of_the_prefix(seed):
    """Row b's answer is the rank-definition top-k of its first lengths[b]
    scores, padded with -1; lengths 0, below k, equal to k and N occur."""
    g = torch.Generator().manual_seed(400 + seed)
    N, k = [(50, 7), (120, 30), (9, 9), (200, 64)][seed]
    x = _rows_with_ties(g, 6, N, levels=[3, 7, 2, 50][seed])
    lengths = np.array([0, 1, min(k - 1, N), k, N, N // 2], np.int32)
    for dt in ("f32", "bf16"):
        xs = x.numpy() if dt == "f32" else bf16_bits(x)
        xv = x if dt == "f32" else x.to(torch.bfloat16).float()
        got = oracle.topk_ragged(xs, lengths, k)
        got_sorted = oracle.topk_ragged(xs, lengths, k, index_order=True)
        for b in range(x.shape[0]):
            n = int(lengths[b])
            want = brute.rank_select(xv[b, :n].tolist(), min(k, n))
            assert got[b].tolist() == want + [-1] * (k - len(want))
            assert got_sorted[b].tolist() == sorted(want) + [-1] * (k - len(want))


def test_topk_ragged_full_lengths_equal_topk():
    g = torch.Generator().manual_seed(410)
    x = torch.randn(4, 3000, generator=g)
    lengths = np.full(4, 3000, np.int32)
    assert np.array_equal(oracle.topk_ragged(x.numpy(), lengths, 100), oracle.topk(x.numpy(), 100))


def test_topk_ragged_rejects_bad_lengths():
    x = np.zeros((2, 10), np.float32)
    with pytest.raises(ValueError):
        oracle.topk_ragged(x, np.array([3, 11], np.int32), 4)
    with pytest.raises(ValueError):
        oracle.topk_ragged(x, np.array([-1, 3], np.int32), 4)


def test_attend_empty_slots_equal_sdpa_on_the_remaining_rows():
    """Slots holding -1 take no part: the result is fp64 SDPA over the rows
    that remain (selected ones in slot order, then the window)."""
    g = torch.Generator().manual_seed(411)
    B, N, k, W, Hq, D = 3, 150, 20, 4, 16, 128
    q = torch.randn(B, Hq, D, generator=g).to(torch.bfloat16)
    kv = torch.randn(B, N, D, generator=g).to(torch.bfloat16)
    win = torch.randn(B, W, D, generator=g).to(torch.bfloat16)
    idx = torch.stack([torch.randperm(N, generator=g)[:k] for _ in range(B)]).int()
    idx[0, 5:] = -1          # a short row
    idx[1, ::3] = -1         # holes anywhere
    idx[2, :] = -1           # only the window remains
    got = oracle.attend(bf16_bits(q), bf16_bits(kv), idx.numpy(), bf16_bits(win), 0.05)
    for b in range(B):
        keep = idx[b][idx[b] >= 0].long()
        rows = torch.cat([kv[b, keep], win[b]], dim=0).unsqueeze(0)
        ref = _sdpa_ref(q[b:b + 1], rows, 0.05)
        assert np.max(np.abs(got[b] - ref[0])) < 1e-12


def test_attend_with_no_rows_is_zero():
    g = torch.Generator().manual_seed(412)
    q = torch.randn(2, 16, 128, generator=g).to(torch.bfloat16)
    kv = torch.randn(2, 30, 128, generator=g).to(torch.bfloat16)
    idx = np.full((2, 4), -1, np.int32)
    idx[1, 2] = 7
    out = oracle.attend(bf16_bits(q), bf16_bits(kv), idx, None, 0.1)
    assert np.all(out[0] == 0.0)
    assert np.array_equal(out[1], np.broadcast_to(kv[1, 7].double().numpy(), (16, 128)))
    with pytest.raises(ValueError):
        oracle.attend(bf16_bits(q), bf16_bits(kv), np.full((2, 4), -2, np.int32), None, 0.1)


def test_step_ragged_is_the_composition():
    s = workloads.StepShape(B=3, N=300, H_I=8, D_I=128, k=20, W=5, H_q=16, D=128)
    inp = workloads.step_inputs(s, 77100)
    b = {k_: (bf16_bits(v) if v.dtype == torch.bfloat16 else v.numpy()) for k_, v in inp.items()}
    lengths = np.array([300, 7, 0], np.int32)
    scores, idx, out = oracle.step_ragged(b["q_idx"], b["k_idx"], b["w"], b["q"], b["kv_cmp"],
                                          b["kv_win"], lengths, s.k, s.scale)
    assert np.array_equal(scores, oracle.indexer(b["q_idx"], b["k_idx"], b["w"]))
    assert np.array_equal(idx, oracle.topk_ragged(scores, lengths, s.k))
    assert np.array_equal(out, oracle.attend(b["q"], b["kv_cmp"], idx, b["kv_win"], s.scale))
    # full lengths: the ordinary step
    full = np.full(3, 300, np.int32)
    a = oracle.step_ragged(b["q_idx"], b["k_idx"], b["w"], b["q"], b["kv_cmp"], b["kv_win"],
                           full, s.k, s.scale)
    c = oracle.step(b["q_idx"], b["k_idx"], b["w"], b["q"], b["kv_cmp"], b["kv_win"], s.k, s.scale)
    assert all(np.array_equal(u, v) for u, v in zip(a, c))


# ---------------------------------------------------------------- several query tokens per row

def _mt_inputs(g, B, T, N, H, DI, Hq, D, W):
    q_idx = torch.randn(B, T, H, DI, generator=g).to(torch.bfloat16)
    k_idx = torch.randn(B, N, DI, generator=g).to(torch.bfloat16)
    w = torch.rand(B, T, H, generator=g).float()
    q = torch.randn(B, T, Hq, D, generator=g).to(torch.bfloat16)
    kv = torch.randn(B, N, D, generator=g).to(torch.bfloat16)
    win = torch.randn(B, T, W, D, generator=g).to(torch.bfloat16)
    return q_idx, k_idx, w, q, kv, win


def test_indexer_mt_equals_fp64_einsum():
    """Token t of row b scores against row b's keys: torch fp64 einsum of
    the definition, rounded to fp32, at most 1 ulp away (sum order)."""
    g = torch.Generator().manual_seed(501)
    B, T, N, H, DI = 3, 3, 97, 5, 128
    q_idx, k_idx, w, *_ = _mt_inputs(g, B, T, N, H, DI, 16, 128, 1)
    got = oracle.indexer_mt(bf16_bits(q_idx), bf16_bits(k_idx), w.numpy())
    dots = torch.einsum("bthd,bnd->btnh", q_idx.double(), k_idx.double())
    ref = (torch.relu(dots) * w.double()[:, :, None, :]).sum(-1).float().numpy()
    assert got.shape == (B, T, N)
    assert np.all(np.abs(got - ref) <= np.spacing(np.abs(ref)))
    # the keys are really shared: a token scored against another row's keys differs
    assert not np.array_equal(got[0, 0], got[1, 0])


def test_indexer_mt_token_equals_the_single_token_indexer():
    g = torch.Generator().manual_seed(502)
    B, T, N, H, DI = 2, 4, 130, 8, 128
    q_idx, k_idx, w, *_ = _mt_inputs(g, B, T, N, H, DI, 16, 128, 1)
    qb, kb, wn = bf16_bits(q_idx), bf16_bits(k_idx), w.numpy()
    got = oracle.indexer_mt(qb, kb, wn)
    for t in range(T):
        assert np.array_equal(got[:, t], oracle.indexer(qb[:, t], kb, wn[:, t]))


def test_attend_mt_equals_sdpa_per_token():
    """Each token attends over its own selection from row b's compressed
    rows (empty slots left out) and its own window: fp64 SDPA."""
    g = torch.Generator().manual_seed(503)
    B, T, N, k, W, Hq, D = 2, 3, 120, 17, 4, 16, 128
    _, _, _, q, kv, win = _mt_inputs(g, B, T, N, 4, 128, Hq, D, W)
    idx = torch.stack([torch.stack([torch.randperm(N, generator=g)[:k] for _ in range(T)])
                       for _ in range(B)]).int()
    idx[0, 1, 6:] = -1
    idx[1, 2, ::2] = -1
    got = oracle.attend_mt(bf16_bits(q), bf16_bits(kv), idx.numpy(), bf16_bits(win), 0.06)
    assert got.shape == (B, T, Hq, D)
    for b in range(B):
        for t in range(T):
            keep = idx[b, t][idx[b, t] >= 0].long()
            rows = torch.cat([kv[b, keep], win[b, t]], dim=0).unsqueeze(0)
            ref = _sdpa_ref(q[b, t].unsqueeze(0), rows, 0.06)
            assert np.max(np.abs(got[b, t] - ref[0])) < 1e-12


def test_step_mt_is_the_composition_and_tokens_are_independent():
    g = torch.Generator().manual_seed(504)
    B, T, N, H, DI, k, W, Hq, D = 2, 3, 260, 8, 128, 19, 5, 16, 128
    q_idx, k_idx, w, q, kv, win = _mt_inputs(g, B, T, N, H, DI, Hq, D, W)
    a = [bf16_bits(q_idx), bf16_bits(k_idx), w.numpy(), bf16_bits(q), bf16_bits(kv),
         bf16_bits(win)]
    lengths = np.array([[260, 40, 3], [0, 19, 200]], np.int32)
    scores, idx, out = oracle.step_mt(*a, lengths, k, 0.08)
    assert np.array_equal(scores, oracle.indexer_mt(a[0], a[1], a[2]))
    flat = oracle.topk_ragged(scores.reshape(B * T, N), lengths.reshape(-1), k)
    assert np.array_equal(idx, flat.reshape(B, T, k))
    assert np.array_equal(out, oracle.attend_mt(a[3], a[4], idx, a[5], 0.08))
    # no lengths: every token sees all N positions
    s2, i2, o2 = oracle.step_mt(*a, None, k, 0.08)
    assert np.array_equal(i2, oracle.topk(s2.reshape(B * T, N), k).reshape(B, T, k))
    # changing token 1's own inputs leaves tokens 0 and 2 as they were
    a2 = [x.copy() for x in a]
    a2[0][:, 1] = a2[0][:, 1][:, ::-1]
    a2[3][:, 1] = 0
    a2[5][:, 1] = a2[5][:, 0]
    s3, i3, o3 = oracle.step_mt(*a2, lengths, k, 0.08)
    for t in (0, 2):
        assert np.array_equal(s3[:, t], scores[:, t]) and np.array_equal(i3[:, t], idx[:, t])
        assert np.array_equal(o3[:, t], out[:, t])
    assert not np.array_equal(o3[:, 1], out[:, 1])


def test_step_mt_with_one_token_is_the_step():
    s = workloads.StepShape(B=3, N=300, H_I=8, D_I=128, k=20, W=5, H_q=16, D=128)
    inp = workloads.step_inputs(s, 77200)
    b = {k_: (bf16_bits(v) if v.dtype == torch.bfloat16 else v.numpy()) for k_, v in inp.items()}
    one = oracle.step_mt(b["q_idx"][:, None], b["k_idx"], b["w"][:, None], b["q"][:, None],
                         b["kv_cmp"], b["kv_win"][:, None], None, s.k, s.scale)
    ref = oracle.step(b["q_idx"], b["k_idx"], b["w"], b["q"], b["kv_cmp"], b["kv_win"], s.k,
                      s.scale)
    assert all(np.array_equal(u[:, 0], v) for u, v in zip(one, ref))
    lengths = np.array([300, 7, 0], np.int32)
    one = oracle.step_mt(b["q_idx"][:, None], b["k_idx"], b["w"][:, None], b["q"][:, None],
                         b["kv_cmp"], b["kv_win"][:, None], lengths[:, None], s.k, s.scale)
    ref = oracle.step_ragged(b["q_idx"], b["k_idx"], b["w"], b["q"], b["kv_cmp"], b["kv_win"],
                             lengths, s.k, s.scale)
    assert all(np.array_equal(u[:, 0], v) for u, v in zip(one, ref))


# ---------------------------------------------------------------- indexer query projection

def test_qproj_equals_fp64_matmul():
    g = torch.Generator().manual_seed(601)
    B, d_in, O = 5, 1000, 300
    x = torch.randn(B, d_in, generator=g).to(torch.bfloat16)
    w = torch.randn(O, d_in, generator=g).to(torch.bfloat16)
    got = oracle.qproj(bf16_bits(x), bf16_bits(w))
    ref = (x.double() @ w.double().T).numpy()
    assert got.shape == (B, O)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_qproj_one_hot_and_scaling_are_exact():
    g = torch.Generator().manual_seed(602)
    B, d_in, O = 3, 256, 64
    w = torch.randn(O, d_in, generator=g).to(torch.bfloat16)
    x = torch.zeros(B, d_in)
    picks = [0, 77, 255]
    for b, i in enumerate(picks):
        x[b, i] = 1.0
    got = oracle.qproj(bf16_bits(x.to(torch.bfloat16)), bf16_bits(w))
    for b, i in enumerate(picks):
        assert np.array_equal(got[b], w[:, i].double().numpy())  # selects a column of w
    xs = torch.randn(B, d_in, generator=g).to(torch.bfloat16)
    a = oracle.qproj(bf16_bits(xs), bf16_bits(w))
    b2 = oracle.qproj(bf16_bits((xs.float() * 2).to(torch.bfloat16)), bf16_bits(w))
    assert np.array_equal(b2, 2 * a)  # exact: powers of two scale every product exactly


# ---------------------------------------------------------------- attention sink

def _sink_inputs(seed, B=2, N=60, k=12, W=5, Hq=16, D=128):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Hq, D, generator=g).to(torch.bfloat16)
    kv = torch.randn(B, N, D, generator=g).to(torch.bfloat16)
    win = torch.randn(B, W, D, generator=g).to(torch.bfloat16)
    idx = torch.stack([torch.randperm(N, generator=g)[:k] for _ in range(B)]).int()
    return q, kv, win, idx


def test_attend_sink_of_minus_infinity_is_plain_attention():
    q, kv, win, idx = _sink_inputs(41)
    Hq = q.shape[1]
    a = oracle.attend(bf16_bits(q), bf16_bits(kv), idx.numpy(), bf16_bits(win), 0.09)
    b = oracle.attend(bf16_bits(q), bf16_bits(kv), idx.numpy(), bf16_bits(win), 0.09,
                      sink=np.full(Hq, -np.inf))
    assert np.array_equal(a, b)


def test_attend_sink_equals_sdpa_with_a_zero_value_row():
    """A sink is a row whose value vector is zero and whose logit is the sink:
    torch's scaled_dot_product_attention over the gathered rows plus one zero
    key/value row, with the sink added to that row's logit as a float mask,
    per head."""
    q, kv, win, idx = _sink_inputs(42)
    B, Hq, D = q.shape
    sink = np.linspace(-3.0, 4.0, Hq)
    scale = 0.08
    got = oracle.attend(bf16_bits(q), bf16_bits(kv), idx.numpy(), bf16_bits(win), scale,
                        sink=sink)
    rows = torch.cat([torch.stack([kv[b, idx[b].long()] for b in range(B)]), win], dim=1).double()
    rows = torch.cat([rows, torch.zeros(B, 1, D, dtype=torch.float64)], dim=1)   # zero row
    R = rows.shape[1]
    mask = torch.zeros(B, Hq, 1, R, dtype=torch.float64)
    mask[:, :, 0, R - 1] = torch.from_numpy(sink)
    kk = rows.unsqueeze(1).expand(B, Hq, R, D)
    ref = torch.nn.functional.scaled_dot_product_attention(q.double().unsqueeze(2), kk, kk,
                                                           attn_mask=mask, scale=scale)
    assert np.max(np.abs(got - ref[:, :, 0, :].numpy())) < 1e-12
    # the sink changes the result (it is not ignored)
    plain = oracle.attend(bf16_bits(q), bf16_bits(kv), idx.numpy(), bf16_bits(win), scale)
    assert np.max(np.abs(got - plain)) > 1e-3


def test_attend_sink_closed_forms():
    g = torch.Generator().manual_seed(43)
    Hq, D = 16, 128
    q = torch.randn(1, Hq, D, generator=g).to(torch.bfloat16)
    kv = torch.randn(1, 8, D, generator=g).to(torch.bfloat16)
    kvd = kv.double().numpy()[0]
    qd = q.double().numpy()[0]
    sink = np.linspace(-2.0, 2.0, Hq)
    scale = 0.1
    # one row: out = sigma(z - sink) * row
    out = oracle.attend(bf16_bits(q), bf16_bits(kv), np.array([[3]], np.int32), None, scale,
                        sink=sink)[0]
    for h in range(Hq):
        z = scale * float(np.dot(qd[h], kvd[3]))
        a, _ = brute.softmax_weights_two_rows(z, sink[h])
        assert np.max(np.abs(out[h] - a * kvd[3])) < 1e-13
    # a batch row with no rows at all still outputs zeros
    out = oracle.attend(bf16_bits(q), bf16_bits(kv), np.array([[-1, -1]], np.int32), None,
                        scale, sink=sink)
    assert np.array_equal(out, np.zeros_like(out))


# ---------------------------------------------------------------- compressor

def _compress_ref(x_bits: np.ndarray, wg: np.ndarray) -> np.ndarray:
    """The compressor written with torch in fp64: gate scores, softmax over
    each group's 4 rows, weighted sum."""
    x = torch.from_numpy(x_bits.view(np.int16).copy()).view(torch.bfloat16).double()
    B, R, D = x.shape
    xg = x.view(B, R // 4, 4, D)
    z = torch.matmul(xg, torch.from_numpy(wg.astype(np.float64)))          # [B, G, 4]
    a = torch.softmax(z, dim=-1)
    return (a.unsqueeze(-1) * xg).sum(2).numpy()


def test_compress_equals_torch_softmax_gate():
    g = torch.Generator().manual_seed(51)
    B, G, D = 3, 5, 128
    x = torch.randn(B, 4 * G, D, generator=g).to(torch.bfloat16)
    wg = (torch.randn(D, generator=g) / math.sqrt(D)).float().numpy()
    got = oracle.compress(bf16_bits(x), wg)
    ref = _compress_ref(bf16_bits(x), wg)
    assert np.max(np.abs(got - ref)) < 1e-12
    # the weights differ from uniform: the result is not the plain mean
    mean = x.double().view(B, G, 4, D).mean(2).numpy()
    assert np.max(np.abs(got - mean)) > 1e-2


def test_compress_closed_forms():
    g = torch.Generator().manual_seed(52)
    B, G, D = 2, 3, 64
    x = torch.randn(B, 4 * G, D, generator=g).to(torch.bfloat16)
    xd = x.double().view(B, G, 4, D).numpy()
    # zero gate: equal weights, the mean of each group's rows
    got = oracle.compress(bf16_bits(x), np.zeros(D, np.float32))
    assert np.max(np.abs(got - xd.mean(2))) < 1e-15
    # a gate that only row 1 of every group passes strongly: that row exactly
    y = x.clone().view(B, G, 4, D)
    y[:, :, :, 0] = 0.0
    y[:, :, 1, 0] = 1000.0                       # exact in bf16
    wg = np.zeros(D, np.float32)
    wg[0] = 1.0
    got = oracle.compress(bf16_bits(y.view(B, 4 * G, D)), wg)
    assert np.array_equal(got, y.double()[:, :, 1, :].numpy())
    # two rows left in the race: logistic weights of their gate gap
    y = x.clone().view(B, G, 4, D)
    y[:, :, 2:, 0] = -1000.0                     # rows 2 and 3 get weight exp(-1000 - ...) = 0
    y[:, :, :2, 0] = torch.tensor([0.5, -0.25], dtype=torch.bfloat16)
    wg = np.zeros(D, np.float32)
    wg[0] = 1.0
    got = oracle.compress(bf16_bits(y.view(B, 4 * G, D)), wg)
    yd = y.double().numpy()
    a, b = brute.softmax_weights_two_rows(0.5, -0.25)
    ref = a * yd[:, :, 0, :] + b * yd[:, :, 1, :]
    assert np.max(np.abs(got - ref)) < 1e-15


def test_compress_row_order_and_group_locality():
    g = torch.Generator().manual_seed(53)
    B, G, D = 2, 4, 128
    x = torch.randn(B, 4 * G, D, generator=g).to(torch.bfloat16)
    wg = torch.randn(D, generator=g).float().numpy() / 8
    base = oracle.compress(bf16_bits(x), wg)
    # the rows of a group may come in any order
    perm = torch.tensor([2, 0, 3, 1])
    xp = x.view(B, G, 4, D)[:, :, perm, :].reshape(B, 4 * G, D)
    assert np.max(np.abs(oracle.compress(bf16_bits(xp), wg) - base)) < 1e-14
    # changing group 2 leaves the other groups alone
    y = x.clone()
    y[:, 8:12] = torch.randn(B, 4, D, generator=g).to(torch.bfloat16)
    got = oracle.compress(bf16_bits(y), wg)
    assert np.array_equal(got[:, [0, 1, 3]], base[:, [0, 1, 3]])
    assert np.max(np.abs(got[:, 2] - base[:, 2])) > 1e-3


def test_compress_rejects_an_incomplete_group():
    with pytest.raises(ValueError):
        oracle.compress(np.zeros((1, 6, 16), np.uint16), np.zeros(16, np.float32))
