"""Comparison rules shared by the GPU parity tests.

- Top-k on an identical score row: the index set (and the values, when
  returned) equals the oracle's exactly; with sorted_index the order too.
- Indexer scores: |s_gpu - s_ref| <= 2 (D_I + H_I + 2) 2^-24 sum_h w_h
  sum_d |q_hd k_jd| + 2^-149, the classical forward-error bound of a float32
  dot product and sum (Higham, Accuracy and Stability of Numerical
  Algorithms, section 3.1) with a factor 2 of slack; the products are exact.
- End-to-end index sets: every position in the symmetric difference has an
  oracle score within 1e-3 relative of the oracle's k-th score tau (when tau
  is 0, relative to the row maximum instead).
- Attention: max|out - ref| <= 1e-2 max|ref| + 1e-3 over the whole output,
  ref computed by the oracle on the index set the GPU used.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import workloads


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy: bf16 as uint16 bits, others as is."""
    if t.dtype == torch.bfloat16:
        return workloads.bits16(t)
    return t.detach().cpu().numpy()


def assert_topk_equal(gpu_idx: np.ndarray, ref_idx: np.ndarray, sorted_index: bool, where=""):
    assert gpu_idx.shape == ref_idx.shape, where
    if sorted_index:
        ref_sorted = np.sort(ref_idx, axis=1)
        bad = np.nonzero(np.any(gpu_idx != ref_sorted, axis=1))[0]
    else:
        bad = np.nonzero(np.any(np.sort(gpu_idx, axis=1) != np.sort(ref_idx, axis=1), axis=1))[0]
    assert bad.size == 0, f"{where}: top-k mismatch in rows {bad[:8].tolist()}"


def assert_values_are_copies(gpu_val: torch.Tensor, scores: torch.Tensor, gpu_idx: torch.Tensor,
                             where=""):
    ref = torch.gather(scores, 1, gpu_idx.long())
    a = gpu_val.contiguous().view(torch.int16 if gpu_val.dtype == torch.bfloat16 else torch.int32)
    b = ref.contiguous().view(torch.int16 if ref.dtype == torch.bfloat16 else torch.int32)
    assert torch.equal(a, b), f"{where}: values are not bit copies"


def indexer_bound(q_bits, k_bits, w) -> np.ndarray:
    """Right-hand side of the indexer error bound, float64 [B,N]."""
    q = torch.from_numpy(q_bits.view(np.int16)).view(torch.bfloat16).double().abs()
    k = torch.from_numpy(k_bits.view(np.int16)).view(torch.bfloat16).double().abs()
    B, H, DI = q.shape
    mag = torch.bmm(k, q.transpose(1, 2).contiguous())            # [B,N,H] sum_d |q k|
    mag = (mag * torch.from_numpy(np.abs(w)).double()[:, None, :]).sum(-1)
    return (2.0 * (DI + H + 2) * 2.0 ** -24 * mag + 2.0 ** -149).numpy()


def assert_scores_close(gpu: np.ndarray, ref: np.ndarray, bound: np.ndarray, where=""):
    err = np.abs(gpu.astype(np.float64) - ref.astype(np.float64))
    bad = err > bound
    assert not bad.any(), (f"{where}: {bad.sum()} scores outside the bound, worst excess "
                           f"{(err - bound).max():.3e}")


def assert_index_sets_close(gpu_idx: np.ndarray, ref_scores: np.ndarray, ref_idx: np.ndarray,
                            where=""):
    B, k = ref_idx.shape
    for b in range(B):
        g = gpu_idx[b]
        assert len(np.unique(g)) == k and g.min() >= 0 and g.max() < ref_scores.shape[1], \
            f"{where}: row {b} is not k distinct in-range indices"
        tau = float(ref_scores[b, ref_idx[b, -1]])
        scale = abs(tau) if tau != 0 else float(np.max(ref_scores[b]))
        diff = np.setxor1d(g, ref_idx[b])
        if diff.size:
            dev = np.abs(ref_scores[b, diff].astype(np.float64) - tau)
            assert np.all(dev <= 1e-3 * scale), \
                f"{where}: row {b}: {int((dev > 1e-3 * scale).sum())} positions beyond the near-tie band"


def assert_attention_close(gpu_out: torch.Tensor, ref: np.ndarray, where=""):
    got = gpu_out.float().cpu().numpy().astype(np.float64)
    err = float(np.max(np.abs(got - ref)))
    lim = 1e-2 * float(np.max(np.abs(ref))) + 1e-3
    assert err <= lim, f"{where}: attention max|diff| {err:.3e} > {lim:.3e}"
    return err
