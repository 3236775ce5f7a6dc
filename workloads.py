"""Seeded synthetic inputs for the sparse-attention decode step.

This module only draws random tensors with the shapes and value
distributions of the five workloads; it holds none of the method's
arithmetic. Both the GPU tests and the CPU oracle consume what it returns,
and the benchmark times the GPU library on the same tensors.

Workload shapes follow the pages: the indexer/top-k/attention shapes of
"feat: Add DeepSeek-V4 CSA attention kernels" (sections "How the algorithm
works" and "Launching a full block": 1024 selected rows, a 128-row window,
128 indexer channels, 128 query heads) and the two top-k scenarios of the
"DeepSelect" project page (bf16 indexer rows with k=512; float32 sampling
logits over a 129280-entry vocabulary).

Seeds: tensor t of workload c is drawn from a generator seeded with
1000*c + t (t: 0 q_idx, 1 k_idx, 2 w, 3 q, 4 kv_cmp, 5 kv_win, 6 score
rows, 7 boost positions, 8 stress levels). bf16 tensors are drawn in float32
and rounded to nearest even by torch's conversion.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np
import torch


@dataclass(frozen=True)
class StepShape:
    """One decode step: batch B, compressed length N, indexer heads H_I of dim
    D_I, top-k k, window W, query heads H_q, KV dim D (one KV head, K = V)."""
    B: int
    N: int
    H_I: int
    D_I: int
    k: int
    W: int
    H_q: int
    D: int

    @property
    def scale(self) -> float:
        # 1/sqrt(D) rounded to float32, the value the kernels receive.
        return float(torch.tensor(1.0 / math.sqrt(self.D), dtype=torch.float32))


@dataclass(frozen=True)
class TopkShape:
    """Top-k only: B rows of N scores, keep k; dtype 'bf16' or 'f32'."""
    B: int
    N: int
    k: int
    dtype: str
    values: bool
    sorted_index: bool


# The five workloads.
C1 = StepShape(B=1, N=4096, H_I=8, D_I=128, k=256, W=64, H_q=16, D=128)
C2 = TopkShape(B=64, N=131072, k=512, dtype="bf16", values=False, sorted_index=False)
C3 = TopkShape(B=128, N=129280, k=1024, dtype="f32", values=True, sorted_index=False)
C4 = StepShape(B=16, N=32768, H_I=64, D_I=128, k=1024, W=128, H_q=128, D=512)
C5 = StepShape(B=64, N=262144, H_I=64, D_I=128, k=2048, W=128, H_q=128, D=512)
C5_TOPK = TopkShape(B=64, N=262144, k=2048, dtype="bf16", values=False, sorted_index=False)

WORKLOADS = {"c1": C1, "c2": C2, "c3": C3, "c4": C4, "c5": C5}


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _normal(shape, g, device, dtype, std: float = 1.0, chunk_elems: int = 1 << 28):
    """Standard normal draws (times std) in float32, converted to dtype.
    Large tensors are drawn in chunks along dim 0 to bound the float32 peak."""
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(shape[0], -1)
    per_row = flat.shape[1]
    rows = max(1, chunk_elems // max(1, per_row))
    for r0 in range(0, shape[0], rows):
        r1 = min(shape[0], r0 + rows)
        x = torch.randn((r1 - r0, per_row), generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        flat[r0:r1].copy_(x)
        del x
    return out


def step_inputs(s: StepShape, seed_base: int, device="cpu") -> dict:
    """Inputs of a decode step. q_idx, k_idx, q, kv_cmp, kv_win ~ N(0,1) bf16;
    w ~ U(0,1) float32."""
    sb = seed_base
    out = {
        "q_idx": _normal((s.B, s.H_I, s.D_I), _gen(device, sb + 0), device, torch.bfloat16),
        "k_idx": _normal((s.B, s.N, s.D_I), _gen(device, sb + 1), device, torch.bfloat16),
        "w": torch.rand((s.B, s.H_I), generator=_gen(device, sb + 2), device=device,
                        dtype=torch.float32),
        "q": _normal((s.B, s.H_q, s.D), _gen(device, sb + 3), device, torch.bfloat16),
        "kv_cmp": _normal((s.B, s.N, s.D), _gen(device, sb + 4), device, torch.bfloat16),
        "kv_win": _normal((s.B, s.W, s.D), _gen(device, sb + 5), device, torch.bfloat16),
    }
    return out


def mt_step_inputs(s: StepShape, T: int, seed_base: int, device="cpu") -> dict:
    """Inputs of a step with T query tokens per batch row: the keys (k_idx,
    kv_cmp) per row as step_inputs, the per-token tensors with a token axis
    after the batch axis (q_idx [B,T,H_I,D_I], w [B,T,H_I], q [B,T,H_q,D],
    kv_win [B,T,W,D]); same distributions as step_inputs."""
    sb = seed_base
    return {
        "q_idx": _normal((s.B, T, s.H_I, s.D_I), _gen(device, sb + 0), device, torch.bfloat16),
        "k_idx": _normal((s.B, s.N, s.D_I), _gen(device, sb + 1), device, torch.bfloat16),
        "w": torch.rand((s.B, T, s.H_I), generator=_gen(device, sb + 2), device=device,
                        dtype=torch.float32),
        "q": _normal((s.B, T, s.H_q, s.D), _gen(device, sb + 3), device, torch.bfloat16),
        "kv_cmp": _normal((s.B, s.N, s.D), _gen(device, sb + 4), device, torch.bfloat16),
        "kv_win": _normal((s.B, T, s.W, s.D), _gen(device, sb + 5), device, torch.bfloat16),
    }


def qproj_inputs(B: int, d_in: int, H_I: int, seed: int, device="cpu") -> dict:
    """Inputs of the indexer query projection: x ~ N(0,1) bf16 [B, d_in] and
    synthetic weights w_q ~ N(0, 1/d_in) bf16 [H_I*128, d_in] (unit-variance
    outputs)."""
    return {
        "x": _normal((B, d_in), _gen(device, seed + 0), device, torch.bfloat16),
        "w_q": _normal((H_I * 128, d_in), _gen(device, seed + 1), device, torch.bfloat16,
                       std=1.0 / math.sqrt(d_in)),
    }


def ragged_lengths(B: int, N: int, k: int, seed: int) -> np.ndarray:
    """int32 [B] sequence lengths for a ragged batch: the edge values 0, 1,
    k - 1, k, k + 1 and N first (those within [0, N]), then lengths drawn
    log-uniformly from [1, N], so short and long sequences mix."""
    edges = [v for v in (0, 1, k - 1, k, k + 1, N) if 0 <= v <= N]
    rng = np.random.default_rng(seed)
    rest = np.exp(rng.uniform(0.0, np.log(N), size=max(B - len(edges), 0)))
    out = np.array(edges[:B] + [int(min(N, max(1, round(x)))) for x in rest], dtype=np.int32)
    return out[:B]


def serving_lengths(B: int, N: int, seed: int) -> np.ndarray:
    """int32 [B] sequence lengths of a serving batch: uniform on [1, N]."""
    rng = np.random.default_rng(seed)
    return rng.integers(1, N + 1, size=B).astype(np.int32)


def normal_rows(B: int, N: int, dtype: str, seed: int, device="cpu", std: float = 1.0):
    """i.i.d. N(0, std^2) score rows (the indexer-shaped top-k workload)."""
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return _normal((B, N), _gen(device, seed), device, dt, std=std)


def sampling_rows(B: int, N: int, seed: int, device="cpu", boosted: int = 32,
                  boost: float = 8.0, std: float = 2.0):
    """float32 logits std*N(0,1) with `boosted` distinct positions per row
    (uniform, without replacement) raised by `boost` (the sampling workload)."""
    x = _normal((B, N), _gen(device, seed), device, torch.float32, std=std)
    g = _gen(device, seed + 1)
    # A random permutation's first entries are distinct uniform positions.
    keys = torch.rand((B, N), generator=g, device=device)
    pos = keys.argsort(dim=1)[:, :boosted]
    x.scatter_add_(1, pos, torch.full((B, boosted), boost, device=device))
    return x


def stress_levels(B: int, N: int, seed: int, device="cpu", dtype: str = "bf16"):
    """Scores quantised to 256 levels with heavy ties, odd rows sorted
    ascending: x ~ N(0,1), level = clamp(floor((x+4)*32), 0, 255),
    score = level/32 (exact in bf16 and float32)."""
    x = _normal((B, N), _gen(device, seed), device, torch.float32)
    lev = torch.clamp(torch.floor((x + 4.0) * 32.0), 0, 255)
    del x
    sc = lev / 32.0
    del lev
    odd = torch.arange(1, B, 2, device=device)
    if odd.numel():
        sc[odd] = torch.sort(sc[odd], dim=1).values
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return sc.to(dt)


def stress_step_inputs(s: StepShape, seed_base: int, device="cpu") -> dict:
    """Step inputs whose indexer scores equal the stress rows exactly:
    q_idx[b,h,:] is the first unit vector, w[b,h] = 1/H_I, k_idx[b,j,0] is
    the stress score and the other channels are N(0,1). Attention inputs are
    N(0,1) as in step_inputs."""
    base = step_inputs(replace(s, N=1), seed_base, device)  # q, kv_win, tiny rest
    sc = stress_levels(s.B, s.N, seed_base + 8, device, dtype="bf16")
    k_idx = _normal((s.B, s.N, s.D_I), _gen(device, seed_base + 1), device, torch.bfloat16)
    k_idx[:, :, 0] = sc
    q_idx = torch.zeros((s.B, s.H_I, s.D_I), dtype=torch.bfloat16, device=device)
    q_idx[:, :, 0] = 1.0
    w = torch.full((s.B, s.H_I), 1.0 / s.H_I, dtype=torch.float32, device=device)
    return {
        "q_idx": q_idx,
        "k_idx": k_idx,
        "w": w,
        "q": base["q"],
        "kv_cmp": _normal((s.B, s.N, s.D), _gen(device, seed_base + 4), device, torch.bfloat16),
        "kv_win": base["kv_win"],
        "stress_scores": sc,
    }


def bits16(t: torch.Tensor):
    """bf16 tensor -> numpy uint16 bit patterns (on the host)."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view("uint16")
