"""The hand-derived worked example in tests/golden/worked_example.json (its
derivation is written out in the file), checked on the CPU oracle and, zero-
padded to the shapes the kernels take, on the GPU path through the C ABI."""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

HERE = os.path.dirname(os.path.abspath(__file__))
G = json.load(open(os.path.join(HERE, "golden", "worked_example.json")))


def bits(a) -> np.ndarray:
    return workloads.bits16(torch.tensor(a, dtype=torch.float32).to(torch.bfloat16))


def test_indexer_worked_example():
    e = G["indexer"]
    s = oracle.indexer(bits(e["q_idx"]), bits(e["k_idx"]), np.array(e["w"], np.float32))
    assert np.array_equal(s, np.array(e["scores"], np.float32))


def test_topk_worked_example():
    e = G["topk"]
    row = np.array(e["scores"], np.float32)
    assert np.array_equal(oracle.topk(row, e["k"], index_order=True), np.array(e["selected_ascending"]))
    assert np.array_equal(oracle.topk(row, e["k_tie"], index_order=True),
                          np.array(e["selected_tie_ascending"]))


def test_attention_worked_example():
    e = G["attention"]
    rows = bits(e["rows"])
    out = oracle.attend(bits(e["q"]), rows, np.array([[0, 1]], np.int32), None, float(np.float32(math.log(3))))
    assert np.allclose(out, np.array(e["out"]), rtol=0, atol=1e-7)


# ---------------------------------------------------------------- GPU path

def _padded(a, dim):
    """[..., d] float list -> torch float32 with the last dim zero-padded."""
    t = torch.tensor(a, dtype=torch.float32)
    pad = torch.zeros(t.shape[:-1] + (dim - t.shape[-1],))
    return torch.cat([t, pad], dim=-1)


@pytest.mark.gpu
def test_gpu_worked_example():
    import indexer_top_gathered_amd as dsa
    dev = "cuda"
    e = G["indexer"]
    q_idx = _padded(e["q_idx"], 128).to(torch.bfloat16).to(dev)
    k_idx = _padded(e["k_idx"], 128).to(torch.bfloat16).to(dev)
    w = torch.tensor(e["w"], dtype=torch.float32, device=dev)
    s = dsa.dsa_indexer_score(q_idx, k_idx, w)
    torch.cuda.synchronize()
    assert torch.equal(s.cpu(), torch.tensor(e["scores"], dtype=torch.float32))

    t = G["topk"]
    row = torch.tensor(t["scores"], dtype=torch.float32, device=dev)
    for k, key in ((t["k"], "selected_ascending"), (t["k_tie"], "selected_tie_ascending")):
        idx = dsa.dsa_topk(row, k, sorted_index=True)
        torch.cuda.synchronize()
        assert idx.cpu().tolist() == t[key]

    a = G["attention"]
    q = _padded(a["q"], 128).repeat(1, 16, 1).to(torch.bfloat16).to(dev)    # 16 identical heads
    kv = _padded(a["rows"], 128).to(torch.bfloat16).to(dev)
    idx = torch.tensor([[0, 1]], dtype=torch.int32, device=dev)
    out = dsa.dsa_sparse_attend(q, kv, idx, None, float(np.float32(math.log(3))))
    torch.cuda.synchronize()
    want = _padded(a["out"], 128).repeat(1, 16, 1)
    assert torch.allclose(out.float().cpu(), want, rtol=0, atol=2 ** -9)
