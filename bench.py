#!/usr/bin/env python3
"""Benchmark of the sparse-attention decode step on one MI355X.

A step is one pass of the whole hot path: indexer scoring, top-k, gather of
the selected rows plus the window, and sparse multi-query attention, run by
dsa_decode_step on the production decode shape (B=16, N=32768 compressed
positions, 64 indexer heads of 128 channels, k=1024, a 128-row window, 128
query heads, one K=V head of 512). Inputs are seeded synthetic tensors that
are already resident in device memory; the timed loop rotates over enough
input copies (> 1 GB) that each step reads its inputs from HBM rather than
the 256 MB Infinity Cache.

Printed: one JSON line. `value` is the step's effective bandwidth (its
compulsory bytes - every input read once, the output written once - divided
by the time per step), `us_per_step` the time per step. `roofline` is the
whole step against its own roofline (bytes at 8 TB/s; `frac_of_step_roofline`
is that time over the measured one), with `kernels`: each stage timed alone
with HIP events on the stream it runs on, in the step's launch configuration
(the indexer alone, the fused indexer + top-k, attention + combine), each
with its algorithmic bytes, flops, achieved rate and fraction of its own
roofline; `traffic` fields carry HBM bytes per call from the rocprofv3
FETCH_SIZE/WRITE_SIZE summary under profiles/ when it was taken on the
current sources (else null). `measured_hbm` holds the rates of a plain torch
row reduction and copy on 1 GiB. `graph` replays the step from one HIP
graph. `single_call_latency` is the median, p10 and p90 of single steps each
run after a 512 MiB cache-evicting write, `torch_step` the same step written
with plain torch ops on this GPU (context), `topk` the top-k-only workload
(bf16 64 x 131072, k=512) with its fraction of the HBM roofline, and
`cpu_baseline` the CPU oracle timed on this host over a bounded sample.
Every timed output is checked: the last step's indices are k distinct
in-range positions per row and both outputs equal an untimed call's.

`--workload` times one of the other workloads instead (for profiling; one
JSON line of its own, no CPU baseline): `tiny-step` (B=1, N=4096; also
replayed from one HIP graph holding a step per input copy),
`topk-sampling` (float32 128 x 129280, k=1024, values), `topk-stress`
(quantised rows, half sorted, 64 x 262144, k=2048, bf16 and float32) or
`stress-step` (B=64, N=262144, k=2048, scores equal to the stress rows) or
`ragged-step` (the production shape over rows of lengths uniform on [1, N],
timed with dsa_decode_step_ragged next to the same call at full length) or
`mtp-step` (the production shape with 2 query tokens per batch row sharing
its keys, dsa_decode_step_mt, next to 1 and 4 tokens), `qproj` (the
indexer query projection of 16 rows, 4096 wide, onto 64 x 128 channels) or
`context-sweep` (the production step at N = 2K .. 32K compressed positions,
8K .. 128K tokens at 4:1), `compress` (the 4-to-1 compressor at D = 512,
one group and 1024 groups per batch row) or `sink-step` (the production
step with a per-head attention sink, dsa_decode_step_sink, next to the same
inputs without one).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "top-k effective HBM GB/s; fused decode-step µs at B=16, N=32K, k=1024"


def parse():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--copies", type=int, default=8, help="rotating input copies")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-topk", action="store_true")
    p.add_argument("--latency-calls", type=int, default=100,
                   help="single-call latency samples, each after a cache-evicting write "
                        "(0 to skip)")
    p.add_argument("--calibrate-copy-mib", type=int, default=0,
                   help="also run one device copy of this many MiB (for counter calibration)")
    p.add_argument("--workload", default="step",
                   choices=["step", "tiny-step", "topk-sampling", "topk-stress", "stress-step",
                            "ragged-step", "mtp-step", "qproj", "context-sweep", "compress",
                            "sink-step"])
    return p.parse_args()


def step_bytes(s) -> int:
    """Compulsory bytes of one decode step: every input read once, the
    output written once (intermediate scores and indices excluded)."""
    b = s.B
    return (b * s.H_I * s.D_I * 2 + b * s.N * s.D_I * 2 + b * s.H_I * 4      # indexer inputs
            + b * s.H_q * s.D * 2                                            # q
            + b * (s.k + s.W) * s.D * 2                                      # gathered rows + window
            + b * s.H_q * s.D * 2)                                           # output


def step_roofline_us(s) -> float:
    """Serial stages, each at the larger of its HBM time (compulsory bytes at
    8 TB/s) and its MFMA time (bf16 flops at 2.5 PFLOP/s)."""
    b = s.B
    is_bytes = b * s.H_I * s.D_I * 2 + b * s.N * s.D_I * 2 + b * s.H_I * 4
    is_flops = 2 * b * s.N * s.H_I * s.D_I
    sa_bytes = step_bytes(s) - is_bytes
    sa_flops = 4 * b * s.H_q * (s.k + s.W) * s.D
    peak_flops = 2.5e15
    return 1e6 * (max(is_bytes / (HBM_PEAK_GBPS * 1e9), is_flops / peak_flops)
                  + max(sa_bytes / (HBM_PEAK_GBPS * 1e9), sa_flops / peak_flops))


def ragged_step_bytes(s, lengths) -> int:
    """Compulsory bytes of a ragged decode step: as step_bytes with row b's
    N keys replaced by its lengths[b] valid ones and its k gathered rows by
    min(k, lengths[b])."""
    total = 0
    for n in (int(x) for x in lengths):
        total += (s.H_I * s.D_I * 2 + n * s.D_I * 2 + s.H_I * 4 + s.H_q * s.D * 2
                  + (min(s.k, n) + s.W) * s.D * 2 + s.H_q * s.D * 2)
    return total


def ragged_step_roofline_us(s, lengths) -> float:
    """step_roofline_us over the valid keys and gathered rows only."""
    n_sum = sum(int(x) for x in lengths)
    g_sum = sum(min(s.k, int(x)) for x in lengths)
    b = s.B
    is_bytes = b * s.H_I * s.D_I * 2 + n_sum * s.D_I * 2 + b * s.H_I * 4
    is_flops = 2 * n_sum * s.H_I * s.D_I
    sa_bytes = ragged_step_bytes(s, lengths) - is_bytes
    sa_flops = 4 * s.H_q * (g_sum + b * s.W) * s.D
    peak_flops = 2.5e15
    return 1e6 * (max(is_bytes / (HBM_PEAK_GBPS * 1e9), is_flops / peak_flops)
                  + max(sa_bytes / (HBM_PEAK_GBPS * 1e9), sa_flops / peak_flops))


def mt_step_bytes(s, T: int) -> int:
    """Compulsory bytes of a step with T query tokens per batch row: the
    keys (K_I) read once for all tokens; per token its indexer query and
    weights, its q, its gathered rows and window, and its output."""
    b = s.B
    return (b * s.N * s.D_I * 2
            + T * b * (s.H_I * s.D_I * 2 + s.H_I * 4 + s.H_q * s.D * 2
                       + (s.k + s.W) * s.D * 2 + s.H_q * s.D * 2))


def mt_step_roofline_us(s, T: int) -> float:
    """step_roofline_us with T tokens: indexer bytes counted once, its
    flops and every attention term T times."""
    b = s.B
    is_bytes = b * s.N * s.D_I * 2 + T * b * (s.H_I * s.D_I * 2 + s.H_I * 4)
    is_flops = 2 * T * b * s.N * s.H_I * s.D_I
    sa_bytes = mt_step_bytes(s, T) - is_bytes
    sa_flops = 4 * T * b * s.H_q * (s.k + s.W) * s.D
    peak_flops = 2.5e15
    return 1e6 * (max(is_bytes / (HBM_PEAK_GBPS * 1e9), is_flops / peak_flops)
                  + max(sa_bytes / (HBM_PEAK_GBPS * 1e9), sa_flops / peak_flops))


def time_calls(fn, n_warm, n_timed, stream):
    """Mean µs per call of fn(i) over n_timed back-to-back calls on stream."""
    import torch
    for i in range(n_warm):
        fn(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n_timed):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / n_timed


def graph_replay_us(s, copies, out, ws, steps) -> dict:
    """The same steps captured into one HIP graph (one step per input copy,
    in rotation order) and replayed back to back: the launch cost per step
    without host enqueue. A failure here is reported, not raised."""
    import torch
    import indexer_top_gathered_amd as dsa
    R = len(copies)

    def record():
        for c in copies:  # on the current stream: the capture stream inside the graph
            dsa.dsa_decode_step(c["q_idx"], c["k_idx"], c["w"], c["q"], c["kv_cmp"],
                                c["kv_win"], s.k, s.scale, out=out, ws=ws)
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            record()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            record()
        torch.cuda.synchronize()
        replays = max(2, steps // R)
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(replays):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (replays * R)
        del g
        return {"us_per_step": round(us, 2), "steps_per_graph": R, "replays": replays}
    except Exception as exc:  # noqa: BLE001
        return {"error": str(exc)[:200]}


def other_workload(args):
    """One JSON line for a workload other than the production step."""
    import torch
    import workloads
    import indexer_top_gathered_amd as dsa

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    line = {"workload": args.workload, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "data": "synthetic", "unit": "GB/s", "higher_is_better": True}
    if args.workload in ("tiny-step", "stress-step"):
        s = workloads.C1 if args.workload == "tiny-step" else workloads.C5
        one = step_bytes(s)
        # Enough copies to exceed 1 GB (the stress step's one copy is ~21 GB).
        R = max(1, min(256, -(-(1 << 30) // one)))
        if args.workload == "tiny-step":
            copies = [workloads.step_inputs(s, 1000 + 10 * r, device=dev) for r in range(R)]
        else:
            copies = [workloads.stress_step_inputs(s, 5000 + 10 * r, device=dev) for r in range(R)]
        dims = dsa.make_dims(s.B, s.N, s.H_I, s.D_I, s.k, s.W, s.H_q, s.D, s.scale)
        ws = torch.empty(dsa.dsa_decode_step_workspace_bytes(dims), dtype=torch.uint8, device=dev)
        out = torch.empty((s.B, s.H_q, s.D), dtype=torch.bfloat16, device=dev)

        def call(i):
            c = copies[i % R]
            dsa.dsa_decode_step(c["q_idx"], c["k_idx"], c["w"], c["q"], c["kv_cmp"], c["kv_win"],
                                s.k, s.scale, out=out, ws=ws, stream=stream)
        us = time_calls(call, args.warmup, args.steps, stream)
        roof = step_roofline_us(s)
        line.update({"us_per_step": round(us, 2), "value": round(one / (us * 1e-6) / 1e9, 1),
                     "compulsory_bytes": one, "roofline_us": round(roof, 3),
                     "frac_of_roofline": round(roof / us, 4), "rotating_input_copies": R,
                     "config": {"B": s.B, "N": s.N, "H_I": s.H_I, "D_I": s.D_I, "k": s.k,
                                "W": s.W, "H_q": s.H_q, "D": s.D}})
        if args.workload == "tiny-step":
            line["graph"] = graph_replay_us(s, copies, out, ws, args.steps)
        print(json.dumps(line), flush=True)
        return
    if args.workload == "sink-step":
        # The production step with an attention sink per query head, next to
        # the same inputs without one (the sink adds one logit per head to the
        # normalisation and no bytes worth counting).
        s = workloads.C4
        R = max(1, min(256, -(-(1 << 30) // step_bytes(s))))
        copies = [workloads.step_inputs(s, 6500 + 10 * r, device=dev) for r in range(R)]
        gen = torch.Generator(device=dev).manual_seed(6599)
        sink = torch.randn(s.H_q, generator=gen, device=dev, dtype=torch.float32)
        dims = dsa.make_dims(s.B, s.N, s.H_I, s.D_I, s.k, s.W, s.H_q, s.D, s.scale)
        ws = torch.empty(dsa.dsa_decode_step_workspace_bytes(dims), dtype=torch.uint8, device=dev)
        out = torch.empty((s.B, s.H_q, s.D), dtype=torch.bfloat16, device=dev)

        def call_sink(i):
            c = copies[i % R]
            dsa.dsa_decode_step_sink(c["q_idx"], c["k_idx"], c["w"], c["q"], c["kv_cmp"],
                                     c["kv_win"], sink, s.k, s.scale, out=out, ws=ws,
                                     stream=stream)

        def call_plain(i):
            c = copies[i % R]
            dsa.dsa_decode_step(c["q_idx"], c["k_idx"], c["w"], c["q"], c["kv_cmp"],
                                c["kv_win"], s.k, s.scale, out=out, ws=ws, stream=stream)
        us = time_calls(call_sink, args.warmup, args.steps, stream)
        us_plain = time_calls(call_plain, args.warmup, args.steps, stream)
        one = step_bytes(s)
        roof = step_roofline_us(s)
        line.update({"us_per_step": round(us, 2), "value": round(one / (us * 1e-6) / 1e9, 1),
                     "compulsory_bytes": one, "roofline_us": round(roof, 3),
                     "frac_of_roofline": round(roof / us, 4),
                     "without_sink_us_per_step": round(us_plain, 2),
                     "rotating_input_copies": R,
                     "config": {"B": s.B, "N": s.N, "H_I": s.H_I, "D_I": s.D_I, "k": s.k,
                                "W": s.W, "H_q": s.H_q, "D": s.D, "sink": "N(0, 1) per head"}})
        print(json.dumps(line), flush=True)
        return
    if args.workload == "ragged-step":
        # The production step's shape over a serving batch of mixed lengths,
        # next to the same inputs at full length.
        s = workloads.C4
        lengths = workloads.serving_lengths(s.B, s.N, 6000)
        lens = torch.from_numpy(lengths).to(dev)
        full = torch.full((s.B,), s.N, dtype=torch.int32, device=dev)
        R = max(1, min(256, -(-(1 << 30) // step_bytes(s))))
        copies = [workloads.step_inputs(s, 6000 + 10 * r, device=dev) for r in range(R)]
        dims = dsa.make_dims(s.B, s.N, s.H_I, s.D_I, s.k, s.W, s.H_q, s.D, s.scale)
        ws = torch.empty(dsa.dsa_decode_step_workspace_bytes(dims), dtype=torch.uint8, device=dev)
        out = torch.empty((s.B, s.H_q, s.D), dtype=torch.bfloat16, device=dev)

        def caller(lv):
            def call(i):
                c = copies[i % R]
                dsa.dsa_decode_step_ragged(c["q_idx"], c["k_idx"], c["w"], c["q"], c["kv_cmp"],
                                           c["kv_win"], lv, s.k, s.scale, out=out, ws=ws,
                                           stream=stream)
            return call
        us = time_calls(caller(lens), args.warmup, args.steps, stream)
        us_full = time_calls(caller(full), args.warmup, args.steps, stream)
        one = ragged_step_bytes(s, lengths)
        roof = ragged_step_roofline_us(s, lengths)
        line.update({"us_per_step": round(us, 2), "value": round(one / (us * 1e-6) / 1e9, 1),
                     "compulsory_bytes": one, "roofline_us": round(roof, 3),
                     "frac_of_roofline": round(roof / us, 4),
                     "mean_length": round(float(lengths.mean()), 1),
                     "full_length_us_per_step": round(us_full, 2),
                     "rotating_input_copies": R,
                     "config": {"B": s.B, "N": s.N, "H_I": s.H_I, "D_I": s.D_I, "k": s.k,
                                "W": s.W, "H_q": s.H_q, "D": s.D,
                                "lengths": "uniform on [1, N], seed 6000"}})
        print(json.dumps(line), flush=True)
        return
    if args.workload == "context-sweep":
        # The production step's shape at compressed lengths N = 2K .. 32K,
        # i.e. 8K .. 128K tokens folded 4 to 1: the context range over which
        # the CSA pull request reports its block latency.
        import dataclasses
        results = []
        for N in (2048, 4096, 8192, 16384, 32768):
            s = dataclasses.replace(workloads.C4, N=N)
            one = step_bytes(s)
            R = max(1, min(256, -(-(1 << 30) // one)))
            copies = [workloads.step_inputs(s, 9000 + N + 10 * r, device=dev) for r in range(R)]
            dims = dsa.make_dims(s.B, s.N, s.H_I, s.D_I, s.k, s.W, s.H_q, s.D, s.scale)
            ws = torch.empty(dsa.dsa_decode_step_workspace_bytes(dims), dtype=torch.uint8,
                             device=dev)
            out = torch.empty((s.B, s.H_q, s.D), dtype=torch.bfloat16, device=dev)

            def call(i, copies=copies, ws=ws, out=out, s=s, R=R):
                c = copies[i % R]
                dsa.dsa_decode_step(c["q_idx"], c["k_idx"], c["w"], c["q"], c["kv_cmp"],
                                    c["kv_win"], s.k, s.scale, out=out, ws=ws, stream=stream)
            us = time_calls(call, args.warmup, args.steps, stream)
            roof = step_roofline_us(s)
            results.append({"N": N, "tokens": 4 * N, "us_per_step": round(us, 2),
                            "effective_GBps": round(one / (us * 1e-6) / 1e9, 1),
                            "roofline_us": round(roof, 3), "frac_of_roofline": round(roof / us, 4),
                            "rotating_input_copies": R})
            del copies
        line.update({"us_per_step": results[-1]["us_per_step"],
                     "value": results[-1]["effective_GBps"], "results": results,
                     "latency_ratio_128k_over_8k": round(results[-1]["us_per_step"]
                                                         / results[0]["us_per_step"], 3),
                     "config": {"B": workloads.C4.B, "N": [r["N"] for r in results],
                                "H_I": 64, "D_I": 128, "k": 1024, "W": 128, "H_q": 128,
                                "D": 512}})
        print(json.dumps(line), flush=True)
        return
    if args.workload == "qproj":
        # The indexer query projection of a decode batch: B = 16 rows of a
        # synthetic 4096-wide input onto 64 heads x 128 channels.
        B, d_in, H = 16, 4096, 64
        nbytes = H * 128 * d_in * 2 + B * d_in * 2 + B * H * 128 * 2
        R = max(1, -(-(1 << 30) // nbytes))
        copies = [workloads.qproj_inputs(B, d_in, H, 8000 + 10 * r, device=dev) for r in range(R)]
        outq = torch.empty((B, H, 128), dtype=torch.bfloat16, device=dev)

        def call(i):
            c = copies[i % R]
            dsa.dsa_indexer_qproj(c["x"], c["w_q"], H, q_idx=outq, stream=stream)
        us = time_calls(call, args.warmup, args.steps, stream)
        gbps = nbytes / (us * 1e-6) / 1e9
        line.update({"us": round(us, 2), "value": round(gbps, 1),
                     "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
                     "compulsory_bytes": nbytes, "rotating_input_copies": R,
                     "config": {"B": B, "d_in": d_in, "H_I": H, "D_I": 128,
                                "weights": "synthetic, N(0, 1/d_in)"}})
        print(json.dumps(line), flush=True)
        return
    if args.workload == "compress":
        # The compressor on the production KV width (D = 512): a decode step's
        # fold of 4 raw rows per batch row (G = 1), and a 4096-token prompt
        # chunk per batch row (G = 1024).
        import math
        B, D = 16, 512
        results = []
        for G in (1, 1024):
            nbytes = B * 4 * G * D * 2 + D * 4 + B * G * D * 2
            R = max(1, min(256, -(-(1 << 30) // nbytes)))
            gen = torch.Generator(device=dev).manual_seed(8500 + G)
            xs = [torch.randn(B, 4 * G, D, generator=gen, device=dev).to(torch.bfloat16)
                  for _ in range(R)]
            wg = (torch.randn(D, generator=gen, device=dev) / math.sqrt(D)).float()
            outc = torch.empty((B, G, D), dtype=torch.bfloat16, device=dev)

            def call(i, xs=xs, wg=wg, outc=outc):
                dsa.dsa_compress(xs[i % R], wg, out=outc, stream=stream)
            us = time_calls(call, args.warmup, args.steps, stream)
            gbps = nbytes / (us * 1e-6) / 1e9
            results.append({"groups_per_row": G, "us": round(us, 2),
                            "effective_GBps": round(gbps, 1),
                            "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
                            "compulsory_bytes": nbytes, "rotating_input_copies": R})
            del xs
        line.update({"value": results[-1]["effective_GBps"], "results": results,
                     "config": {"B": B, "D": D, "groups": [1, 1024],
                                "gate": "synthetic, N(0, 1/D)"}})
        print(json.dumps(line), flush=True)
        return
    if args.workload == "mtp-step":
        # The production step's shape with T = 2 query tokens per batch row
        # (one draft token), next to T = 1 and T = 4; the keys are read once
        # per step whatever T is.
        s = workloads.C4
        R = max(1, min(256, -(-(1 << 30) // step_bytes(s))))
        results = []
        for T in (1, 2, 4):
            copies = [workloads.mt_step_inputs(s, T, 7000 + 10 * r, device=dev) for r in range(R)]
            dims = dsa.make_dims(s.B, s.N, s.H_I, s.D_I, s.k, s.W, s.H_q, s.D, s.scale)
            ws = torch.empty(dsa.dsa_decode_step_mt_workspace_bytes(dims, T), dtype=torch.uint8,
                             device=dev)
            out = torch.empty((s.B, T, s.H_q, s.D), dtype=torch.bfloat16, device=dev)
            sc = torch.empty((s.B, T, s.N), dtype=torch.float32, device=dev)

            def call(i, T=T, copies=copies, ws=ws, out=out):
                c = copies[i % R]
                dsa.dsa_decode_step_mt(c["q_idx"], c["k_idx"], c["w"], c["q"], c["kv_cmp"],
                                       c["kv_win"], s.k, s.scale, out=out, ws=ws, stream=stream)

            def call_is(i, copies=copies, sc=sc):
                c = copies[i % R]
                dsa.dsa_indexer_score_mt(c["q_idx"], c["k_idx"], c["w"], scores=sc,
                                         stream=stream)
            us = time_calls(call, args.warmup, args.steps, stream)
            us_is = time_calls(call_is, args.warmup, args.steps, stream)
            one = mt_step_bytes(s, T)
            roof = mt_step_roofline_us(s, T)
            results.append({"tokens": T, "us_per_step": round(us, 2),
                            "us_per_token": round(us / T, 2),
                            "effective_GBps": round(one / (us * 1e-6) / 1e9, 1),
                            "compulsory_bytes": one, "roofline_us": round(roof, 3),
                            "frac_of_roofline": round(roof / us, 4),
                            "indexer_us": round(us_is, 2)})
            del copies
        two = results[1]
        line.update({"us_per_step": two["us_per_step"], "value": two["effective_GBps"],
                     "results": results, "rotating_input_copies": R,
                     "config": {"B": s.B, "N": s.N, "H_I": s.H_I, "D_I": s.D_I, "k": s.k,
                                "W": s.W, "H_q": s.H_q, "D": s.D, "tokens": 2}})
        print(json.dumps(line), flush=True)
        return
    # Top-k workloads.
    if args.workload == "topk-sampling":
        t = workloads.C3
        cases = [("f32", lambda r: workloads.sampling_rows(t.B, t.N, 3006 + r, device=dev))]
    else:
        t = workloads.C5_TOPK
        cases = [(dt, (lambda r, dt=dt: workloads.stress_levels(t.B, t.N, 5008 + r, device=dev, dtype=dt)))
                 for dt in ("bf16", "f32")]
    results = []
    for dt, make in cases:
        esz = 2 if dt == "bf16" else 4
        tbytes = t.B * t.N * esz + t.B * t.k * 4 + (t.B * t.k * esz if t.values else 0)
        R = max(1, -(-(1 << 30) // (t.B * t.N * esz)))
        rows = [make(r) for r in range(R)]
        tdt = torch.bfloat16 if dt == "bf16" else torch.float32
        tws = torch.empty(dsa.dsa_topk_workspace_bytes(t.B, t.N, t.k, tdt), dtype=torch.uint8,
                          device=dev)
        oidx = torch.empty((t.B, t.k), dtype=torch.int32, device=dev)
        oval = torch.empty((t.B, t.k), dtype=tdt, device=dev) if t.values else None

        def call(i):
            dsa.dsa_topk(rows[i % R], t.k, out_idx=oidx, out_val=oval, ws=tws, stream=stream)
        us = time_calls(call, args.warmup, args.steps, stream)
        gbps = tbytes / (us * 1e-6) / 1e9
        results.append({"dtype": dt, "us": round(us, 2), "effective_GBps": round(gbps, 1),
                        "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
                        "compulsory_bytes": tbytes, "rotating_input_copies": R})
        del rows
    line.update({"value": results[0]["effective_GBps"], "results": results,
                 "config": {"B": t.B, "N": t.N, "k": t.k, "values": t.values}})
    print(json.dumps(line), flush=True)


def indexer_bytes(s) -> int:
    """Algorithmic bytes of one indexer-score launch: k_idx, q_idx and w read
    once, the float32 score rows written once."""
    b = s.B
    return b * s.N * s.D_I * 2 + b * s.H_I * s.D_I * 2 + b * s.H_I * 4 + b * s.N * 4


def topk_stage_bytes(B: int, N: int, k: int, esz: int, values: bool = False) -> int:
    """Algorithmic bytes of one top-k call: the score rows read once, the
    indices (and values) written once."""
    return B * N * esz + B * k * 4 + (B * k * esz if values else 0)


def attend_bytes(s) -> int:
    """Algorithmic bytes of one sparse-attention call: q, the index array,
    the k gathered rows and W window rows of every batch row read once (a
    row is both K and V), the output written once."""
    b = s.B
    return (b * s.H_q * s.D * 2 + b * s.k * 4 + b * (s.k + s.W) * s.D * 2
            + b * s.H_q * s.D * 2)


def attend_flops(s) -> int:
    return 4 * s.B * s.H_q * (s.k + s.W) * s.D


def source_digest(parts) -> str:
    """Hash of the code a kernel is built and launched from. parts: paths,
    or (path, start, stop) to take the text from the first `start` up to the
    first `stop` after it (None: the file's start or end). Comments and
    blank space are dropped, so a comment edit does not void counters taken
    on the same code."""
    import re
    h = hashlib.sha256()
    for part in parts:
        path, start, stop = (part, None, None) if isinstance(part, str) else part
        with open(path, encoding="utf-8") as f:
            text = f.read()
        if start is not None:
            text = text[text.index(start):]
        if stop is not None:
            text = text[:text.index(stop)]
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def library_source_parts():
    """Every source libdsa.so is built from (kernels, launchers, the ABI)."""
    csrc = os.path.join(ROOT, "indexer_top_gathered_amd", "csrc")
    return [os.path.join(csrc, f) for f in sorted(os.listdir(csrc))
            if f.endswith((".hip", ".h"))]


COUNTERS = os.path.join(ROOT, "profiles", "decode_step_b16_n32768_counters.md")
# The production step's kernels, in launch order: the indexer with the chunk
# cut, attention whose workgroups select their rows from the cut's candidates
# (4 candidate slots per thread), and the split combine.
STEP_KERNELS = ("indexer_score_cut_kernel<4>", "sparse_attend_kernel<512, 4, 2, 4>",
                "attend_combine_kernel<512>")
# The stage legs: dsa_indexer_topk (the cut and its merge kernel) and
# dsa_sparse_attend on given indices (attention and the combine).
ITK_KERNELS = ("indexer_score_cut_kernel<4>", "topk_merge_kernel<false, 4, true>")
ATTEND_KERNELS = ("sparse_attend_kernel<512, 4, 2, 0>", "attend_combine_kernel<512>")


def traffic_from_profile():
    """HBM bytes per dispatch of each kernel, from the two rocprofv3 counter
    passes summarised in profiles/ (FETCH_SIZE and WRITE_SIZE, scaled by a
    copy of known size), if they were taken on the current library sources
    (source_digest of library_source_parts); else {}."""
    if not os.path.exists(COUNTERS):
        return {}
    vals = {}
    for line in open(COUNTERS, encoding="utf-8"):
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            vals[k.strip().strip("`")] = v.strip().strip("`")
    if vals.get("library_source_sha256_16") != source_digest(library_source_parts()):
        return {}
    out = {}
    for k, v in vals.items():
        if k.startswith("hbm_bytes_per_dispatch "):
            try:
                out[k.split(" ", 1)[1]] = float(v)
            except ValueError:
                pass
    return out


def check_topk_output(idx, N: int, k: int, where: str) -> None:
    """Every row holds k distinct positions in [0, N) (checked on the
    device); raises otherwise."""
    import torch
    srt = torch.sort(idx.long(), dim=1).values
    ok = (bool((srt[:, 0] >= 0).all()) and bool((srt[:, -1] < N).all())
          and (k == 1 or bool((srt[:, 1:] != srt[:, :-1]).all())))
    if idx.shape[1] != k or not ok:
        raise RuntimeError(f"{where}: the timed output is not k distinct in-range indices")


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo", encoding="utf-8"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def torch_step(c, s):
    """The decode step written with plain torch ops on the GPU (context for
    the fused kernels, as the pages compare against a naive baseline): a
    batched matmul for the indexer (fp32 results, so that the selection is
    the fused path's), torch.topk, a gather and matmul/softmax attention.
    Right-hand matmul operands are made contiguous first."""
    import torch
    kt = c["k_idx"].transpose(1, 2).contiguous()                      # [B, 128, N]
    dots = torch.bmm(c["q_idx"], kt, out_dtype=torch.float32)          # [B, H_I, N]
    scores = (torch.relu(dots) * c["w"][:, :, None]).sum(1)            # [B, N]
    idx = torch.topk(scores, s.k, dim=1, sorted=False).indices         # [B, k]
    rows = torch.gather(c["kv_cmp"], 1, idx[:, :, None].expand(-1, -1, s.D))
    rows = torch.cat([rows, c["kv_win"]], dim=1)                       # [B, k+W, D]
    logits = torch.bmm(c["q"], rows.transpose(1, 2).contiguous(), out_dtype=torch.float32)
    logits = logits * s.scale
    p = torch.softmax(logits, dim=-1).to(torch.bfloat16)
    return torch.bmm(p, rows.contiguous())                             # [B, H_q, D]


def single_call_latency(call, n: int, dev, stream) -> dict:
    """Latency of one call from cold caches: before each call a 512 MiB
    buffer is written (twice the 256 MB Infinity Cache, far beyond the L2s),
    then the call alone is bracketed by events. Median, p10 and p90 in us."""
    import torch
    import numpy as np
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    samples = []
    for i in range(n):
        scratch.fill_(i & 0xFF)
        e0.record(stream)
        call(i)
        e1.record(stream)
        e1.synchronize()
        samples.append(e0.elapsed_time(e1) * 1e3)
    del scratch
    a = np.array(samples)
    return {"calls": n, "median_us": round(float(np.median(a)), 2),
            "p10_us": round(float(np.percentile(a, 10)), 2),
            "p90_us": round(float(np.percentile(a, 90)), 2),
            "eviction": "512 MiB device write before each call"}


def bandwidth_probe(dev, stream) -> dict:
    """Measured HBM rates of plain torch kernels on 1 GiB, for the roofline
    fraction against what this GPU delivers as well as against 8 TB/s: a
    read-only row reduction (sums of rows of 4096 floats; of the torch
    reductions tried it streams fastest, a whole-tensor sum reaches about
    two thirds of it) and a copy (read + write). The row reduction is also
    timed in calls of 128 MiB each, the indexer's key bytes per step, taken
    in turn from the 8 eighths of the GiB (so none is served from the 256 MB
    Infinity Cache): the rate a single launch of that size reaches, its
    start and drain included."""
    import torch
    n = 1 << 30
    x = torch.ones(n // 4, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    out = {}
    eighths = x.view(8, -1, 4096)
    calls = [0]

    def eighth_sum():
        calls[0] += 1
        return eighths[calls[0] % 8].sum(1)

    for name, fn, nbytes, reps in (
            ("read_GBps (row sums, 1 GiB)", lambda: x.view(-1, 4096).sum(1), n, 10),
            ("copy_GBps (read + write, 1 GiB each)", lambda: y.copy_(x), 2 * n, 10),
            ("read_GBps (row sums, 128 MiB per call)", eighth_sum, n // 8, 80)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        out[name] = round(nbytes / (us * 1e-6) / 1e9, 1)
    del x, y
    return out


def stage(name: str, kernels: str, nbytes: int, us: float, flops: int = 0, traffic=None) -> dict:
    """One stage of the step against its own roofline: the larger of its
    HBM time at 8 TB/s and its MFMA time at 2.5 PFLOP/s."""
    t_hbm = nbytes / (HBM_PEAK_GBPS * 1e9) * 1e6
    t_mfma = flops / 2.5e15 * 1e6
    d = {"kernels": kernels, "us": round(us, 3), "algorithmic_bytes": nbytes,
         "achieved_GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
         "roofline_us": round(max(t_hbm, t_mfma), 3),
         "frac": round(max(t_hbm, t_mfma) / us, 4),
         "bound": "hbm" if t_hbm >= t_mfma else "mfma"}
    if flops:
        d["flops"] = flops
        d["mfma_TFLOPs"] = round(flops / (us * 1e-6) / 1e12, 1)
    d["traffic"] = traffic
    return d


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(batch rows are independent, so N GPUs would each run this same kernel set "
              "on B/N rows).", file=sys.stderr)
        sys.exit(2)
    if args.workload != "step":
        other_workload(args)
        return
    import torch
    import workloads
    import indexer_top_gathered_amd as dsa

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    s = workloads.C4
    R = max(1, args.copies)
    copies = [workloads.step_inputs(s, 4000 + 10 * r, device=dev) for r in range(R)]
    dims = dsa.make_dims(s.B, s.N, s.H_I, s.D_I, s.k, s.W, s.H_q, s.D, s.scale)
    ws = torch.empty(dsa.dsa_decode_step_workspace_bytes(dims), dtype=torch.uint8, device=dev)
    out = torch.empty((s.B, s.H_q, s.D), dtype=torch.bfloat16, device=dev)
    oidx = torch.empty((s.B, s.k), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        c = copies[i % R]
        dsa.dsa_decode_step(c["q_idx"], c["k_idx"], c["w"], c["q"], c["kv_cmp"], c["kv_win"],
                            s.k, s.scale, out=out, out_idx=oidx, ws=ws, stream=stream)

    us_step = time_calls(step, args.warmup, args.steps, stream)
    ms_per_step = us_step / 1e3
    sbytes = step_bytes(s)
    value = sbytes / (us_step * 1e-6) / 1e9
    # The timed loop's last output: k distinct in-range indices per row, and
    # bit-identical to an untimed call on the same inputs.
    last = (args.steps - 1) % R
    check_topk_output(oidx, s.N, s.k, "decode step")
    c = copies[last]
    out_chk, idx_chk = dsa.dsa_decode_step(c["q_idx"], c["k_idx"], c["w"], c["q"], c["kv_cmp"],
                                           c["kv_win"], s.k, s.scale, return_idx=True)
    torch.cuda.synchronize()
    if not (torch.equal(idx_chk, oidx) and torch.equal(out_chk.view(torch.int16),
                                                      out.view(torch.int16))):
        raise RuntimeError("decode step: the timed output differs from an untimed call")
    del out_chk, idx_chk

    # Each stage alone, in the step's launch configuration, on the same
    # stream over the same rotation.
    traffic = traffic_from_profile()

    def tsum(*names):
        vals = [traffic.get(n) for n in names]
        return None if not vals or any(v is None for v in vals) else round(sum(vals))

    scores = torch.empty((s.B, s.N), dtype=torch.float32, device=dev)
    sel = torch.empty((s.B, s.k), dtype=torch.int32, device=dev)
    itws = torch.empty(dsa.dsa_indexer_topk_workspace_bytes(s.B, s.N, s.H_I, s.k, False),
                       dtype=torch.uint8, device=dev)
    aws = torch.empty(max(256, dsa.dsa_sparse_attend_workspace_bytes(dims)), dtype=torch.uint8,
                      device=dev)

    def is_call(i):
        c = copies[i % R]
        dsa.dsa_indexer_score(c["q_idx"], c["k_idx"], c["w"], scores=scores, stream=stream)
    is_us = time_calls(is_call, args.warmup, args.steps, stream)

    def itk_call(i):
        c = copies[i % R]
        dsa.dsa_indexer_topk(c["q_idx"], c["k_idx"], c["w"], s.k, out_idx=sel, scores=scores,
                             ws=itws, stream=stream)
    itk_us = time_calls(itk_call, args.warmup, args.steps, stream)
    # Selections of every copy for the attention leg.
    all_idx = [dsa.dsa_indexer_topk(c["q_idx"], c["k_idx"], c["w"], s.k) for c in copies]

    def sa_call(i):
        c = copies[i % R]
        dsa.dsa_sparse_attend(c["q"], c["kv_cmp"], all_idx[i % R], c["kv_win"], s.scale,
                              out=out, ws=aws, stream=stream)
    sa_us = time_calls(sa_call, args.warmup, args.steps, stream)
    del all_idx

    kernels = {
        "indexer": stage("indexer", "indexer_score_kernel<4>", indexer_bytes(s), is_us,
                         flops=2 * s.B * s.N * s.H_I * s.D_I,
                         traffic=tsum("indexer_score_kernel<4>")),
        "indexer_topk": stage("indexer_topk", " + ".join(ITK_KERNELS),
                              indexer_bytes(s) + s.B * s.k * 4, itk_us,
                              flops=2 * s.B * s.N * s.H_I * s.D_I, traffic=tsum(*ITK_KERNELS)),
        "attention": stage("attention", " + ".join(ATTEND_KERNELS),
                           attend_bytes(s), sa_us, flops=attend_flops(s),
                           traffic=tsum(*ATTEND_KERNELS)),
    }
    roof_us = step_roofline_us(s)
    step_traffic = tsum(*STEP_KERNELS)
    roofline = {"bound": "hbm", "achieved": round(value, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(value / HBM_PEAK_GBPS, 4), "traffic": step_traffic,
                "what": "the whole decode step: compulsory bytes per step / time per step",
                "step_kernels": list(STEP_KERNELS),
                "roofline_us": round(roof_us, 3), "us_per_step": round(us_step, 2),
                "frac_of_step_roofline": round(roof_us / us_step, 4),
                "bytes_per_step": sbytes, "kernels": kernels}

    if args.latency_calls > 0:
        probe = bandwidth_probe(dev, stream)
        roofline["measured_hbm"] = probe
        ia = kernels["indexer"]["achieved_GBps"]
        kernels["indexer"]["frac_of_measured_read"] = round(
            ia / probe["read_GBps (row sums, 1 GiB)"], 4)
        kernels["indexer"]["frac_of_measured_read_same_size"] = round(
            ia / probe["read_GBps (row sums, 128 MiB per call)"], 4)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(us_step, 2), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "decode step B=16 N=32768 H_I=64 D_I=128 k=1024 W=128 "
                               "H_q=128 D=512 (K=V)", "global_batch": s.B,
                   "compulsory_bytes_per_step": sbytes, "rotating_input_copies": R,
                   "parallelism": "single GPU"},
        "roofline": roofline,
    }
    del scores, sel, itws, aws

    line["graph"] = graph_replay_us(s, copies, out, ws, args.steps)
    if args.latency_calls > 0:
        line["single_call_latency"] = single_call_latency(step, args.latency_calls, dev, stream)
        # The same step in plain torch ops on this GPU, over the same rotation
        # (context only: a failure here is reported, not raised).
        try:
            n_ref = max(10, args.steps // 10)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                for i in range(3):
                    torch_step(copies[i % R], s)
                torch.cuda.synchronize()
                e0.record(stream)
                for i in range(n_ref):
                    torch_step(copies[i % R], s)
                e1.record(stream)
            torch.cuda.synchronize()
            t_us = e0.elapsed_time(e1) * 1e3 / n_ref
            line["torch_step"] = {"us": round(t_us, 2), "speedup": round(t_us / us_step, 2),
                                  "ops": "bmm indexer, torch.topk, gather, bmm/softmax attention"}
        except Exception as exc:  # noqa: BLE001
            line["torch_step"] = {"error": str(exc)[:200]}

    if not args.no_topk:
        t = workloads.C2
        rows = [workloads.normal_rows(t.B, t.N, "bf16", 2006 + r, device=dev) for r in range(R)]
        tws = torch.empty(dsa.dsa_topk_workspace_bytes(t.B, t.N, t.k, torch.bfloat16),
                          dtype=torch.uint8, device=dev)
        tidx = torch.empty((t.B, t.k), dtype=torch.int32, device=dev)

        def tk2(i):
            dsa.dsa_topk(rows[i % R], t.k, out_idx=tidx, ws=tws, stream=stream)
        tk_us = time_calls(tk2, args.warmup, args.steps, stream)
        check_topk_output(tidx, t.N, t.k, "top-k")
        again = dsa.dsa_topk(rows[(args.steps - 1) % R], t.k)
        torch.cuda.synchronize()
        if not torch.equal(again, tidx):
            raise RuntimeError("top-k: the timed output differs from an untimed call")
        tbytes = topk_stage_bytes(t.B, t.N, t.k, 2)

        def ref(i):
            torch.topk(rows[i % R], t.k, dim=1, sorted=False)
        ref_us = time_calls(ref, 3, max(10, args.steps // 10), stream)
        gbps = tbytes / (tk_us * 1e-6) / 1e9
        line["topk"] = {"workload": "bf16 scores 64 x 131072, k=512, indices only, unsorted",
                        "us": round(tk_us, 2), "effective_GBps": round(gbps, 1),
                        "frac": round(gbps / HBM_PEAK_GBPS, 4),
                        "roofline_us": round(tbytes / (HBM_PEAK_GBPS * 1e9) * 1e6, 3),
                        "compulsory_bytes": tbytes, "torch_topk_us": round(ref_us, 2),
                        "speedup_vs_torch_topk": round(ref_us / tk_us, 2),
                        "output_checked": "k distinct in-range indices per row; equal to an "
                                          "untimed call"}
        line["metric_parts"] = {"topk_effective_GBps": round(gbps, 1),
                                "decode_step_us": round(us_step, 2)}
        del rows

    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        line["calibration_copy_bytes"] = n
        del src, dst

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(copies[0], s, sbytes)

    print(json.dumps(line), flush=True)


def cpu_baseline(inp, s, sbytes):
    """The CPU oracle (plain C, double precision) on the same workload: the
    whole step (indexer, sort-based top-k, softmax attention) over all 16
    batch rows, with one OpenMP thread per batch row at most, repeated until
    about 10 s of CPU time have passed (at least once)."""
    import torch
    import oracle
    import workloads

    h = {k: (workloads.bits16(v) if v.dtype == torch.bfloat16 else v.cpu().numpy())
         for k, v in inp.items()}
    ncpu = len(os.sched_getaffinity(0))
    threads = max(1, min(ncpu, s.B))
    oracle.set_threads(threads)
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.step(h["q_idx"], h["k_idx"], h["w"], h["q"], h["kv_cmp"], h["kv_win"], s.k, s.scale)
        reps += 1
        if time.perf_counter() - t0 >= 10.0 or reps >= 32:
            break
    dt = (time.perf_counter() - t0) / reps
    return {"value": round(sbytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "seconds_per_step": round(dt, 3), "host_cpus": ncpu,
            "cpu_model": cpu_model(),
            "sample": f"the whole decode step (all 16 batch rows of the production shape), "
                      f"{reps} repetitions, mean time per step"}


if __name__ == "__main__":
    main()
