"""Throughput of the chunked LaCT fast-weight layer on one MI355X.

A step is one ttt_lact_forward call over the LM-layer workload: 4 sequences x 8 heads,
h = 128, r = 2 (rh = 256), 32768 tokens per sequence in 16 chunks of 2048, apply-then-update,
per-token eta, momentum 0.9, Newton-Schulz-5 and input-dim renormalisation, bf16 I/O,
final state written. Inputs are seeded synthetic data already resident in HBM.

Prints one JSON line with the throughput (tokens/s over all heads), the roofline of the
dominant kernel (algorithmic FLOPs per launch / its average launch time, timed with HIP events
on the library's stream) and the CPU oracle timed on the host cores on a bounded sample.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU oracle sample")
    return ap.parse_args()


def cpu_baseline(p, x, budget_s):
    """The oracle (float32 NumPy, as it stands) on whole (sequence, head) pairs of the same
    workload until the time budget is used; scaled to tokens/s over all heads."""
    import numpy as np
    from oracle import lact as oracle_lact
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    done = 0
    t0 = time.perf_counter()
    pairs = [(b, h) for b in range(p.B) for h in range(p.H)]
    for (b, h) in pairs:
        oracle_lact.lact_pair(x["Q"][b, h], x["K"][b, h], x["V"][b, h], x["eta"][b, h],
                              x["W0"][h], x["W1"][h], x["W2"][h], chunk_q=p.chunk_q, chunk_kv=p.chunk_kv,
                              order=p.order, update_mask=p.update_mask, weight_norm=p.weight_norm,
                              muon=p.muon, momentum=p.momentum, eps_norm=p.eps_norm, eps_ns=p.eps_ns,
                              dtype=np.float32)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    tokens = done * p.Nq / p.H  # one pair carries 1/H of a token's heads
    return {"value": tokens / el, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {len(pairs)} (sequence, head) pairs, all {p.Nk // p.chunk_kv} chunks each, "
                      f"float32 NumPy oracle, {el:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the layer's pairs "
              "shard across GPUs without communication, see DESIGN.md", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import linear_attention_lact_amd as ttt
    from linear_attention_lact_amd import accounting as acc
    from workloads import CONFIGS, CONFIG_NAMES, make_lact_inputs

    p = CONFIGS[2]
    x = make_lact_inputs(p, 2)
    dev = torch.device("cuda:0")
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dev, dt)
    Q, K, V = (t(x[k], torch.bfloat16) for k in ("Q", "K", "V"))
    eta = t(x["eta"], torch.float32)
    W0, W1, W2 = (t(x[k], torch.float32) for k in ("W0", "W1", "W2"))
    stream = torch.cuda.current_stream()

    def step():
        return ttt.lact_forward(Q, K, V, eta, W0, W1, W2, chunk_q=p.chunk_q, chunk_kv=p.chunk_kv,
                                order=p.order, update_mask=p.update_mask, weight_norm=p.weight_norm,
                                muon=p.muon, momentum=p.momentum, eps_norm=p.eps_norm, eps_ns=p.eps_ns,
                                stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps

    tokens = p.B * p.Nq
    flops = acc.lact_flops(p.B, p.H, p.Nq, p.Nk, p.h, p.r, p.chunk_q, p.chunk_kv, p.update_mask, p.muon)
    achieved = flops / (ms * 1e-3) / 1e12
    roof = {"bound": "mfma", "kernel": "ttt_lact_forward (whole call)", "achieved": round(achieved, 2),
            "peak": acc.PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / acc.PEAK_BF16_TFLOPS, 4),
            "traffic": None, "flops_per_launch": flops, "launch_ms": round(ms, 4)}
    out = {
        "metric": "TTT-layer tokens/sec at h=128, chunk 2048 bf16; % of bf16 MFMA peak",
        "value": round(tokens / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": CONFIG_NAMES[2], "B": p.B, "H": p.H, "h": p.h, "r": p.r,
                   "seq_len": p.Nq, "chunk": p.chunk_kv, "order": "apply-then-update",
                   "momentum": p.momentum, "muon": p.muon, "weight_norm": p.weight_norm,
                   "parallelism": "single GPU"},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(p, x, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
