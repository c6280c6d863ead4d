"""Throughput of the chunked TTT-KVB fast-weight layer on one MI355X.

Default workload (the headline metric): one ttt_lact_forward call over the LM layer --
4 sequences x 8 heads, h = 128, r = 2 (rh = 256), 32768 tokens per sequence in 16 chunks of
2048, apply-then-update, per-token eta, momentum 0.9, Newton-Schulz-5 and input-dim
renormalisation, bf16 I/O, final state written. Inputs are seeded synthetic data already
resident in HBM when the timed region starts.

Prints one JSON line: throughput over all heads (tokens/s), the roofline of the dominant
kernel class (largest total time; algorithmic FLOPs or bytes per launch over its average
launch time from HIP events recorded on the library's stream), and the CPU oracle timed on
the host cores on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2] [--no-cpu-baseline]

--config 1 / 3 / 4 time the linear-attention scan, the view-synthesis shape and the In-Place
update instead (their lines are reported separately; the default line is config 2).
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
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU oracle sample")
    ap.add_argument("--momentum", type=float, default=0.0,
                    help="scan workload only: heavy-ball momentum per chunk (the momentum form)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one plain 256 MiB device-to-device copy (reference for HBM byte counters)")
    return ap.parse_args()


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_baseline_lact(p, x, budget_s):
    """The oracle (float32 NumPy, as it stands) on whole (sequence, head) pairs of the same
    workload until the time budget is used; scaled to tokens/s over all heads."""
    import numpy as np
    from oracle import lact as oracle_lact
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
    tokens = done * p.Nk / p.H  # one pair carries 1/H of each token's heads
    return {"value": round(tokens / el, 1), "unit": "tokens/s", "cores": int(blas_threads()), "kind": "oracle",
            "sample": f"{done} of {len(pairs)} (sequence, head) pairs, all {p.Nk // p.chunk_kv} chunks each, "
                      f"float32 NumPy oracle, {el:.1f} s"}


def cpu_baseline_linattn(p, x, budget_s):
    import numpy as np
    from oracle import linattn as LA
    done, t0 = 0, time.perf_counter()
    pairs = [(b, h) for b in range(p.B) for h in range(p.H)]
    for (b, h) in pairs:
        LA.linattn_pair(x["Q"][b, h], x["K"][b, h], x["V"][b, h], x["eta"][b, h], x["W0"][h], x["W1"][h],
                        x["W2"][h], chunk=p.chunk_kv, order=p.order, momentum=p.momentum, dtype=np.float32)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": round(done * p.Nk / p.H / el, 1), "unit": "tokens/s", "cores": int(blas_threads()),
            "kind": "oracle", "sample": f"{done} of {len(pairs)} pairs, float32 NumPy oracle, {el:.1f} s"}


def cpu_baseline_inplace(p, x, budget_s):
    import numpy as np
    from oracle import inplace as IP
    W = np.asarray(x["W_down"], np.float32).copy()
    done, t0 = 0, time.perf_counter()
    for i in range(p.N // p.chunk):
        sl = slice(i * p.chunk, (i + 1) * p.chunk)
        Z = IP.gated_activation(x["Hs"][0, sl], x["W_gate"], x["W_up"])
        _ = Z @ W.T
        W += np.float32(x["eta"]) * (x["Vbar"][0, sl].T @ Z)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": round(done * p.chunk / el, 1), "unit": "tokens/s", "cores": int(blas_threads()),
            "kind": "oracle", "sample": f"first {done} of {p.N // p.chunk} chunks, float32 NumPy oracle, {el:.1f} s"}


def time_steps(step, steps, warmup, stream):
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps


def kernel_breakdown(ttt, step, steps):
    """Per kernel class: launches and average launch time (HIP events on the launch stream)."""
    import torch
    torch.cuda.synchronize()
    ttt.timing_collect()
    ttt.timing_enable(True)
    try:
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        rec = ttt.timing_collect()
    finally:
        ttt.timing_enable(False)
    return {k: {"launches": n // steps, "avg_us": round(1000.0 * ms / n, 3), "total_ms_per_step": round(ms / steps, 4)}
            for k, (n, ms) in rec.items()}


# profiles/<stem>_*.txt: the committed rocprofv3 summaries of each workload
PROFILE_STEMS = {1: "linattn_scan_b4h8_h64_seq8192_chunk512", 2: "lact_lm_layer_b4h8_h128_seq32768_chunk2048",
                 3: "lact_nvs_b1h4_h192_ctx196608_q4096", 4: "inplace_down_d4096_dh14336_seq32768_chunk1024"}


def roofline(kern, work, bound, peak, unit):
    """Roofline of the class with the largest total time: work[class] = algorithmic FLOPs (or
    bytes) per launch."""
    dom = max(kern, key=lambda k: kern[k]["total_ms_per_step"])
    per_launch = work.get(dom, 0.0)
    avg_s = kern[dom]["avg_us"] * 1e-6
    scale = 1e12 if unit == "TFLOP/s" else 1e9
    achieved = per_launch / avg_s / scale if avg_s > 0 else 0.0
    return {"bound": bound, "kernel": dom, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": None,
            "work_per_launch": per_launch, "avg_launch_us": kern[dom]["avg_us"]}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the layer's "
              "(sequence, head) pairs shard across GPUs without communication, see DESIGN.md",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import linear_attention_lact_amd as ttt
    from linear_attention_lact_amd import accounting as acc
    from workloads import CONFIGS, CONFIG_NAMES, make_inplace_inputs, make_lact_inputs

    ttt.load()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dev, dt)
    k = args.config
    p = CONFIGS[k]
    stem = PROFILE_STEMS[k]
    if args.momentum != 0.0:
        if k != 1:
            print("--momentum applies to the scan workload (--config 1) only", file=sys.stderr)
            sys.exit(2)
        from dataclasses import replace
        p = replace(p, momentum=args.momentum)
        stem = "linattn_scan_momentum_b4h8_h64_seq8192_chunk512"
    if k == 4:
        x = make_inplace_inputs(p, k)
        Hs, Wg, Wu, Vb = (t(x[n], torch.bfloat16) for n in ("Hs", "W_gate", "W_up", "Vbar"))
        Wd = t(x["W_down"], torch.float32)

        def step():
            return ttt.inplace_down_forward(Hs, Wg, Wu, Wd, Vb, chunk=p.chunk, eta=float(x["eta"]), stream=stream)
        tokens = p.B * p.N
        flops = acc.inplace_flops(p.B, p.N, p.d_model, p.d_hidden)
        nch = p.N // p.chunk
        per = 2.0 * p.chunk * p.d_model * p.d_hidden
        work = {"inplace_z": 2 * per, "inplace_apply": per, "inplace_update": per}
        bound, peak, unit = "mfma", acc.PEAK_BF16_TFLOPS, "TFLOP/s"
        metric = "In-Place TTT W_down update tokens/sec (d_model 4096, d_hidden 14336, chunk 1024), bf16"
        cfg = {"workload": CONFIG_NAMES[4], "B": p.B, "seq_len": p.N, "d_model": p.d_model,
               "d_hidden": p.d_hidden, "chunk": p.chunk, "eta": p.eta}
    else:
        x = make_lact_inputs(p, k)
        io = torch.bfloat16 if p.dtype == 1 else torch.float32
        Q, K, V = (t(x[n], io) for n in ("Q", "K", "V"))
        eta = t(x["eta"], torch.float32)
        W0, W1, W2 = (t(x[n], torch.float32) for n in ("W0", "W1", "W2"))
        if k == 1:
            def step():
                return ttt.linattn_forward(Q, K, V, eta, W0, W2, W1, chunk=p.chunk_kv, order=p.order,
                                           momentum=p.momentum, stream=stream)
            flops = acc.linattn_flops(p.B, p.H, p.Nk, p.h, p.r)
            nbytes = acc.linattn_bytes(p.B, p.H, p.Nk, p.h, p.r)
            P, rh, nch = p.B * p.H, p.rh, p.Nk // p.chunk_kv
            work = {"linattn_delta": P * 2.0 * p.Nk * p.h * 2 + P * p.Nk * 4 + P * nch * rh * p.h * 4,
                    "linattn_scan": P * nch * rh * p.h * (4 + 2),
                    "linattn_apply": P * p.Nk * p.h * 2 * 2 + P * nch * rh * p.h * 2,
                    "linattn_fused": nbytes}
            bound, peak, unit = "hbm", acc.PEAK_HBM_GBS, "GB/s"
            metric = "linear-attention scan form tokens/sec (h=64, r=2, chunk 512), bf16; % of HBM roofline"
            if p.momentum:
                metric = metric.replace("scan form", f"scan form with momentum {p.momentum:g}")
        else:
            def step():
                return ttt.lact_forward(Q, K, V, eta, W0, W1, W2, chunk_q=p.chunk_q, chunk_kv=p.chunk_kv,
                                        order=p.order, update_mask=p.update_mask, weight_norm=p.weight_norm,
                                        muon=p.muon, momentum=p.momentum, eps_norm=p.eps_norm, eps_ns=p.eps_ns,
                                        stream=stream)
            flops = acc.lact_flops(p.B, p.H, p.Nq, p.Nk, p.h, p.r, p.chunk_q, p.chunk_kv, p.update_mask, p.muon)
            P, rh = p.B * p.H, p.rh
            n_upd = bin(p.update_mask & 7).count("1")
            work = {"lact_grad": P * 6 * 2.0 * p.chunk_kv * p.h * rh,
                    "lact_apply": P * 3 * 2.0 * p.chunk_q * p.h * rh,
                    "lact_update": P * n_upd * acc.ns5_flops(p.h, rh) if p.muon else 0.0}
            # apply-then-update order: the update and the same chunk's apply share one launch
            work["lact_update_apply"] = work["lact_update"] + work["lact_apply"]
            bound, peak, unit = "mfma", acc.PEAK_BF16_TFLOPS, "TFLOP/s"
            metric = ("TTT-layer tokens/sec at h=128, chunk 2048 bf16; % of bf16 MFMA peak" if k == 2 else
                      "TTT-layer tokens/sec, view-synthesis shape (h=192, 196608 context + 4096 query), bf16")
        # every token of the LM layer is both a query and a key; the scene has distinct context
        # (written) and query (read) tokens
        tokens = p.B * (p.Nk if p.Nq == p.Nk else p.Nk + p.Nq)
        cfg = {"workload": CONFIG_NAMES[k], "B": p.B, "H": p.H, "h": p.h, "r": p.r, "seq_len": p.Nk,
               "query_len": p.Nq, "chunk": p.chunk_kv,
               "order": "apply-then-update" if p.order == 0 else "update-then-apply"}
        if k != 1:
            cfg.update({"momentum": p.momentum, "muon": p.muon, "weight_norm": p.weight_norm})
        elif p.momentum:
            cfg["workload"] += f" + momentum {p.momentum:g}"
            cfg["momentum"] = p.momentum
    cfg["parallelism"] = "single GPU"

    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    ms = time_steps(step, args.steps, args.warmup, stream)
    kern = kernel_breakdown(ttt, step, args.steps)
    roof = roofline(kern, work, bound, peak, unit)
    roof["traffic"] = acc.profiled_traffic(ROOT, roof["kernel"], stem)
    out = {
        "metric": metric,
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
        "config": cfg,
        "roofline": roof,
        "step_flops": flops,
        "step_tflops": round(flops / (ms * 1e-3) / 1e12, 2),
        "step_frac_of_bf16_peak": round(flops / (ms * 1e-3) / 1e12 / acc.PEAK_BF16_TFLOPS, 4),
        "kernels": kern,
    }
    if not args.no_cpu_baseline:
        if k == 4:
            out["cpu_baseline"] = cpu_baseline_inplace(p, x, args.cpu_seconds)
        elif k == 1:
            out["cpu_baseline"] = cpu_baseline_linattn(p, x, args.cpu_seconds)
        else:
            out["cpu_baseline"] = cpu_baseline_lact(p, x, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
