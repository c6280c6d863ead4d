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
update instead (--config 1 --feature-map identity: the scan with one linear fast-weight layer,
an h x h state; --config 1 --backward, --config 4 --backward: the gradients of the scan form,
of the In-Place update). The default run (the LM layer) also measures those workloads and adds
them to its JSON line under "other_workloads" (--no-extras skips them). The scan workload's
136 MB fit in the 256 MB last-level cache, so it is timed both warm and with a 512 MB buffer
read between repetitions (flushed; its headline figure).
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
    ap.add_argument("--feature-map", default="swiglu", choices=["swiglu", "identity"],
                    help="scan workload only: the identity map is one linear fast-weight layer (h x h state)")
    ap.add_argument("--backward", action="store_true",
                    help="scan workload and In-Place update: time the backward (gradients of every input) instead")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one plain 256 MiB device-to-device copy (reference for HBM byte counters)")
    ap.add_argument("--no-extras", action="store_true",
                    help="default run: do not measure the other workloads")
    return ap.parse_args()


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def blas_vendor():
    """The BLAS library NumPy uses (name and version), as threadpoolctl reports it."""
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        return ", ".join(f"{i.get('internal_api')} {i.get('version')}" for i in libs) or "unknown"
    except Exception:  # pragma: no cover
        return "unknown"


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
            "blas": blas_vendor(),
            "sample": f"{done} of {len(pairs)} (sequence, head) pairs, all {p.Nk // p.chunk_kv} chunks each, "
                      f"float32 NumPy oracle, {el:.1f} s"}


def cpu_baseline_linattn(p, x, budget_s, feature_map="swiglu"):
    import numpy as np
    from oracle import linattn as LA
    done, t0 = 0, time.perf_counter()
    pairs = [(b, h) for b in range(p.B) for h in range(p.H)]
    ident = feature_map == "identity"
    for (b, h) in pairs:
        LA.linattn_pair(x["Q"][b, h], x["K"][b, h], x["V"][b, h], x["eta"][b, h], None if ident else x["W0"][h],
                        x["W1"][h], None if ident else x["W2"][h], chunk=p.chunk_kv, order=p.order,
                        momentum=p.momentum, feature_map=feature_map, dtype=np.float32)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": round(done * p.Nk / p.H / el, 1), "unit": "tokens/s", "cores": int(blas_threads()),
            "kind": "oracle", "blas": blas_vendor(),
            "sample": f"{done} of {len(pairs)} pairs, float32 NumPy oracle, {el:.1f} s"}


def cpu_baseline_linattn_backward(p, x, budget_s):
    import numpy as np
    from oracle import linattn as LA
    dO = np.random.default_rng(11).standard_normal(x["Q"].shape[2:]).astype(np.float32)
    done, t0 = 0, time.perf_counter()
    pairs = [(b, h) for b in range(p.B) for h in range(p.H)]
    for (b, h) in pairs:
        LA.linattn_backward_pair(x["Q"][b, h], x["K"][b, h], x["V"][b, h], x["eta"][b, h], x["W0"][h], x["W1"][h],
                                 x["W2"][h], dO, chunk=p.chunk_kv, order=p.order, momentum=p.momentum,
                                 dtype=np.float32)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": round(done * p.Nk / p.H / el, 1), "unit": "tokens/s", "cores": int(blas_threads()),
            "kind": "oracle", "blas": blas_vendor(),
            "sample": f"{done} of {len(pairs)} pairs, float32 NumPy oracle backward, {el:.1f} s"}


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
            "kind": "oracle", "blas": blas_vendor(),
            "sample": f"first {done} of {p.N // p.chunk} chunks, float32 NumPy oracle, {el:.1f} s"}


def cpu_baseline_inplace_backward(p, x, n_chunks=4):
    """The oracle's backward over the first n_chunks chunks of the sequence, taken as a sequence
    of its own (the backward's work per chunk does not depend on the sequence length)."""
    import numpy as np
    from oracle import inplace as IP
    T = n_chunks * p.chunk
    dO = np.random.default_rng(12).standard_normal((T, p.d_model)).astype(np.float32)
    t0 = time.perf_counter()
    IP.inplace_backward_sequence(x["Hs"][0, :T], x["W_gate"], x["W_up"], x["W_down"], x["Vbar"][0, :T],
                                 float(x["eta"]), dO, chunk=p.chunk, dtype=np.float32)
    el = time.perf_counter() - t0
    return {"value": round(T / el, 1), "unit": "tokens/s", "cores": int(blas_threads()), "kind": "oracle",
            "blas": blas_vendor(),
            "sample": f"backward of the first {n_chunks} of {p.N // p.chunk} chunks as one sequence, float32 "
                      f"NumPy oracle, {el:.1f} s"}


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


def flush_buffer(flush_bytes):
    import torch
    return torch.ones(flush_bytes // 4, dtype=torch.float32, device="cuda:0") if flush_bytes else None


def flush(buf):
    """Read a buffer larger than the last-level cache (256 MB): the cache then holds none of
    the step's inputs and no dirty lines of the flush itself (a written flush buffer would leave
    its write-backs to the timed step)."""
    buf.max()


def time_steps_flushed(step, steps, stream, flush_bytes=512 << 20):
    """Each step timed alone after a 512 MB read pass, so that the step's inputs come from HBM;
    returns the mean step time in ms."""
    import torch
    buf = flush_buffer(flush_bytes)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    step()
    for i in range(steps):
        flush(buf)
        evs[i][0].record(stream)
        step()
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    del buf
    return sum(a.elapsed_time(b) for a, b in evs) / steps


def kernel_breakdown(ttt, step, steps, flush_bytes=0):
    """Per kernel class: launches and average launch time. The hot kernels are launched with
    start/stop events attached to the dispatch itself (the kernel's own begin and end
    timestamps, the figures a kernel trace reports); see ttt_timing_enable in the C header.
    With flush_bytes a buffer that large is read before every step."""
    import torch
    buf = flush_buffer(flush_bytes)
    torch.cuda.synchronize()
    ttt.timing_collect()
    ttt.timing_enable(True)
    try:
        for i in range(steps):
            if buf is not None:
                flush(buf)
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

DTYPES = {
    "lact": "bf16 I/O; fp16 MFMA operands for the per-chunk products; split-bf16 Newton-Schulz; fp32 accumulate/state",
    "linattn": "bf16 I/O; fp16 MFMA operands; fp32 accumulate/state",
    "inplace": "bf16 I/O and MFMA operands; fp32 accumulate and W_down state",
}


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


def measure(k, args, momentum=0.0, cpu=True, feature_map="swiglu", backward=False):
    """One workload: its JSON record (without the fields common to every line)."""
    import numpy as np
    import torch
    import linear_attention_lact_amd as ttt
    from linear_attention_lact_amd import accounting as acc
    from workloads import CONFIGS, CONFIG_NAMES, make_inplace_inputs, make_lact_inputs

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dev, dt)
    p = CONFIGS[k]
    stem = PROFILE_STEMS[k]
    flush_bytes = 0
    if momentum != 0.0:
        from dataclasses import replace
        p = replace(p, momentum=momentum)
        stem = "linattn_scan_momentum_b4h8_h64_seq8192_chunk512"
    ident = k == 1 and feature_map == "identity"
    if ident:
        from dataclasses import replace
        p = replace(p, r=1)
        stem = "linattn_identity_b4h8_h64_seq8192_chunk512" + ("_momentum" if momentum else "")
    if k == 1 and backward:
        stem = "linattn_backward_b4h8_h64_seq8192_chunk512"
    if k == 4:
        x = make_inplace_inputs(p, k)
        Hs, Wg, Wu, Vb = (t(x[n], torch.bfloat16) for n in ("Hs", "W_gate", "W_up", "Vbar"))
        Wd = t(x["W_down"], torch.float32)

        per = 2.0 * p.chunk * p.d_model * p.d_hidden  # one chunk-sized product
        work = {"inplace_z": 2 * per, "inplace_apply": per, "inplace_update": per, "inplace_apply_z": 3 * per}
        if backward:
            nch = p.N // p.chunk
            # per launch, averaged over a step: dZ is two products but one for the last chunk
            # (no later chunk); the apply class holds dVbar (one product, all chunks but the last)
            # and dH (two products); the weight gradients are one product over all chunks each
            work.update({"inplace_swiglu_bwd": (2 * (nch - 1) + 1) * per / nch,
                         "inplace_apply": ((nch - 1) + 2 * nch) * per / (2 * nch - 1),
                         "inplace_wgrad": nch * per})
            dO = t(np.random.default_rng(12).standard_normal(x["Hs"].shape).astype(np.float32), torch.bfloat16)
            stem = "inplace_backward_d4096_dh14336_seq32768_chunk1024"

            def step():
                return ttt.inplace_down_backward(Hs, Wg, Wu, Wd, Vb, dO, chunk=p.chunk, eta=float(x["eta"]),
                                                 stream=stream)
            flops = acc.inplace_backward_flops(p.B, p.N, p.d_model, p.d_hidden)
            metric = "In-Place TTT W_down update backward tokens/sec (d_model 4096, d_hidden 14336, chunk 1024), bf16"
        else:
            def step():
                return ttt.inplace_down_forward(Hs, Wg, Wu, Wd, Vb, chunk=p.chunk, eta=float(x["eta"]),
                                                stream=stream)
            flops = acc.inplace_flops(p.B, p.N, p.d_model, p.d_hidden)
            metric = "In-Place TTT W_down update tokens/sec (d_model 4096, d_hidden 14336, chunk 1024), bf16"
        tokens = p.B * p.N
        bound, peak, unit = "mfma", acc.PEAK_BF16_TFLOPS, "TFLOP/s"
        cfg = {"workload": CONFIG_NAMES[4] + (", backward" if backward else ""), "B": p.B, "seq_len": p.N,
               "d_model": p.d_model, "d_hidden": p.d_hidden, "chunk": p.chunk, "eta": p.eta}
        if backward:
            cfg["pass"] = "backward"
        dtype = DTYPES["inplace"]
    else:
        x = make_lact_inputs(p, k)
        io = torch.bfloat16 if p.dtype == 1 else torch.float32
        Q, K, V = (t(x[n], io) for n in ("Q", "K", "V"))
        eta = t(x["eta"], torch.float32)
        W0, W1, W2 = (t(x[n], torch.float32) for n in ("W0", "W1", "W2"))
        if k == 1 and backward:
            dO = t(np.random.default_rng(11).standard_normal(x["Q"].shape).astype(np.float32), io)

            def step():
                return ttt.linattn_backward(Q, K, V, eta, W0, W2, W1, dO, chunk=p.chunk_kv, order=p.order,
                                            momentum=p.momentum, stream=stream)
            flops = acc.linattn_backward_flops(p.B, p.H, p.Nk, p.h, p.r)
            P, rh = p.B * p.H, p.rh
            unit_p = P * 2.0 * p.Nk * p.h * rh  # one product of 2 N h rh over all pairs
            # per launch: the aggregate kernel (phi and one contraction: 3 products), the token
            # kernels (query side 7, key side 8: 7.5 on average)
            work = {"linattn_delta": 3 * unit_p, "linattn_apply": 7.5 * unit_p}
            bound, peak, unit = "mfma", acc.PEAK_BF16_TFLOPS, "TFLOP/s"
            metric = "linear-attention scan form backward tokens/sec (h=64, r=2, chunk 512), bf16"
            dtype = DTYPES["linattn"]
        elif k == 1:
            fw0, fw2 = (None, None) if ident else (W0, W2)

            def step():
                return ttt.linattn_forward(Q, K, V, eta, fw0, fw2, W1, chunk=p.chunk_kv, order=p.order,
                                           momentum=p.momentum, feature_map=feature_map, stream=stream)
            if ident:
                flops = acc.linattn_identity_flops(p.B, p.H, p.Nk, p.h)
                nbytes = acc.linattn_identity_bytes(p.B, p.H, p.Nk, p.h)
            else:
                flops = acc.linattn_flops(p.B, p.H, p.Nk, p.h, p.r)
                nbytes = acc.linattn_bytes(p.B, p.H, p.Nk, p.h, p.r)
            P, rh, nch = p.B * p.H, p.rh, p.Nk // p.chunk_kv
            work = {"linattn_delta": P * 2.0 * p.Nk * p.h * 2 + P * p.Nk * 4 + P * nch * rh * p.h * 4,
                    "linattn_scan": P * nch * rh * p.h * (4 + 2),
                    "linattn_apply": P * p.Nk * p.h * 2 * 2 + P * nch * rh * p.h * 2,
                    "linattn_fused": nbytes}
            bound, peak, unit = "hbm", acc.PEAK_HBM_GBS, "GB/s"
            metric = "linear-attention scan form tokens/sec (h=64, r=2, chunk 512), bf16; % of HBM roofline"
            if ident:
                metric = ("linear-attention scan form, identity feature map (h x h state, h=64, chunk 512), "
                          "bf16; % of HBM roofline")
            if p.momentum:
                metric = metric.replace("scan form", f"scan form with momentum {p.momentum:g}")
            flush_bytes = 512 << 20
            dtype = DTYPES["linattn"]
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
            dtype = DTYPES["lact"]
        # every token of the LM layer is both a query and a key; the scene has distinct context
        # (written) and query (read) tokens
        tokens = p.B * (p.Nk if p.Nq == p.Nk else p.Nk + p.Nq)
        cfg = {"workload": CONFIG_NAMES[k], "B": p.B, "H": p.H, "h": p.h, "r": p.r, "seq_len": p.Nk,
               "query_len": p.Nq, "chunk": p.chunk_kv,
               "order": "apply-then-update" if p.order == 0 else "update-then-apply"}
        if k != 1:
            cfg.update({"momentum": p.momentum, "muon": p.muon, "weight_norm": p.weight_norm})
        else:
            if ident:
                cfg["workload"] += ", identity feature map"
                cfg["feature_map"] = "identity"
            if backward:
                cfg["workload"] += ", backward"
                cfg["pass"] = "backward"
            if p.momentum:
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
    ms_warm = time_steps(step, args.steps, args.warmup, stream)
    ms = time_steps_flushed(step, args.steps, stream, flush_bytes) if flush_bytes else ms_warm
    kern = kernel_breakdown(ttt, step, args.steps, flush_bytes)
    roof = roofline(kern, work, bound, peak, unit)
    roof["traffic"] = acc.profiled_traffic(ROOT, roof["kernel"], stem)
    # the same class's average duration in the committed rocprofv3 profile (the profiler slows the
    # kernels a little): its roofline fraction beside the live one
    prof_us = acc.profiled_avg_us(ROOT, roof["kernel"], stem)
    if prof_us:
        scale = 1e12 if unit == "TFLOP/s" else 1e9
        roof["profiled_avg_us"] = round(prof_us, 3)
        roof["frac_profiled"] = round(roof["work_per_launch"] / (prof_us * 1e-6) / scale / peak, 4)
    rec = {"metric": metric, "value": round(tokens / (ms * 1e-3), 1), "unit": "tokens/s", "ms_per_step": round(ms, 4),
           "dtype": dtype, "config": cfg, "roofline": roof, "step_flops": flops,
           "step_tflops": round(flops / (ms * 1e-3) / 1e12, 2),
           "step_frac_of_bf16_peak": round(flops / (ms * 1e-3) / 1e12 / acc.PEAK_BF16_TFLOPS, 4), "kernels": kern}
    if flush_bytes:
        rec["timing"] = f"flushed: a {flush_bytes >> 20} MiB buffer read before each timed step"
        rec["warm"] = {"ms_per_step": round(ms_warm, 4), "value": round(tokens / (ms_warm * 1e-3), 1)}
    if cpu:
        if k == 4 and backward:
            rec["cpu_baseline"] = cpu_baseline_inplace_backward(p, x)
        elif k == 4:
            rec["cpu_baseline"] = cpu_baseline_inplace(p, x, args.cpu_seconds)
        elif k == 1 and backward:
            rec["cpu_baseline"] = cpu_baseline_linattn_backward(p, x, args.cpu_seconds)
        elif k == 1:
            rec["cpu_baseline"] = cpu_baseline_linattn(p, x, args.cpu_seconds, feature_map)
        else:
            rec["cpu_baseline"] = cpu_baseline_lact(p, x, args.cpu_seconds)
    return rec


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the layer's "
              "(sequence, head) pairs shard across GPUs without communication, see DESIGN.md",
              file=sys.stderr)
        sys.exit(2)
    if (args.momentum != 0.0 or args.feature_map != "swiglu") and args.config != 1:
        print("--momentum and --feature-map apply to the scan workload (--config 1) only", file=sys.stderr)
        sys.exit(2)
    if args.backward and args.config not in (1, 4):
        print("--backward applies to the scan workload (--config 1) and the In-Place update (--config 4)",
              file=sys.stderr)
        sys.exit(2)
    if args.backward and args.feature_map != "swiglu":
        print("--backward is built for the SwiGLU feature map", file=sys.stderr)
        sys.exit(2)
    import linear_attention_lact_amd as ttt
    ttt.load()
    rec = measure(args.config, args, args.momentum, cpu=not args.no_cpu_baseline, feature_map=args.feature_map,
                  backward=args.backward)
    out = {"metric": rec.pop("metric"), "value": rec.pop("value"), "unit": rec.pop("unit"), "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": rec.pop("ms_per_step"),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": rec.pop("dtype"),
           "data": "synthetic", "config": rec.pop("config"), "roofline": rec.pop("roofline")}
    if "cpu_baseline" in rec:
        out["cpu_baseline"] = rec.pop("cpu_baseline")
    out.update(rec)
    if args.config == 2 and not args.no_extras:
        others = {}
        for k, fm, bwd in ((1, "swiglu", False), (1, "identity", False), (1, "swiglu", True), (3, "swiglu", False),
                           (4, "swiglu", False), (4, "swiglu", True)):
            r = measure(k, args, cpu=False, feature_map=fm, backward=bwd)
            others[r["config"]["workload"]] = {
                "metric": r["metric"], "value": r["value"], "unit": r["unit"], "ms_per_step": r["ms_per_step"],
                "roofline": {key: r["roofline"][key] for key in ("bound", "kernel", "achieved", "peak", "unit", "frac")},
                **({"warm": r["warm"], "timing": r["timing"]} if "warm" in r else {})}
        out["other_workloads"] = others
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
