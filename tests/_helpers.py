"""Shared helpers of the GPU parity tests: seeded inputs to device tensors, and a
printout that names each case before its GPU step runs."""
import sys

import numpy as np

BF16_TOL = 2e-2   # max|gpu - oracle| / max|oracle|, bf16 I/O
FP32_TOL = 1e-4   # same, fp32 I/O


def announce(msg: str) -> None:
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def dev(a, dtype):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0").to(dtype)


def host(t):
    return t.float().cpu().numpy()


def lact_on_gpu(ttt, p, x, **kw):
    import torch
    io = torch.bfloat16 if p.dtype == 1 else torch.float32
    args = dict(chunk_q=p.chunk_q, chunk_kv=p.chunk_kv, order=p.order, update_mask=p.update_mask,
                weight_norm=p.weight_norm, muon=p.muon, momentum=p.momentum, eps_norm=p.eps_norm,
                eps_ns=p.eps_ns)
    args.update(kw)
    return ttt.lact_forward(dev(x["Q"], io), dev(x["K"], io), dev(x["V"], io), dev(x["eta"], torch.float32),
                            dev(x["W0"], torch.float32), dev(x["W1"], torch.float32),
                            dev(x["W2"], torch.float32), **args)


def lact_oracle(p, x, pairs=None, **kw):
    from oracle import lact as L
    args = dict(chunk_q=p.chunk_q, chunk_kv=p.chunk_kv, order=p.order, update_mask=p.update_mask,
                weight_norm=p.weight_norm, muon=p.muon, momentum=p.momentum, eps_norm=p.eps_norm,
                eps_ns=p.eps_ns, pairs=pairs)
    args.update(kw)
    return L.lact_forward(x["Q"], x["K"], x["V"], x["eta"], x["W0"], x["W1"], x["W2"], **args)
