"""Re-entrancy of the C ABI: two calls issued back to back on two caller streams (so that they
may run concurrently) give bit-identical results to the same calls made one after the other.
The library keeps no per-process streams, events or scratch: each call uses only its own
workspace and the caller's stream."""
import numpy as np
import pytest

from tests._helpers import announce, dev, host
from workloads import BF16, InplaceProblem, LactProblem, make_inplace_inputs, make_lact_inputs

pytestmark = pytest.mark.gpu


def _two_ways(run, xs):
    """run(x, stream) -> tuple of tensors. Sequential on the current stream, then concurrent on
    two new streams (default priority)."""
    import torch
    seq = [tuple(host(t) for t in run(x, None) if t is not None) for x in xs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [run(x, s) for x, s in zip(xs, streams)]
    torch.cuda.synchronize()
    conc = [tuple(host(t) for t in o if t is not None) for o in outs]
    for a, b in zip(seq, conc):
        for u, v in zip(a, b):
            assert np.array_equal(u, v)


def test_inplace_concurrent_calls_match_sequential(lib):
    import torch
    p = InplaceProblem(B=1, N=512, d_model=512, d_hidden=2048, chunk=256, eta=1e-3)
    announce(f"streams: inplace {p}")
    xs = []
    for seed in (61, 62):
        x = make_inplace_inputs(p, seed)
        xs.append({k: dev(x[k], torch.bfloat16) for k in ("Hs", "W_gate", "W_up", "Vbar")} |
                  {"W_down": dev(x["W_down"], torch.float32), "eta": float(x["eta"])})
    torch.cuda.synchronize()

    def run(x, s):
        return lib.inplace_down_forward(x["Hs"], x["W_gate"], x["W_up"], x["W_down"], x["Vbar"], chunk=p.chunk,
                                        eta=x["eta"], stream=s)
    _two_ways(run, xs)


def test_linattn_concurrent_calls_match_sequential(lib):
    import torch
    p = LactProblem(B=2, H=4, h=64, r=2, Nq=2048, Nk=2048, chunk_q=512, chunk_kv=512, dtype=BF16)
    announce(f"streams: linattn {p}")
    xs = []
    for seed in (63, 64):
        x = make_lact_inputs(p, seed)
        xs.append({k: dev(x[k], torch.bfloat16) for k in ("Q", "K", "V")} |
                  {k: dev(x[k], torch.float32) for k in ("eta", "W0", "W1", "W2")})
    torch.cuda.synchronize()

    def run(x, s):
        return lib.linattn_forward(x["Q"], x["K"], x["V"], x["eta"], x["W0"], x["W2"], x["W1"], chunk=p.chunk_kv,
                                   stream=s)
    _two_ways(run, xs)


def test_lact_concurrent_calls_match_sequential(lib):
    import torch
    p = LactProblem(B=1, H=4, h=128, r=2, Nq=1024, Nk=1024, chunk_q=256, chunk_kv=256, dtype=BF16, muon=True,
                    momentum=0.9, v_normalised=False)
    announce(f"streams: lact {p}")
    xs = []
    for seed in (65, 66):
        x = make_lact_inputs(p, seed)
        xs.append({k: dev(x[k], torch.bfloat16) for k in ("Q", "K", "V")} |
                  {k: dev(x[k], torch.float32) for k in ("eta", "W0", "W1", "W2")})
    torch.cuda.synchronize()

    def run(x, s):
        return lib.lact_forward(x["Q"], x["K"], x["V"], x["eta"], x["W0"], x["W1"], x["W2"], chunk_q=p.chunk_q,
                                muon=True, momentum=0.9, stream=s)
    _two_ways(run, xs)
