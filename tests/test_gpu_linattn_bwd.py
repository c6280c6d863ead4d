"""GPU parity of ttt_linattn_backward (the scan form's gradients) against the CPU oracle's
backward, which is pinned to torch autograd. Every gradient is compared element by element at
the bf16 bar (max-abs-relative 2e-2): dQ, dK, dV, deta and the three weight gradients."""
import numpy as np
import pytest

from tests._helpers import BF16_TOL, announce, dev, host
from workloads import BF16, LactProblem, bf16_round, make_lact_inputs, max_abs_rel

pytestmark = pytest.mark.gpu

NAMES = ("dQ", "dK", "dV", "deta", "dW0", "dW2", "dW1")


def _run(lib, p, x, dO, per_seq=False):
    import torch
    W = {k: (np.stack([x[k]] * p.B) if per_seq else x[k]) for k in ("W0", "W1", "W2")}
    return lib.linattn_backward(dev(x["Q"], torch.bfloat16), dev(x["K"], torch.bfloat16), dev(x["V"], torch.bfloat16),
                                dev(x["eta"], torch.float32), dev(W["W0"], torch.float32), dev(W["W2"], torch.float32),
                                dev(W["W1"], torch.float32), dev(dO, torch.bfloat16), chunk=p.chunk_kv, order=p.order,
                                momentum=p.momentum), W


def _check(label, got, ref, sel=lambda a: a):
    errs = {k: max_abs_rel(sel(host(got[k])), sel(ref[k])) for k in NAMES}
    print(f"{label}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    for k, v in errs.items():
        assert v <= BF16_TOL, (label, k, v)


CASES = [
    ("AU h64 r2", dict(h=64, r=2, N=1024, chunk=256), 1),
    ("UA h64 r2 momentum 0.9", dict(h=64, r=2, N=1024, chunk=128, order=1, momentum=0.9), 2),
    ("AU h32 r4 ragged chunk 96", dict(h=32, r=4, N=480, chunk=96, momentum=0.5), 3),
    ("UA h32 r2 chunk 32", dict(h=32, r=2, N=256, chunk=32, order=1), 4),
    ("AU h64 r2 one chunk", dict(h=64, r=2, N=256, chunk=256), 5),
]


@pytest.mark.parametrize("label,kw,seed", CASES, ids=[c[0] for c in CASES])
def test_small_cases(lib, label, kw, seed):
    from oracle import linattn as LA
    kw = dict(kw)
    N, chunk = kw.pop("N"), kw.pop("chunk")
    p = LactProblem(B=2, H=2, Nq=N, Nk=N, chunk_q=chunk, chunk_kv=chunk, dtype=BF16, weight_norm=False, **kw)
    announce(f"linattn backward {label}")
    for variant, xs in (("plain", dict()), ("eta x100", dict(eta_scale=1.0))):
        x = make_lact_inputs(p, 800 + seed, **xs)
        dO = bf16_round(np.random.default_rng(seed).standard_normal((p.B, p.H, N, p.h)).astype(np.float32))
        got, _ = _run(lib, p, x, dO)
        ref = LA.linattn_backward(x["Q"], x["K"], x["V"], x["eta"], x["W0"], x["W1"], x["W2"], dO, chunk=chunk,
                                  order=p.order, momentum=p.momentum)
        _check(f"{label} [{variant}]", got, ref)


def test_per_sequence_weights(lib):
    from oracle import linattn as LA
    p = LactProblem(B=2, H=2, h=64, r=2, Nq=512, Nk=512, chunk_q=128, chunk_kv=128, dtype=BF16, weight_norm=False,
                    momentum=0.9)
    announce("linattn backward per-sequence weights")
    x = make_lact_inputs(p, 820)
    dO = bf16_round(np.random.default_rng(21).standard_normal((2, 2, 512, 64)).astype(np.float32))
    got, W = _run(lib, p, x, dO, per_seq=True)
    ref = LA.linattn_backward(x["Q"], x["K"], x["V"], x["eta"], W["W0"], W["W1"], W["W2"], dO, chunk=128,
                              momentum=0.9)
    assert tuple(got["dW0"].shape) == (2, 2, 64, 128)
    _check("per-sequence", got, ref)


def test_scan_workload_shape(lib):
    """The scan workload's shape (B4 H8 h64 r2, 8192 tokens, chunk 512): token gradients of three
    pairs and the weight gradients of two heads (summed over the four sequences) against the
    oracle; repeated calls bit for bit."""
    import torch
    from oracle import linattn as LA
    p = LactProblem(B=4, H=8, h=64, r=2, Nq=8192, Nk=8192, chunk_q=512, chunk_kv=512, dtype=BF16, weight_norm=False)
    announce("linattn backward scan workload B4 H8 h64 r2 N8192 chunk512")
    x = make_lact_inputs(p, 830)
    dO = bf16_round(np.random.default_rng(22).standard_normal((4, 8, 8192, 64)).astype(np.float32))
    got, _ = _run(lib, p, x, dO)
    for hd in (0, 5):
        sub = {k: x[k][:, hd:hd + 1] for k in ("Q", "K", "V", "eta")}
        ref = LA.linattn_backward(sub["Q"], sub["K"], sub["V"], sub["eta"], x["W0"][hd:hd + 1], x["W1"][hd:hd + 1],
                                  x["W2"][hd:hd + 1], dO[:, hd:hd + 1], chunk=512)
        errs = {}
        for k in ("dQ", "dK", "dV", "deta"):
            errs[k] = max_abs_rel(host(got[k])[:, hd], ref[k][:, 0])
        for k in ("dW0", "dW2", "dW1"):
            errs[k] = max_abs_rel(host(got[k])[hd], ref[k][0])
        print(f"scan workload head {hd}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
        assert all(v <= BF16_TOL for v in errs.values()), errs
    again, _ = _run(lib, p, x, dO)
    for k in NAMES:
        assert torch.equal(got[k], again[k]), k


@pytest.mark.parametrize("per_seq", [False, True])
def test_empty_sequence_gives_zero_weight_gradients(lib, per_seq):
    """No tokens: the weight gradients are exactly zero (per-sequence or shared shapes) and the
    token gradients are empty."""
    import torch
    p = LactProblem(B=2, H=2, h=64, r=2, Nq=256, Nk=256, chunk_q=128, chunk_kv=128, dtype=BF16, weight_norm=False)
    announce(f"linattn backward empty sequence per_seq={per_seq}")
    x = make_lact_inputs(p, 840)
    empty = {k: x[k][:, :, :0] for k in ("Q", "K", "V", "eta")}
    y = dict(x, **empty)
    dO = np.zeros((2, 2, 0, 64), np.float32)
    got, W = _run(lib, LactProblem(B=2, H=2, h=64, r=2, Nq=0, Nk=0, chunk_q=128, chunk_kv=128, dtype=BF16,
                                   weight_norm=False), y, dO, per_seq=per_seq)
    for k in ("dW0", "dW2", "dW1"):
        assert tuple(got[k].shape) == W[k.replace("d", "", 1)].shape
        assert not bool(got[k].any()), k
    for k in ("dQ", "dK", "dV", "deta"):
        assert got[k].numel() == 0
    torch.cuda.synchronize()
