"""GPU parity of the scan form with the identity feature map (one linear fast-weight layer,
h x h state: the summary page's simplification ladder, step 3) against the CPU oracle.

Every case runs three input variants, as the other scan tests do: the configs' own
distributions, step sizes x100 (the state update then dominates the outputs) and a zero initial
state (the outputs are the update alone)."""
import numpy as np
import pytest

from tests._helpers import BF16_TOL, announce, dev, host
from workloads import BF16, LactProblem, make_lact_inputs, max_abs_rel

pytestmark = pytest.mark.gpu


def _problem(B=2, H=2, h=64, N=1024, chunk=256, order=0, momentum=0.0):
    return LactProblem(B=B, H=H, h=h, r=1, Nq=N, Nk=N, chunk_q=chunk, chunk_kv=chunk, dtype=BF16,
                       order=order, momentum=momentum, weight_norm=False)


def _gpu(lib, p, x):
    import torch
    return lib.linattn_forward(dev(x["Q"], torch.bfloat16), dev(x["K"], torch.bfloat16),
                               dev(x["V"], torch.bfloat16), dev(x["eta"], torch.float32), None, None,
                               dev(x["W1"], torch.float32), chunk=p.chunk_kv, order=p.order,
                               momentum=p.momentum, feature_map="identity")


def _ref(p, x, pairs=None):
    from oracle import linattn as LA
    return LA.linattn_forward(x["Q"], x["K"], x["V"], x["eta"], None, x["W1"], None, chunk=p.chunk_kv,
                              order=p.order, momentum=p.momentum, feature_map="identity", pairs=pairs)


def _check(lib, p, x, label, pairs=None):
    O, S = _gpu(lib, p, x)
    ref = _ref(p, x, pairs)
    if pairs is None:
        eo, es = max_abs_rel(host(O), ref["O"]), max_abs_rel(host(S), ref["S"])
    else:
        sel = lambda a: np.stack([a[b, hd] for b, hd in pairs])
        eo, es = max_abs_rel(sel(host(O)), sel(ref["O"])), max_abs_rel(sel(host(S)), sel(ref["S"]))
    print(f"{label} O={eo:.2e} S={es:.2e}", flush=True)
    assert eo <= BF16_TOL and es <= BF16_TOL, (label, eo, es)
    return O, S


CASES = [
    ("AU h64", dict(h=64, N=1024, chunk=256), 1),
    ("UA h64 momentum 0.9", dict(h=64, N=1024, chunk=128, order=1, momentum=0.9), 2),
    ("AU h128", dict(h=128, N=1024, chunk=256), 3),
    ("UA h128 one tile", dict(h=128, N=512, chunk=64, order=1), 4),
    ("AU h128 momentum 0.5", dict(h=128, N=1024, chunk=128, momentum=0.5), 5),
    ("AU h64 chunk shorter than a tile", dict(h=64, N=320, chunk=32), 6),
    ("UA h64 chunk 160", dict(h=64, N=640, chunk=160, order=1), 7),
    ("AU h64 three pairs", dict(B=1, H=3, h=64, N=512, chunk=128), 8),
]


@pytest.mark.parametrize("label,kw,seed", CASES, ids=[c[0] for c in CASES])
def test_small_cases(lib, label, kw, seed):
    p = _problem(**kw)
    announce(f"identity {label}")
    for variant, xs in (("plain", dict()), ("eta x100", dict(eta_scale=1.0)), ("W1=0", dict(w1_zero=True))):
        x = make_lact_inputs(p, 700 + seed, **xs)
        _check(lib, p, x, f"{label} [{variant}]")


@pytest.mark.parametrize("momentum", [0.0, 0.9])
@pytest.mark.parametrize("order", [0, 1])
def test_grouped_chunks_many_pairs(lib, order, momentum):
    """64 pairs x 16 chunks: four chunks per workgroup; sampled pairs."""
    p = _problem(B=8, H=8, h=64, N=4096, chunk=256, order=order, momentum=momentum)
    announce(f"identity grouped B8 H8 h64 N4096 chunk256 order={order} momentum={momentum}")
    x = make_lact_inputs(p, 720 + order)
    _check(lib, p, x, "grouped", pairs=[(0, 0), (3, 5), (7, 7)])


def test_eight_chunks_per_workgroup(lib):
    """32 pairs x 64 chunks of 256 tokens: the largest group (eight chunks per workgroup)."""
    p = _problem(B=4, H=8, h=64, N=16384, chunk=256, order=1)
    announce("identity eight chunks per workgroup B4 H8 h64 N16384 chunk256 UA")
    x = make_lact_inputs(p, 730)
    _check(lib, p, x, "eight per group", pairs=[(0, 1), (3, 7)])


@pytest.mark.parametrize("h,momentum", [(64, 0.0), (64, 0.9), (128, 0.0), (128, 0.9)])
def test_scan_workload_shape(lib, h, momentum):
    """The scan workload's shape (B4 H8, 8192 tokens, chunk 512) with an h x h state: sampled
    pairs against the oracle, then repeated calls bit for bit."""
    p = _problem(B=4, H=8, h=h, N=8192, chunk=512, momentum=momentum)
    announce(f"identity scan workload B4 H8 h{h} N8192 chunk512 momentum={momentum}")
    x = make_lact_inputs(p, 740 + h)
    O, S = _check(lib, p, x, f"h{h} full size", pairs=[(0, 0), (1, 3), (3, 7)])
    for _ in range(2):
        O2, S2 = _gpu(lib, p, x)
        assert np.array_equal(host(O2), host(O)) and np.array_equal(host(S2), host(S))


def test_token_chunks_are_causal_linear_attention(lib):
    """Chunks of 32 tokens, update-then-apply, against the oracle's token-level form: the state a
    chunk reads includes its own writes."""
    p = _problem(B=1, H=2, h=64, N=256, chunk=32, order=1)
    announce("identity UA chunk32")
    x = make_lact_inputs(p, 750)
    _check(lib, p, x, "UA chunk 32")
