"""GPU parity of ttt_lact_forward for heads wider than 192 (the LaCT notes' own d = 768 defaults),
which run the composed path (fp16 products, tiled Newton-Schulz), against the CPU oracle at the
bf16 bar (max-abs-relative 2e-2); every output is compared: O, the final fast weights and the
final momentum."""
import numpy as np
import pytest

from tests._helpers import BF16_TOL, announce, lact_on_gpu, lact_oracle
from tests.test_gpu_lact import _compare
from workloads import BF16, LactProblem, UPD_W1, make_lact_inputs

pytestmark = pytest.mark.gpu

CASES = [
    # (label, problem kwargs, input variant, seed)
    ("h256 r2 AU muon mom renorm", dict(B=1, H=2, h=256, r=2, N=512, chunk=128, muon=True, momentum=0.9), {}, 1),
    ("h256 r1 UA sgd", dict(B=1, H=2, h=256, r=1, N=512, chunk=256, order=1), {}, 2),
    ("h384 r2 AU W1 only eta x100", dict(B=2, H=1, h=384, r=2, N=256, chunk=128, update_mask=UPD_W1),
     dict(eta_scale=1.0), 3),
    ("h768 r1 AU muon mom renorm", dict(B=1, H=1, h=768, r=1, N=512, chunk=256, muon=True, momentum=0.9), {}, 4),
    ("h768 r2 UA muon", dict(B=1, H=1, h=768, r=2, N=256, chunk=128, muon=True, order=1), {}, 5),
    # the view-synthesis pattern: one write from every context token, then the queries (UA)
    ("h256 r2 UA scene 1024 context 128 queries",
     dict(B=1, H=2, h=256, r=2, N=1024, chunk=1024, Nq=128, chunk_q=128, muon=True, order=1), {}, 6),
]


@pytest.mark.parametrize("label,kw,xs,seed", CASES, ids=[c[0] for c in CASES])
def test_wide_heads(lib, label, kw, xs, seed):
    kw = dict(kw)
    N, chunk = kw.pop("N"), kw.pop("chunk")
    Nq, chunk_q = kw.pop("Nq", N), kw.pop("chunk_q", chunk)
    base = dict(Nq=Nq, Nk=N, chunk_q=chunk_q, chunk_kv=chunk, dtype=BF16, v_normalised=False)
    base.update(kw)
    p = LactProblem(**base)
    announce(f"lact wide heads {label}")
    x = make_lact_inputs(p, 1100 + seed, **xs)
    gpu = lact_on_gpu(lib, p, x)
    ref = lact_oracle(p, x)
    _compare(gpu, ref, BF16_TOL, label=label)


def test_wide_heads_repeat_bitwise(lib):
    import torch
    p = LactProblem(B=1, H=2, h=256, r=2, Nq=256, Nk=256, chunk_q=128, chunk_kv=128, dtype=BF16, muon=True,
                    momentum=0.9, v_normalised=False)
    announce("lact wide heads h256 repeat")
    x = make_lact_inputs(p, 1120)
    a, b = lact_on_gpu(lib, p, x), lact_on_gpu(lib, p, x)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_wide_heads_per_sequence_weights_and_initial_momentum(lib):
    """Per-sequence fast weights and a given initial momentum on the composed path (h 256)."""
    import torch
    from tests._helpers import dev, host
    from oracle import lact as Lo
    from workloads import max_abs_rel
    p = LactProblem(B=2, H=1, h=256, r=2, Nq=256, Nk=256, chunk_q=128, chunk_kv=128, dtype=BF16, muon=True,
                    momentum=0.9, v_normalised=False)
    announce("lact wide heads h256 per-sequence weights, initial momentum")
    x = make_lact_inputs(p, 1130)
    rng = np.random.default_rng(31)
    W = {k: np.stack([x[k] * (1.0 + 0.2 * b) for b in range(2)]).astype(np.float32) for k in ("W0", "W1", "W2")}
    n = p.h * p.rh
    M = (0.01 * rng.standard_normal((2, 1, 3, n))).astype(np.float32)
    io = torch.bfloat16
    O, W0o, W1o, W2o, Mo = lib.lact_forward(
        dev(x["Q"], io), dev(x["K"], io), dev(x["V"], io), dev(x["eta"], torch.float32), dev(W["W0"], torch.float32),
        dev(W["W1"], torch.float32), dev(W["W2"], torch.float32), M_in=dev(M, torch.float32), chunk_q=128,
        chunk_kv=128, order=0, update_mask=7, weight_norm=True, muon=True, momentum=0.9, eps_norm=p.eps_norm,
        eps_ns=p.eps_ns)
    Md = {"W0": M[:, :, 0].reshape(2, 1, p.h, p.rh), "W1": M[:, :, 1].reshape(2, 1, p.rh, p.h),
          "W2": M[:, :, 2].reshape(2, 1, p.h, p.rh)}
    ref = Lo.lact_forward(x["Q"], x["K"], x["V"], x["eta"], W["W0"], W["W1"], W["W2"], chunk_q=128, chunk_kv=128,
                          order=0, update_mask=7, weight_norm=True, muon=True, momentum=0.9, eps_norm=p.eps_norm,
                          eps_ns=p.eps_ns, M_in=Md)
    errs = dict(O=max_abs_rel(host(O), ref["O"]), W0=max_abs_rel(host(W0o), ref["W0"]),
                W1=max_abs_rel(host(W1o), ref["W1"]), W2=max_abs_rel(host(W2o), ref["W2"]))
    Mh = host(Mo)
    for i in range(3):
        errs[f"M{i}"] = max_abs_rel(Mh[:, :, i].reshape(ref[f"M{i}"].shape), ref[f"M{i}"])
    print("per-sequence: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    assert all(v <= BF16_TOL for v in errs.values()), errs
