"""GPU parity of ttt_lact_forward against the CPU oracle (element by element, same seeded
inputs). Tolerance: max-abs-relative 1e-4 in fp32 mode, 2e-2 in bf16 mode."""
import numpy as np
import pytest

from tests._helpers import BF16_TOL, FP32_TOL, announce, host, lact_on_gpu, lact_oracle
from workloads import (BF16, CONFIGS, FP32, LactProblem, UPD_ALL, UPD_W0, UPD_W1, UPD_W2,
                       make_lact_inputs, max_abs_rel)

pytestmark = pytest.mark.gpu


def _compare(gpu, ref, tol, pairs=None, label=""):
    """Every output of the call against the oracle: O, the final fast weights and the final
    momentum (M_out [B,H,3,h*rh] holds W0 [h,rh], W1 [rh,h], W2 [h,rh] in row form)."""
    O, W0, W1, W2, M = gpu
    errs = {}
    sel = (lambda a: a) if pairs is None else (lambda a: np.stack([a[b, h] for b, h in pairs]))
    errs["O"] = max_abs_rel(sel(host(O)), sel(ref["O"]))
    for name, g in (("W0", W0), ("W1", W1), ("W2", W2)):
        errs[name] = max_abs_rel(sel(host(g)), sel(ref[name]))
    Mh = host(M)
    for i, name in enumerate(("M0", "M1", "M2")):
        m = sel(Mh[:, :, i].reshape(ref[name].shape))
        r = sel(ref[name])
        if np.max(np.abs(r)) == 0.0:  # no momentum, or a matrix outside the update mask
            assert np.all(m == 0.0), (label, name)
        else:
            errs[name] = max_abs_rel(m, r)
    print(f"{label} errors: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    for k, v in errs.items():
        assert v <= tol, (label, k, v)
    return errs


def test_config0_fp32_full(lib):
    p = CONFIGS[0]
    announce("lact config0 fp32 B1 H2 h32 r2 N256 chunk64")
    x = make_lact_inputs(p, 0)
    gpu = lact_on_gpu(lib, p, x)
    ref = lact_oracle(p, x)
    _compare(gpu, ref, FP32_TOL, label="config0")
    # momentum buffers too (zero here: no momentum)
    assert np.all(host(gpu[4]) == 0)


CASES = [
    # (label, problem kwargs, seed)
    ("bf16 AU sgd renorm h64", dict(h=64, Nq=512, Nk=512, chunk_q=128, chunk_kv=128), 1),
    ("bf16 AU muon mom renorm h128", dict(h=128, Nq=1024, Nk=1024, chunk_q=256, chunk_kv=256, muon=True, momentum=0.9), 2),
    ("bf16 UA muon renorm h64", dict(h=64, Nq=512, Nk=512, chunk_q=128, chunk_kv=128, muon=True, order=1), 3),
    ("bf16 AU mom no-renorm h32", dict(h=32, Nq=384, Nk=384, chunk_q=96, chunk_kv=96, momentum=0.5, weight_norm=False), 4),
    ("bf16 W1-only h64", dict(h=64, Nq=512, Nk=512, chunk_q=128, chunk_kv=128, update_mask=UPD_W1, weight_norm=False), 5),
    ("bf16 W0|W2 muon h96", dict(h=96, Nq=384, Nk=384, chunk_q=192, chunk_kv=192, update_mask=UPD_W0 | UPD_W2, muon=True), 6),
    ("bf16 ragged tile chunk 80 h64", dict(h=64, Nq=320, Nk=320, chunk_q=80, chunk_kv=80, muon=True, momentum=0.9), 7),
    ("bf16 h192 r2 muon UA", dict(h=192, Nq=256, Nk=1024, chunk_q=128, chunk_kv=512, muon=True, order=1), 8),
    ("bf16 h160 r2", dict(h=160, r=2, Nq=256, Nk=256, chunk_q=128, chunk_kv=128, muon=True), 9),
    ("bf16 single chunk UA", dict(h=64, Nq=256, Nk=256, chunk_q=256, chunk_kv=256, muon=True, order=1), 10),
    ("fp32 h64 muon mom", dict(h=64, Nq=256, Nk=256, chunk_q=64, chunk_kv=64, dtype=FP32, muon=True, momentum=0.9), 11),
    ("fp32 h32 UA ragged", dict(h=32, Nq=200, Nk=200, chunk_q=40, chunk_kv=40, dtype=FP32, order=1, momentum=0.9), 12),
    # as many chunks as the LM and tiny workloads have (16), with Muon and momentum, in fp32
    ("fp32 h64 muon mom 16 chunks", dict(h=64, Nq=1024, Nk=1024, chunk_q=64, chunk_kv=64, dtype=FP32, muon=True,
                                         momentum=0.9), 13),
    ("fp32 h32 muon mom renorm 16 chunks UA", dict(h=32, Nq=1024, Nk=1024, chunk_q=64, chunk_kv=64, dtype=FP32,
                                                   muon=True, momentum=0.9, order=1), 14),
    # larger chunks with pair counts that do not fill the XCDs evenly (4, 6, 12 pairs)
    ("bf16 h128 chunk 512", dict(h=128, Nq=2048, Nk=2048, chunk_q=512, chunk_kv=512, muon=True,
                                               momentum=0.9), 15),
    ("bf16 h64 chunk 1024 6 pairs", dict(B=2, H=3, h=64, Nq=4096, Nk=4096, chunk_q=1024,
                                                       chunk_kv=1024, muon=True, momentum=0.9), 16),
    ("bf16 h128 sgd 12 pairs", dict(B=3, H=4, h=128, Nq=2048, Nk=2048, chunk_q=1024, chunk_kv=1024,
                                                  momentum=0.5), 17),
    # every (h, rh) instance of the LDS-resident Newton-Schulz update: its upper-triangle task
    # tables differ at h = 32 (one block), 64 (three), 96 (six) and 128 (ten)
    ("bf16 h32 r2 muon mom", dict(h=32, Nq=512, Nk=512, chunk_q=128, chunk_kv=128, muon=True, momentum=0.9), 18),
    ("bf16 h32 r4 muon UA", dict(h=32, r=4, Nq=512, Nk=512, chunk_q=128, chunk_kv=128, muon=True, order=1), 19),
    ("bf16 h64 r4 muon mom", dict(h=64, r=4, Nq=512, Nk=512, chunk_q=128, chunk_kv=128, muon=True, momentum=0.9), 20),
    ("bf16 h96 r4 muon mom", dict(h=96, r=4, Nq=768, Nk=768, chunk_q=192, chunk_kv=192, muon=True, momentum=0.9), 21),
    ("bf16 h96 r2 muon all", dict(h=96, Nq=768, Nk=768, chunk_q=192, chunk_kv=192, muon=True), 22),
]


@pytest.mark.parametrize("label,kw,seed", CASES, ids=[c[0] for c in CASES])
def test_small_cases(lib, label, kw, seed):
    base = dict(B=2, H=2, h=64, r=2, dtype=BF16, v_normalised=False)
    base.update(kw)
    p = LactProblem(**base)
    announce(f"lact {label}: {p}")
    x = make_lact_inputs(p, 100 + seed)
    gpu = lact_on_gpu(lib, p, x)
    ref = lact_oracle(p, x)
    _compare(gpu, ref, BF16_TOL if p.dtype == BF16 else FP32_TOL, label=label)


@pytest.mark.parametrize("stress", ["eta x100", "W1 = 0"])
def test_stress_variants(lib, stress):
    """At the configs' own distributions a write changes W by ~1e-3 per chunk, so parity at
    2e-2 alone would not see an update bug; these variants make the writes dominate."""
    # with W1 = 0 the renorm target of W1 is 0 (it would stay 0), so that variant runs without it
    p = LactProblem(B=1, H=2, h=64, r=2, Nq=512, Nk=512, chunk_q=128, chunk_kv=128, dtype=BF16,
                    momentum=0.9, v_normalised=False, weight_norm=stress != "W1 = 0")
    announce(f"lact stress {stress}")
    x = make_lact_inputs(p, 21, eta_scale=1.0 if stress == "eta x100" else 0.01, w1_zero=stress == "W1 = 0")
    gpu = lact_on_gpu(lib, p, x)
    ref = lact_oracle(p, x)
    _compare(gpu, ref, BF16_TOL, label=stress)
    # the writes must be visible: the final state differs from the initial one
    w1f, w1i = np.asarray(ref["W1"][0], np.float64), np.asarray(x["W1"], np.float64)
    assert np.max(np.abs(w1f - w1i)) > 0.05 * max(np.max(np.abs(w1f)), np.max(np.abs(w1i)))


def test_per_sequence_weights_and_momentum_resume(lib):
    import torch
    from tests._helpers import dev
    p = LactProblem(B=2, H=2, h=64, r=2, Nq=512, Nk=512, chunk_q=128, chunk_kv=128, dtype=BF16,
                    muon=True, momentum=0.9, eps_norm=0.0, v_normalised=False)
    announce("lact resume: two half calls vs one call")
    x = make_lact_inputs(p, 31)
    full = lact_oracle(p, x)
    half = 256
    xa = {k: (v[:, :, :half] if k in ("Q", "K", "V", "eta") else v) for k, v in x.items()}
    xb = {k: (v[:, :, half:] if k in ("Q", "K", "V", "eta") else v) for k, v in x.items()}
    pa = p.replace(Nq=half, Nk=half)
    O1, W0a, W1a, W2a, Ma = lact_on_gpu(lib, pa, xa)
    io = torch.bfloat16
    O2, W0b, W1b, W2b, Mb = lib.lact_forward(
        dev(xb["Q"], io), dev(xb["K"], io), dev(xb["V"], io), dev(xb["eta"], torch.float32),
        W0a, W1a, W2a, chunk_q=128, muon=True, momentum=0.9, eps_norm=0.0, M_in=Ma)
    O = np.concatenate([host(O1), host(O2)], axis=2)
    err = max_abs_rel(O, full["O"])
    errw = max_abs_rel(host(W1b), full["W1"])
    print(f"resume errors O={err:.2e} W1={errw:.2e}")
    assert err <= BF16_TOL and errw <= BF16_TOL


def test_empty_sequence_returns_initial_state(lib):
    import torch
    from tests._helpers import dev
    p = LactProblem(B=1, H=2, h=64, r=2, Nq=128, Nk=128, chunk_q=64, chunk_kv=64, dtype=BF16)
    x = make_lact_inputs(p, 41)
    announce("lact empty sequence")
    z = lambda a: dev(a[:, :, :0], torch.bfloat16)
    O, W0o, W1o, W2o, Mo = lib.lact_forward(z(x["Q"]), z(x["K"]), z(x["V"]),
                                            dev(x["eta"][:, :, :0], torch.float32), dev(x["W0"], torch.float32),
                                            dev(x["W1"], torch.float32), dev(x["W2"], torch.float32), chunk_q=64)
    torch.cuda.synchronize()
    assert O.numel() == 0
    assert np.array_equal(host(W1o)[0], x["W1"]) and np.array_equal(host(W0o)[0], x["W0"])
    assert np.all(host(Mo) == 0)


@pytest.mark.parametrize("chunk", [256, 512])
def test_runs_are_bitwise_deterministic(lib, chunk):
    """Fixed-order reductions make repeated calls bit-identical (two chunk sizes, so two segment
    splits of the gradient)."""
    p = LactProblem(B=2, H=4, h=128, r=2, Nq=2048, Nk=2048, chunk_q=chunk, chunk_kv=chunk, dtype=BF16,
                    muon=True, momentum=0.9, v_normalised=False)
    announce(f"lact determinism chunk {chunk}")
    x = make_lact_inputs(p, 51)
    a = lact_on_gpu(lib, p, x)
    b = lact_on_gpu(lib, p, x)
    for u, v in zip(a, b):
        assert np.array_equal(host(u), host(v))


def test_config2_full_size_sampled_pairs(lib):
    """The LM-layer workload (B4 H8 h128 r2, seq 32768, chunk 2048, momentum 0.9, Muon, renorm)
    at full size in the benchmark's launch configuration; the oracle evaluates three of the 32
    independent pairs."""
    p = CONFIGS[2]
    announce("lact config2 full size")
    x = make_lact_inputs(p, 2)
    gpu = lact_on_gpu(lib, p, x)
    pairs = [(0, 0), (1, 5), (3, 7)]
    ref = lact_oracle(p, x, pairs=pairs)
    _compare(gpu, ref, BF16_TOL, pairs=pairs, label="config2")


def test_config3_full_size_sampled_head(lib):
    """NVS scene shape: 4 heads of h=192, one update from 196,608 context tokens, then apply to
    4096 query tokens (update-then-apply), Muon on, momentum off, renorm on."""
    p = CONFIGS[3]
    announce("lact config3 full size")
    x = make_lact_inputs(p, 3)
    gpu = lact_on_gpu(lib, p, x)
    pairs = [(0, 2)]
    ref = lact_oracle(p, x, pairs=pairs)
    _compare(gpu, ref, BF16_TOL, pairs=pairs, label="config3")
