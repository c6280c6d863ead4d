"""GPU parity of ttt_inplace_down_forward against the CPU oracle: full recurrence at small
sizes; at the full In-Place size (d_model 4096, d_hidden 14336, seq 32768, chunk 1024) sampled
final fast-weight columns and output rows of the first two, a middle and the last chunk."""
import numpy as np
import pytest

from tests._helpers import BF16_TOL, announce, dev, host
from workloads import CONFIGS, InplaceProblem, make_inplace_inputs, max_abs_rel

pytestmark = pytest.mark.gpu


def _gpu(lib, p, x):
    import torch
    return lib.inplace_down_forward(dev(x["Hs"], torch.bfloat16), dev(x["W_gate"], torch.bfloat16),
                                    dev(x["W_up"], torch.bfloat16), dev(x["W_down"], torch.float32),
                                    dev(x["Vbar"], torch.bfloat16), chunk=p.chunk, eta=float(x["eta"]))


@pytest.mark.parametrize("kw", [
    dict(B=2, N=512, d_model=256, d_hidden=512, chunk=128, eta=1e-3),
    dict(B=1, N=1024, d_model=512, d_hidden=768, chunk=256, eta=1e-2),
    dict(B=1, N=256, d_model=256, d_hidden=256, chunk=256, eta=1e-3),
    # apply product 256 x 512 over K = 2048: the large-tile kernel with a four-way K split
    dict(B=1, N=512, d_model=512, d_hidden=2048, chunk=256, eta=1e-3),
])
def test_small_cases(lib, kw):
    from oracle import inplace as IP
    p = InplaceProblem(**kw)
    announce(f"inplace {p}")
    x = make_inplace_inputs(p, 500 + p.N)
    O, W = _gpu(lib, p, x)
    ref = IP.inplace_forward(x["Hs"], x["W_gate"], x["W_up"], x["W_down"], x["Vbar"], float(x["eta"]),
                             chunk=p.chunk)
    eo, ew = max_abs_rel(host(O), ref["O"]), max_abs_rel(host(W), ref["W_down"])
    print(f"inplace O={eo:.2e} W={ew:.2e}")
    assert eo <= BF16_TOL and ew <= BF16_TOL
    # the writes are visible in the outputs
    assert max_abs_rel(ref["W_down"][0], x["W_down"]) > 1e-3


def test_config4_full_size_sampled(lib):
    from oracle import inplace as IP
    p = CONFIGS[4]
    announce("inplace config4 full size (sampled)")
    x = make_inplace_inputs(p, 4)
    O, W = _gpu(lib, p, x)
    cols = [0, 777, 8191, 14335]
    # rows of the first two chunks, a middle chunk (16) and the last chunk (31): the late rows
    # see the writes of every earlier chunk
    rows = [0, 511, 1023, 1024, 1500, 2047, 16 * 1024 + 3, 16 * 1024 + 700, 31 * 1024, 31 * 1024 + 555,
            32 * 1024 - 1]
    f32 = np.float32
    refW = IP.final_wdown_columns(x["Hs"][0], x["W_gate"], x["W_up"], x["W_down"], x["Vbar"][0],
                                  float(x["eta"]), cols, dtype=f32)
    refO = IP.output_rows(x["Hs"][0], x["W_gate"], x["W_up"], x["W_down"], x["Vbar"][0], float(x["eta"]),
                          chunk=p.chunk, rows=rows, dtype=f32)
    ew = max_abs_rel(host(W[0][:, cols]), refW)
    eo = max_abs_rel(host(O[0][rows]), refO)
    print(f"config4 sampled: W cols {ew:.2e}, O rows {eo:.2e}")
    assert ew <= BF16_TOL and eo <= BF16_TOL


# ---- the LM-aligned target built on the device (section 3.2, Eq. 3) ----

def _gpu_target(lib, p, x, taps, W_target=None):
    import torch
    return lib.inplace_down_forward(dev(x["Hs"], torch.bfloat16), dev(x["W_gate"], torch.bfloat16),
                                    dev(x["W_up"], torch.bfloat16), dev(x["W_down"], torch.float32), None,
                                    chunk=p.chunk, eta=float(x["eta"]), X0=dev(x["X0"], torch.bfloat16),
                                    conv_taps=dev(taps, torch.float32),
                                    W_target=None if W_target is None else dev(W_target, torch.bfloat16))


def test_next_token_target_is_bitwise_the_given_shift(lib):
    """Taps (0, 1) and no projection: the device builds exactly the next-token shift, so the call
    equals the one that is handed the shifted embeddings, bit for bit."""
    import torch
    p = InplaceProblem(B=2, N=512, d_model=256, d_hidden=512, chunk=128, eta=1e-2)
    announce(f"inplace next-token target on the device {p}")
    x = make_inplace_inputs(p, 610)
    taps = np.stack([np.zeros(p.d_model, np.float32), np.ones(p.d_model, np.float32)])
    O1, W1 = _gpu(lib, p, x)
    O2, W2 = _gpu_target(lib, p, x, taps)
    assert torch.equal(O1, O2) and torch.equal(W1, W2)


@pytest.mark.parametrize("kw,k,proj", [
    (dict(B=2, N=512, d_model=256, d_hidden=512, chunk=128, eta=5e-2), 3, False),
    (dict(B=1, N=1024, d_model=512, d_hidden=768, chunk=256, eta=5e-2), 4, True),
    # projection product 1024 x 2048 over K = 1024: the large-tile kernel
    (dict(B=1, N=2048, d_model=1024, d_hidden=2048, chunk=256, eta=2e-2), 2, True),
])
def test_general_target(lib, kw, k, proj):
    """General taps and a projection, against the oracle's target and recurrence. The step size is
    raised so that the writes carry weight in the outputs."""
    from oracle import inplace as IP
    from workloads import bf16_round
    p = InplaceProblem(**kw)
    announce(f"inplace LM-aligned target k={k} projection={proj} {p}")
    x = make_inplace_inputs(p, 620 + k)
    rng = np.random.default_rng(k)
    taps = rng.uniform(-1.0, 1.0, (k, p.d_model)).astype(np.float32)
    W_target = bf16_round((rng.standard_normal((p.d_model, p.d_model)) / np.sqrt(p.d_model)).astype(np.float32)) \
        if proj else None
    O, W = _gpu_target(lib, p, x, taps, W_target)
    Vbar = np.stack([IP.lm_aligned_target(x["X0"][b], taps, W_target) for b in range(p.B)])
    ref = IP.inplace_forward(x["Hs"], x["W_gate"], x["W_up"], x["W_down"], Vbar, float(x["eta"]), chunk=p.chunk)
    eo, ew = max_abs_rel(host(O), ref["O"]), max_abs_rel(host(W), ref["W_down"])
    print(f"inplace target O={eo:.2e} W={ew:.2e}", flush=True)
    assert eo <= BF16_TOL and ew <= BF16_TOL
    assert max_abs_rel(ref["W_down"][0], x["W_down"]) > 1e-2  # the writes are visible


# ---- backward (ttt_inplace_down_backward) ----

BWD_NAMES = ("dHs", "dW_gate", "dW_up", "dW_down", "dVbar")


def _gpu_bwd(lib, p, x, dO, W_down=None):
    import torch
    return lib.inplace_down_backward(dev(x["Hs"], torch.bfloat16), dev(x["W_gate"], torch.bfloat16),
                                     dev(x["W_up"], torch.bfloat16),
                                     dev(x["W_down"] if W_down is None else W_down, torch.float32),
                                     dev(x["Vbar"], torch.bfloat16), dev(dO, torch.bfloat16), chunk=p.chunk,
                                     eta=float(x["eta"]))


@pytest.mark.parametrize("kw,per_seq", [
    (dict(B=2, N=512, d_model=256, d_hidden=512, chunk=128, eta=1e-3), False),
    (dict(B=2, N=512, d_model=256, d_hidden=512, chunk=128, eta=1e-2), True),
    (dict(B=1, N=1024, d_model=512, d_hidden=768, chunk=256, eta=3e-3), False),
    (dict(B=1, N=256, d_model=256, d_hidden=256, chunk=256, eta=1e-3), False),  # one chunk: no write reaches O
    # products whose M and N are multiples of 256 (the large-tile update kernel)
    (dict(B=1, N=1024, d_model=512, d_hidden=1024, chunk=256, eta=2e-3), True),
])
def test_backward_small_cases(lib, kw, per_seq):
    from oracle import inplace as IP
    from workloads import bf16_round
    p = InplaceProblem(**kw)
    announce(f"inplace backward {p} per_seq={per_seq}")
    x = make_inplace_inputs(p, 600 + p.N + p.d_hidden)
    rng = np.random.default_rng(p.N + p.d_model)
    dO = bf16_round(rng.standard_normal((p.B, p.N, p.d_model)).astype(np.float32))
    Wd = np.stack([x["W_down"]] * p.B) if per_seq else x["W_down"]
    if per_seq:
        Wd = bf16_round(Wd * (1.0 + 0.1 * np.arange(p.B, dtype=np.float32))[:, None, None])
    got = _gpu_bwd(lib, p, x, dO, W_down=Wd)
    ref = IP.inplace_backward(x["Hs"], x["W_gate"], x["W_up"], Wd, x["Vbar"], float(x["eta"]), dO, chunk=p.chunk)
    ref["dHs"] = ref.pop("dH")
    errs = {k: max_abs_rel(host(got[k]), ref[k]) for k in BWD_NAMES}
    print("inplace backward: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    assert all(v <= BF16_TOL for v in errs.values()), errs
    if p.N > p.chunk:  # the writes' terms are visible in the gradients
        flat = IP.inplace_backward(x["Hs"], x["W_gate"], x["W_up"], Wd, x["Vbar"], 0.0, dO, chunk=p.chunk)
        assert max_abs_rel(flat["dH"], ref["dHs"]) > 0.05
        assert np.abs(ref["dVbar"]).max() > 0


def test_backward_full_width_two_chunks(lib):
    """The In-Place widths (d_model 4096, d_hidden 14336, chunk 1024) over two chunks: every
    gradient against the oracle (in float32, the only size it finishes in seconds)."""
    from oracle import inplace as IP
    from workloads import bf16_round
    p = InplaceProblem(B=1, N=2048, d_model=4096, d_hidden=14336, chunk=1024, eta=1e-4)
    announce(f"inplace backward full width {p}")
    x = make_inplace_inputs(p, 640)
    dO = bf16_round(np.random.default_rng(41).standard_normal((1, p.N, p.d_model)).astype(np.float32))
    got = _gpu_bwd(lib, p, x, dO)
    ref = IP.inplace_backward(x["Hs"], x["W_gate"], x["W_up"], x["W_down"], x["Vbar"], float(x["eta"]), dO,
                              chunk=p.chunk, dtype=np.float32)
    ref["dHs"] = ref.pop("dH")
    errs = {k: max_abs_rel(host(got[k]), ref[k]) for k in BWD_NAMES}
    print("full width: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    assert all(v <= BF16_TOL for v in errs.values()), errs


def test_backward_full_size_sampled_units(lib):
    """The full In-Place size (seq 32768, 32 chunks): the weight gradients of sampled hidden units
    (rows of dW_gate and dW_up, columns of dW_down) against the oracle's per-unit evaluator;
    dVbar of the last chunk is zero (no later chunk reads its write); repeated calls bit for bit."""
    import torch
    from oracle import inplace as IP
    from workloads import bf16_round
    p = CONFIGS[4]
    announce("inplace backward config4 full size (sampled units)")
    x = make_inplace_inputs(p, 4)
    dO = bf16_round(np.random.default_rng(42).standard_normal((p.B, p.N, p.d_model)).astype(np.float32))
    got = _gpu_bwd(lib, p, x, dO)
    units = [0, 777, 8191, 14335]
    ref = IP.backward_hidden_units(x["Hs"][0], x["W_gate"], x["W_up"], x["W_down"], x["Vbar"][0], float(x["eta"]),
                                   dO[0], units, chunk=p.chunk)
    errs = dict(dW_gate=max_abs_rel(host(got["dW_gate"][units]), ref["dW_gate"]),
                dW_up=max_abs_rel(host(got["dW_up"][units]), ref["dW_up"]),
                dW_down=max_abs_rel(host(got["dW_down"][:, units]).T, ref["dW_down"]))
    print("config4 sampled units: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    assert all(v <= BF16_TOL for v in errs.values()), errs
    assert not bool(got["dVbar"][0, -p.chunk:].any())
    again = _gpu_bwd(lib, p, x, dO)
    for k in BWD_NAMES:
        assert torch.equal(got[k], again[k]), k


@pytest.mark.parametrize("per_seq", [False, True])
def test_backward_empty_sequence(lib, per_seq):
    """No tokens: every weight gradient is exactly zero (shared or per-sequence W_down)."""
    p = InplaceProblem(B=2, N=256, d_model=256, d_hidden=512, chunk=128, eta=1e-3)
    announce(f"inplace backward empty sequence per_seq={per_seq}")
    x = make_inplace_inputs(p, 650)
    for k in ("Hs", "Vbar"):
        x[k] = x[k][:, :0]
    dO = np.zeros((2, 0, 256), np.float32)
    Wd = np.stack([x["W_down"]] * 2) if per_seq else x["W_down"]
    got = _gpu_bwd(lib, p.replace(N=0), x, dO, W_down=Wd)
    assert tuple(got["dW_down"].shape) == Wd.shape
    for k in ("dW_gate", "dW_up", "dW_down"):
        assert not bool(got[k].any()), k
    assert got["dHs"].numel() == 0 and got["dVbar"].numel() == 0


# ---- the LM-aligned target on its own, and the gradients reaching X0, the taps, W_target ----

def _target_case(seed, B=2, N=512, d=256, k=3, proj=True):
    rng = np.random.default_rng(seed)
    from workloads import bf16_round
    X0 = bf16_round(rng.standard_normal((B, N, d)).astype(np.float32))
    taps = rng.standard_normal((k, d)).astype(np.float32)
    W = bf16_round((rng.standard_normal((d, d)) / np.sqrt(d)).astype(np.float32)) if proj else None
    return X0, taps, W


@pytest.mark.parametrize("proj,k", [(False, 2), (True, 3), (True, 16)])
def test_target_forward_and_backward_against_the_oracle(lib, proj, k):
    import torch
    from oracle import inplace as IP
    from workloads import bf16_round
    X0, taps, W = _target_case(70 + k, k=k, proj=proj)
    announce(f"inplace target forward/backward k={k} projection={proj}")
    dX = dev(X0, torch.bfloat16)
    dT = dev(taps, torch.float32)
    dW = None if W is None else dev(W, torch.bfloat16)
    V = lib.inplace_target_forward(dX, dT, dW)
    refV = np.stack([IP.lm_aligned_target(X0[b], taps, W) for b in range(2)])
    ev = max_abs_rel(host(V), refV)
    dV = bf16_round(np.random.default_rng(k).standard_normal(X0.shape).astype(np.float32))
    g = lib.inplace_target_backward(dX, dT, dev(dV, torch.bfloat16), dW)
    refs = [IP.lm_aligned_target_backward(X0[b], taps, W, dV[b]) for b in range(2)]
    errs = dict(V=ev, dX0=max_abs_rel(host(g["dX0"]), np.stack([r[0] for r in refs])),
                dtaps=max_abs_rel(host(g["dtaps"]), sum(r[1] for r in refs)))
    if proj:
        errs["dW_target"] = max_abs_rel(host(g["dW_target"]), sum(r[2] for r in refs))
    else:
        assert g["dW_target"] is None
    print("target: " + " ".join(f"{a}={b:.2e}" for a, b in errs.items()), flush=True)
    assert all(v <= BF16_TOL for v in errs.values()), errs


def test_update_with_the_target_built_alone_matches_the_built_in_target(lib):
    """ttt_inplace_down_forward with X0 given and with Vbar from ttt_inplace_target_forward give
    the same outputs bit for bit (the projection's products, in either orientation, sum the same
    terms in the same order)."""
    import torch
    p = InplaceProblem(B=2, N=512, d_model=256, d_hidden=512, chunk=128, eta=0.05)
    announce("inplace target built alone vs built in")
    x = make_inplace_inputs(p, 660)
    X0, taps, W = _target_case(661, N=512, d=256, k=3)
    dW = dev(W, torch.bfloat16)
    args = [dev(x[k], torch.bfloat16) for k in ("Hs", "W_gate", "W_up")] + [dev(x["W_down"], torch.float32)]
    V = lib.inplace_target_forward(dev(X0, torch.bfloat16), dev(taps, torch.float32), dW)
    O1, W1 = lib.inplace_down_forward(*args, V, chunk=p.chunk, eta=p.eta)
    O2, W2 = lib.inplace_down_forward(*args, None, chunk=p.chunk, eta=p.eta, X0=dev(X0, torch.bfloat16),
                                      conv_taps=dev(taps, torch.float32), W_target=dW)
    assert torch.equal(O1, O2) and torch.equal(W1, W2)


def test_backward_through_the_lm_aligned_target(lib):
    """Every gradient of the update with the LM-aligned target: the update's backward with Vbar
    from ttt_inplace_target_forward, chained through ttt_inplace_target_backward, against the
    oracle's chain (dX0, dtaps, dW_target and the update's own gradients)."""
    import torch
    from oracle import inplace as IP
    from workloads import bf16_round
    p = InplaceProblem(B=2, N=512, d_model=256, d_hidden=512, chunk=128, eta=0.02)
    announce("inplace backward through the LM-aligned target")
    x = make_inplace_inputs(p, 670)
    X0, taps, W = _target_case(671, N=512, d=256, k=2)
    dO = bf16_round(np.random.default_rng(672).standard_normal((2, 512, 256)).astype(np.float32))
    dX, dT, dW = dev(X0, torch.bfloat16), dev(taps, torch.float32), dev(W, torch.bfloat16)
    V = lib.inplace_target_forward(dX, dT, dW)
    args = [dev(x[k], torch.bfloat16) for k in ("Hs", "W_gate", "W_up")] + [dev(x["W_down"], torch.float32)]
    g = lib.inplace_down_backward(*args, V, dev(dO, torch.bfloat16), chunk=p.chunk, eta=p.eta)
    t = lib.inplace_target_backward(dX, dT, g["dVbar"], dW)
    Vref = np.stack([IP.lm_aligned_target(X0[b], taps, W) for b in range(2)])
    ref = IP.inplace_backward(x["Hs"], x["W_gate"], x["W_up"], x["W_down"], Vref, p.eta, dO, chunk=p.chunk)
    tref = [IP.lm_aligned_target_backward(X0[b], taps, W, ref["dVbar"][b]) for b in range(2)]
    errs = dict(dHs=max_abs_rel(host(g["dHs"]), ref["dH"]), dW_gate=max_abs_rel(host(g["dW_gate"]), ref["dW_gate"]),
                dW_down=max_abs_rel(host(g["dW_down"]), ref["dW_down"]),
                dX0=max_abs_rel(host(t["dX0"]), np.stack([r[0] for r in tref])),
                dtaps=max_abs_rel(host(t["dtaps"]), sum(r[1] for r in tref)),
                dW_target=max_abs_rel(host(t["dW_target"]), sum(r[2] for r in tref)))
    print("through the target: " + " ".join(f"{a}={b:.2e}" for a, b in errs.items()), flush=True)
    assert all(v <= BF16_TOL for v in errs.values()), errs
