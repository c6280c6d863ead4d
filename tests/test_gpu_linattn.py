"""GPU parity of ttt_linattn_forward against the CPU oracle, plus the properties the pages
state: the recurrent last-layer-only layer equals the scan form, and gradient ascent is a
sign flip of the values."""
import numpy as np
import pytest

from tests._helpers import BF16_TOL, FP32_TOL, announce, dev, host, lact_on_gpu
from workloads import BF16, CONFIGS, FP32, LactProblem, UPD_W1, make_lact_inputs, max_abs_rel

pytestmark = pytest.mark.gpu


def _lin_gpu(lib, p, x, V=None, eta=None):
    import torch
    io = torch.bfloat16 if p.dtype == BF16 else torch.float32
    return lib.linattn_forward(dev(x["Q"], io), dev(x["K"], io), dev(x["V"] if V is None else V, io),
                               dev(x["eta"] if eta is None else eta, torch.float32),
                               dev(x["W0"], torch.float32), dev(x["W2"], torch.float32),
                               dev(x["W1"], torch.float32), chunk=p.chunk_kv, order=p.order,
                               momentum=p.momentum)


def _lin_ref(p, x, pairs=None, V=None):
    from oracle import linattn as LA
    return LA.linattn_forward(x["Q"], x["K"], x["V"] if V is None else V, x["eta"], x["W0"], x["W1"], x["W2"],
                              chunk=p.chunk_kv, order=p.order, momentum=p.momentum, pairs=pairs)


CASES = [
    ("bf16 AU h64", dict(h=64, N=1024, chunk=256), 1),
    ("bf16 UA h64", dict(h=64, N=1024, chunk=256, order=1), 2),
    ("bf16 ragged tile chunk 96 h32", dict(h=32, N=480, chunk=96), 3),
    ("bf16 single chunk h128", dict(h=128, N=512, chunk=512), 4),
    ("bf16 h192 r2", dict(h=192, N=512, chunk=128), 5),
    ("bf16 h256 r1", dict(h=256, r=1, N=256, chunk=128), 6),
    ("fp32 AU h64", dict(h=64, N=512, chunk=128, dtype=FP32), 7),
    ("fp32 UA h128 r1", dict(h=128, r=1, N=256, chunk=64, dtype=FP32, order=1), 8),
    # single-pass kernel shapes: chunks shorter than one 64-token tile, one tile, rh = 4h
    ("bf16 h32 r4 chunk 32", dict(h=32, r=4, N=320, chunk=32), 9),
    ("bf16 h32 r4 UA chunk 160", dict(h=32, r=4, N=640, chunk=160, order=1), 10),
    ("bf16 h64 one tile UA", dict(h=64, N=64, chunk=64, order=1), 11),
]


@pytest.mark.parametrize("label,kw,seed", CASES, ids=[c[0] for c in CASES])
def test_small_cases(lib, label, kw, seed):
    kw = dict(kw)
    N, chunk = kw.pop("N"), kw.pop("chunk")
    base = dict(B=2, H=2, h=64, r=2, Nq=N, Nk=N, chunk_q=chunk, chunk_kv=chunk, dtype=BF16,
                update_mask=UPD_W1, weight_norm=False)
    base.update(kw)
    p = LactProblem(**base)
    announce(f"linattn {label}")
    for variant, xs in (("plain", dict()), ("eta x100", dict(eta_scale=1.0)), ("W1=0", dict(w1_zero=True))):
        x = make_lact_inputs(p, 200 + seed, **xs)
        O, S = _lin_gpu(lib, p, x)
        ref = _lin_ref(p, x)
        eo, es = max_abs_rel(host(O), ref["O"]), max_abs_rel(host(S), ref["S"])
        print(f"{label} [{variant}] O={eo:.2e} S={es:.2e}", flush=True)
        tol = BF16_TOL if p.dtype == BF16 else FP32_TOL
        assert eo <= tol and es <= tol, (variant, eo, es)


def test_config1_full_size(lib):
    p = CONFIGS[1]
    announce("linattn config1 full size B4 H8 h64 r2 N8192 chunk512")
    x = make_lact_inputs(p, 1)
    O, S = _lin_gpu(lib, p, x)
    pairs = [(0, 0), (1, 3), (2, 6), (3, 7)]
    ref = _lin_ref(p, x, pairs=pairs)
    sel = lambda a: np.stack([a[b, h] for b, h in pairs])
    eo, es = max_abs_rel(sel(host(O)), sel(ref["O"])), max_abs_rel(sel(host(S)), sel(ref["S"]))
    print(f"config1 O={eo:.2e} S={es:.2e}")
    assert eo <= BF16_TOL and es <= BF16_TOL
    for _ in range(3):  # repeated calls agree bit for bit (the prefixes are left-to-right sums)
        O2, S2 = _lin_gpu(lib, p, x)
        assert np.array_equal(host(O2), host(O)) and np.array_equal(host(S2), host(S))


@pytest.mark.parametrize("momentum", [0.0, 0.9])
@pytest.mark.parametrize("order", [0, 1])
def test_grouped_chunks_many_pairs(lib, order, momentum):
    """64 sequence-head pairs x 16 chunks: the single-pass kernel handles four chunks per
    workgroup (one round of workgroups); both orders, with and without momentum, sampled pairs
    against the oracle."""
    p = LactProblem(B=8, H=8, h=64, r=2, Nq=4096, Nk=4096, chunk_q=256, chunk_kv=256, dtype=BF16,
                    update_mask=UPD_W1, weight_norm=False, order=order, momentum=momentum)
    announce(f"linattn grouped chunks B8 H8 N4096 chunk256 order={order} momentum={momentum}")
    x = make_lact_inputs(p, 400 + order)
    O, S = _lin_gpu(lib, p, x)
    pairs = [(0, 0), (3, 5), (7, 7)]
    ref = _lin_ref(p, x, pairs=pairs)
    sel = lambda a: np.stack([a[b, h] for b, h in pairs])
    eo, es = max_abs_rel(sel(host(O)), sel(ref["O"])), max_abs_rel(sel(host(S)), sel(ref["S"]))
    print(f"grouped order={order} O={eo:.2e} S={es:.2e}")
    assert eo <= BF16_TOL and es <= BF16_TOL


@pytest.mark.parametrize("order,momentum", [(0, 0.0), (1, 0.8)])
def test_eight_chunks_per_workgroup(lib, order, momentum):
    """32 pairs x 64 chunks of 256 tokens: the single-pass kernel groups eight chunks per
    workgroup (its largest group), so each workgroup stores seven partial sums before its
    aggregate; sampled pairs against the oracle, plain apply-then-update and
    update-then-apply with momentum (eight-chunk affine group maps)."""
    p = LactProblem(B=4, H=8, h=64, r=2, Nq=16384, Nk=16384, chunk_q=256, chunk_kv=256, dtype=BF16,
                    update_mask=UPD_W1, weight_norm=False, order=order, momentum=momentum)
    announce(f"linattn eight chunks per workgroup B4 H8 N16384 chunk256 order={order} momentum={momentum}")
    x = make_lact_inputs(p, 450)
    O, S = _lin_gpu(lib, p, x)
    pairs = [(0, 1), (2, 4), (3, 7)]
    ref = _lin_ref(p, x, pairs=pairs)
    sel = lambda a: np.stack([a[b, h] for b, h in pairs])
    eo, es = max_abs_rel(sel(host(O)), sel(ref["O"])), max_abs_rel(sel(host(S)), sel(ref["S"]))
    print(f"eight chunks per group O={eo:.2e} S={es:.2e}")
    assert eo <= BF16_TOL and es <= BF16_TOL


def test_recurrent_layer_equals_scan_on_gpu(lib):
    """Theorem 5.2 on the device: the LaCT layer writing only W1, without renormalisation,
    momentum or Muon, gives the scan form's outputs."""
    for order in (0, 1):
        p = LactProblem(B=2, H=2, h=64, r=2, Nq=1024, Nk=1024, chunk_q=256, chunk_kv=256, dtype=BF16,
                        update_mask=UPD_W1, weight_norm=False, order=order)
        announce(f"linattn vs recurrent layer order={order}")
        x = make_lact_inputs(p, 300 + order, eta_scale=1.0)
        Ol, _ = _lin_gpu(lib, p, x)
        Or = lact_on_gpu(lib, p, x)[0]
        err = max_abs_rel(host(Ol), host(Or))
        print(f"order {order}: scan vs recurrent {err:.2e}")
        assert err <= BF16_TOL


@pytest.mark.parametrize("dtype", [FP32, BF16])
def test_gradient_ascent_is_a_value_sign_flip(lib, dtype):
    """The state increment is linear in V, so writing with -V (gradient ascent) flips the sign
    of O - phi(Q) W1: O(V) + O(-V) = 2 O(eta = 0). In fp32 mode the update parts are compared
    directly; in bf16 mode (outputs rounded to bf16) against the output scale."""
    p = LactProblem(B=1, H=2, h=64, r=2, Nq=1024, Nk=1024, chunk_q=256, chunk_kv=256, dtype=dtype,
                    update_mask=UPD_W1, weight_norm=False)
    announce(f"linattn ascent sign flip dtype={dtype}")
    x = make_lact_inputs(p, 400, eta_scale=1.0)
    Op, _ = _lin_gpu(lib, p, x)
    On, _ = _lin_gpu(lib, p, x, V=-x["V"])
    O0, _ = _lin_gpu(lib, p, x, eta=np.zeros_like(x["eta"]))
    op, on, o0 = host(Op).astype(np.float64), host(On).astype(np.float64), host(O0).astype(np.float64)
    if dtype == FP32:
        err = max_abs_rel(op - o0, -(on - o0))
        tol = FP32_TOL
    else:
        err = float(np.max(np.abs(op + on - 2 * o0)) / np.max(np.abs(2 * o0)))
        tol = BF16_TOL
    print(f"ascent flip ({dtype}) {err:.2e}")
    assert err <= tol
    assert max_abs_rel(op, o0) > 0.05  # the writes are visible


MOMENTUM_CASES = [
    ("bf16 AU h64 a0.9", dict(h=64, N=1024, chunk=128, momentum=0.9), 21),
    ("bf16 UA h32 r4 a0.5", dict(h=32, r=4, N=640, chunk=160, order=1, momentum=0.5), 22),
    ("bf16 h128 ragged tile a0.9", dict(h=128, N=480, chunk=96, momentum=0.9), 23),
    ("fp32 AU h64 a0.9", dict(h=64, N=512, chunk=64, dtype=FP32, momentum=0.9), 24),
    ("fp32 UA h32 a0.99", dict(h=32, N=512, chunk=32, dtype=FP32, order=1, momentum=0.99), 25),
]


@pytest.mark.parametrize("label,kw,seed", MOMENTUM_CASES, ids=[c[0] for c in MOMENTUM_CASES])
def test_momentum_cases(lib, label, kw, seed):
    """Theorem 5.3's momentum form (heavy-ball per chunk) against the oracle's cumulative
    coefficients, plain and with eta x100 so that the momentum-weighted writes dominate."""
    kw = dict(kw)
    N, chunk = kw.pop("N"), kw.pop("chunk")
    base = dict(B=2, H=2, h=64, r=2, Nq=N, Nk=N, chunk_q=chunk, chunk_kv=chunk, dtype=BF16,
                update_mask=UPD_W1, weight_norm=False)
    base.update(kw)
    p = LactProblem(**base)
    announce(f"linattn momentum {label}")
    for variant, xs in (("plain", dict()), ("eta x100", dict(eta_scale=1.0))):
        x = make_lact_inputs(p, 500 + seed, **xs)
        O, S = _lin_gpu(lib, p, x)
        ref = _lin_ref(p, x)
        eo, es = max_abs_rel(host(O), ref["O"]), max_abs_rel(host(S), ref["S"])
        print(f"{label} [{variant}] O={eo:.2e} S={es:.2e}", flush=True)
        tol = BF16_TOL if p.dtype == BF16 else FP32_TOL
        assert eo <= tol and es <= tol, (variant, eo, es)


def test_momentum_config1_shape(lib):
    """The scan workload's shape (B4 H8 h64 r2, 8192 tokens, chunks of 512) with momentum 0.9,
    sampled pairs against the oracle; and the same inputs without momentum differ."""
    from dataclasses import replace
    p = replace(CONFIGS[1], momentum=0.9)
    announce("linattn momentum 0.9 at B4 H8 h64 r2 N8192 chunk512")
    x = make_lact_inputs(p, 1)
    O, S = _lin_gpu(lib, p, x)
    pairs = [(0, 0), (1, 3), (3, 7)]
    ref = _lin_ref(p, x, pairs=pairs)
    sel = lambda a: np.stack([a[b, h] for b, h in pairs])
    eo, es = max_abs_rel(sel(host(O)), sel(ref["O"])), max_abs_rel(sel(host(S)), sel(ref["S"]))
    print(f"momentum config1 shape O={eo:.2e} S={es:.2e}")
    assert eo <= BF16_TOL and es <= BF16_TOL
    O0, _ = _lin_gpu(lib, replace(p, momentum=0.0), x)
    assert max_abs_rel(host(O), host(O0)) > 1e-3
    # where each group's lookback stops depends on timing, but every inclusive (S, m) is the same
    # sequence of group maps from the start, so repeated calls agree bit for bit
    for _ in range(3):
        O2, S2 = _lin_gpu(lib, p, x)
        assert np.array_equal(host(O2), host(O)) and np.array_equal(host(S2), host(S))


def test_momentum_scan_equals_recurrent_layer_on_gpu(lib):
    """Theorem 5.3 on the device: the LaCT layer writing only W1 with heavy-ball momentum 0.9,
    without renormalisation or Muon, gives the momentum scan form's outputs."""
    for order in (0, 1):
        p = LactProblem(B=2, H=2, h=64, r=2, Nq=1024, Nk=1024, chunk_q=256, chunk_kv=256, dtype=BF16,
                        update_mask=UPD_W1, weight_norm=False, momentum=0.9, order=order)
        announce(f"linattn momentum vs recurrent layer order={order}")
        x = make_lact_inputs(p, 310 + order, eta_scale=1.0)
        Ol, _ = _lin_gpu(lib, p, x)
        Or = lact_on_gpu(lib, p, x)[0]
        err = max_abs_rel(host(Ol), host(Or))
        print(f"order {order}: momentum scan vs recurrent {err:.2e}")
        assert err <= BF16_TOL


@pytest.mark.parametrize("momentum", [0.0, 0.9])
def test_no_learning_rate_variant(lib, momentum):
    """The simplification without a per-token learning rate (summary page, step 4): eta = 1
    for every token, through the single-pass kernel (momentum 0) and the multi-launch path."""
    p = LactProblem(B=2, H=2, h=64, r=2, Nq=1024, Nk=1024, chunk_q=256, chunk_kv=256, dtype=BF16,
                    update_mask=UPD_W1, weight_norm=False, momentum=momentum)
    announce(f"linattn eta = 1 momentum={momentum}")
    x = make_lact_inputs(p, 600)
    x["eta"] = np.ones_like(x["eta"])
    O, S = _lin_gpu(lib, p, x)
    ref = _lin_ref(p, x)
    eo, es = max_abs_rel(host(O), ref["O"]), max_abs_rel(host(S), ref["S"])
    print(f"eta=1 momentum={momentum} O={eo:.2e} S={es:.2e}")
    assert eo <= BF16_TOL and es <= BF16_TOL


@pytest.mark.parametrize("h,momentum", [(64, 0.0), (64, 0.9), (128, 0.9)])
def test_per_sequence_weights(lib, h, momentum):
    """Weights given per sequence ([B, H, ...], w_batch_stride = H*h*rh): the single-pass kernel
    (h = 64) and the multi-launch path (h = 128), with and without momentum."""
    p = LactProblem(B=2, H=2, h=h, r=2, Nq=1024, Nk=1024, chunk_q=256, chunk_kv=256, dtype=BF16,
                    update_mask=UPD_W1, weight_norm=False, momentum=momentum)
    announce(f"linattn per-sequence weights h={h} momentum={momentum}")
    x = make_lact_inputs(p, 700 + h)
    rng = np.random.default_rng(701)
    for k in ("W0", "W1", "W2"):
        x[k] = np.stack([x[k], x[k] * (1.0 + 0.2 * rng.standard_normal(x[k].shape))]).astype(np.float32)
    O, S = _lin_gpu(lib, p, x)
    ref = _lin_ref(p, x)
    eo, es = max_abs_rel(host(O), ref["O"]), max_abs_rel(host(S), ref["S"])
    print(f"per-sequence weights h={h} momentum={momentum} O={eo:.2e} S={es:.2e}")
    assert eo <= BF16_TOL and es <= BF16_TOL


# ---- per-chunk flags (apply-only chunks, resets) in the scan form: the multi-launch path ----

@pytest.mark.parametrize("dtype,order,momentum", [(BF16, 0, 0.0), (BF16, 1, 0.9), (FP32, 0, 0.9), (FP32, 1, 0.0)])
def test_chunk_flags(lib, dtype, order, momentum):
    import torch
    from oracle import linattn as LA
    p = LactProblem(B=3, H=2, h=64, r=2, Nq=1024, Nk=1024, chunk_q=128, chunk_kv=128, dtype=dtype,
                    update_mask=UPD_W1, weight_norm=False, order=order, momentum=momentum)
    flags = np.zeros((3, 8), np.uint8)
    flags[0, 4] = LA.CHUNK_RESET
    flags[1, [1, 5]] = LA.CHUNK_NO_UPDATE
    flags[2, [0, 3]] = LA.CHUNK_NO_UPDATE | LA.CHUNK_RESET
    flags[2, 6] = LA.CHUNK_RESET
    announce(f"linattn flags dtype={dtype} order={order} momentum={momentum}: {flags.tolist()}")
    x = make_lact_inputs(p, 470 + order, eta_scale=1.0)
    io = torch.bfloat16 if dtype == BF16 else torch.float32
    O, S = lib.linattn_forward(dev(x["Q"], io), dev(x["K"], io), dev(x["V"], io), dev(x["eta"], torch.float32),
                               dev(x["W0"], torch.float32), dev(x["W2"], torch.float32), dev(x["W1"], torch.float32),
                               chunk=128, order=order, momentum=momentum, chunk_flags=dev(flags, torch.uint8))
    ref = LA.linattn_forward(x["Q"], x["K"], x["V"], x["eta"], x["W0"], x["W1"], x["W2"], chunk=128, order=order,
                             momentum=momentum, chunk_flags=flags)
    eo, es = max_abs_rel(host(O), ref["O"]), max_abs_rel(host(S), ref["S"])
    print(f"flags O={eo:.2e} S={es:.2e}", flush=True)
    tol = BF16_TOL if dtype == BF16 else FP32_TOL
    assert eo <= tol and es <= tol


@pytest.mark.parametrize("feature_map,momentum,order", [("swiglu", 0.0, 0), ("swiglu", 0.9, 1), ("identity", 0.9, 0)])
def test_lookback_stress_is_bitwise_the_plain_run(lib, monkeypatch, feature_map, momentum, order):
    """The single-pass kernel with random delays before every publication (the lookback meets
    other arrival orders, groups of one and of several chunks): O and the final state equal the
    undelayed call bit for bit."""
    import torch
    ident = feature_map == "identity"
    p = LactProblem(B=4, H=8, h=64, r=1 if ident else 2, Nq=8192, Nk=8192, chunk_q=512, chunk_kv=512, dtype=BF16,
                    weight_norm=False, order=order, momentum=momentum)
    announce(f"linattn lookback stress {feature_map} momentum={momentum} order={order}")
    x = make_lact_inputs(p, 460 + order)
    args = [dev(x[k], torch.bfloat16) for k in ("Q", "K", "V")] + [dev(x["eta"], torch.float32)]
    W = [None, None] if ident else [dev(x["W0"], torch.float32), dev(x["W2"], torch.float32)]
    call = lambda: lib.linattn_forward(*args, *W, dev(x["W1"], torch.float32), chunk=512, order=order,
                                       momentum=momentum, feature_map=feature_map)
    monkeypatch.delenv("TTT_LOOKBACK_STRESS", raising=False)
    O0, S0 = call()
    for seed in ("1", "77"):
        monkeypatch.setenv("TTT_LOOKBACK_STRESS", seed)
        O1, S1 = call()
        torch.cuda.synchronize()
        assert torch.equal(O0, O1) and torch.equal(S0, S1), seed
    monkeypatch.delenv("TTT_LOOKBACK_STRESS")
