"""C-ABI checks that need no GPU: the library loads, exports every function the header
declares, answers workspace queries and rejects bad arguments before any launch; the
product package never reaches into the oracle."""
import ctypes
import os
import re

import pytest

import linear_attention_lact_amd as ttt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ttt_lact.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ttt.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return ttt.load()


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:ttt_status|const char\*)\s+(ttt_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_three_entry_points():
    d = _declared()
    for name in ("ttt_lact_forward", "ttt_linattn_forward", "ttt_inplace_down_forward", "ttt_linattn_backward",
                 "ttt_inplace_down_backward"):
        assert name in d


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    assert set(_declared()) == set(ttt.EXPORTED)


def test_status_strings(lib):
    for s in (ttt.TTT_OK, ttt.TTT_ERR_ARG, ttt.TTT_ERR_SHAPE, ttt.TTT_ERR_UNSUPPORTED,
              ttt.TTT_ERR_WORKSPACE, ttt.TTT_ERR_HIP):
        assert ttt.status_string(s)


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(ttt, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        ttt.load("/nonexistent/libttt_lact.so")


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: only validation and queries run here


def _lact(lib, p, ws=None, size=None, **ptrs):
    names = ["Q", "K", "V", "eta", "W0", "W1", "W2", "M_in", "O", "W0o", "W1o", "W2o", "Mo"]
    default = dict(Q=FAKE, K=FAKE, V=FAKE, eta=FAKE, W0=FAKE, W1=FAKE, W2=FAKE, O=FAKE)
    default.update(ptrs)
    sz = ctypes.c_size_t(size or 0)
    st = lib.ttt_lact_forward(ctypes.byref(p), *[default.get(n) for n in names], ws, ctypes.byref(sz), None)
    return st, sz.value


def _lp(**kw):
    base = dict(B=4, H=8, Nq=32768, Nk=32768, h=128, r=2, chunk_q=2048, chunk_kv=2048, order=0,
                dtype=ttt.BF16, update_mask=7, weight_norm=1, muon=1, momentum=0.9, eps_norm=1e-5,
                eps_ns=1e-7, w_batch_stride=0)
    base.update(kw)
    return ttt.LactParams(**base)


def test_lact_wide_heads_take_the_composed_path(lib):
    """Heads wider than 192 (the pages' d = 768 defaults): accepted in bf16 with the plain loop;
    the loop variants are not built there."""
    for kw in (dict(h=256), dict(h=768, r=2, B=1, H=1), dict(h=768, r=1, B=1, H=4)):
        st, size = _lact(lib, _lp(**kw))
        assert st == ttt.TTT_OK and size > 0, kw
    assert _lact(lib, _lp(h=768, r=1, dtype=ttt.FP32))[0] == ttt.TTT_ERR_UNSUPPORTED
    for kw in (dict(inner_steps=2), dict(eta_per_matrix=1), dict(chunk_flags=0x6000)):
        assert _lact(lib, _lp(h=256, **kw))[0] == ttt.TTT_ERR_UNSUPPORTED, kw


def test_lact_workspace_query(lib):
    st, size = _lact(lib, _lp())
    assert st == ttt.TTT_OK and size > 0
    st2, size2 = _lact(lib, _lp(B=8))
    assert st2 == ttt.TTT_OK and size2 > size


@pytest.mark.parametrize("kw,code", [
    (dict(h=0), ttt.TTT_ERR_ARG),
    (dict(B=-1), ttt.TTT_ERR_ARG),
    (dict(order=2), ttt.TTT_ERR_ARG),
    (dict(dtype=7), ttt.TTT_ERR_ARG),
    (dict(update_mask=8), ttt.TTT_ERR_ARG),
    (dict(Nk=32768 + 64), ttt.TTT_ERR_SHAPE),              # ragged last chunk
    (dict(Nq=16384, chunk_q=2048), ttt.TTT_ERR_SHAPE),     # chunk counts differ
    (dict(h=100), ttt.TTT_ERR_SHAPE),
    (dict(h=128, r=16), ttt.TTT_ERR_SHAPE),                # rh > 1024 (h <= 192)
    (dict(h=256, r=16), ttt.TTT_ERR_SHAPE),                # rh > 2048 (wider heads)
    (dict(h=1152, r=1), ttt.TTT_ERR_UNSUPPORTED),          # wider than the composed path
    (dict(h=224), ttt.TTT_ERR_SHAPE),                      # wider heads come in multiples of 128
    (dict(h=256, chunk_q=192, chunk_kv=192, Nq=192 * 16, Nk=192 * 16), ttt.TTT_ERR_SHAPE),
    (dict(dtype=ttt.FP32, h=128), ttt.TTT_ERR_UNSUPPORTED),
    (dict(w_batch_stride=5), ttt.TTT_ERR_SHAPE),
    (dict(momentum=-0.5), ttt.TTT_ERR_ARG),
    (dict(momentum=1.0), ttt.TTT_ERR_ARG),
    (dict(momentum=float("nan")), ttt.TTT_ERR_ARG),
    (dict(eps_norm=-1e-5), ttt.TTT_ERR_ARG),
    (dict(eps_ns=float("inf")), ttt.TTT_ERR_ARG),
    (dict(eps_ns=float("nan")), ttt.TTT_ERR_ARG),
])
def test_lact_rejects_bad_arguments(lib, kw, code):
    assert _lact(lib, _lp(**kw))[0] == code


def test_lact_rejects_null_pointers_and_short_workspace(lib):
    assert _lact(lib, _lp(), Q=None)[0] == ttt.TTT_ERR_ARG
    assert _lact(lib, _lp(), W1=None)[0] == ttt.TTT_ERR_ARG
    assert lib.ttt_lact_forward(None, *([FAKE] * 13), None, ctypes.byref(ctypes.c_size_t(0)), None) == ttt.TTT_ERR_ARG
    st, need = _lact(lib, _lp())
    assert _lact(lib, _lp(), ws=ctypes.c_void_p(0x100000), size=need - 1)[0] == ttt.TTT_ERR_WORKSPACE
    assert _lact(lib, _lp(), ws=ctypes.c_void_p(0x100010), size=need)[0] == ttt.TTT_ERR_WORKSPACE  # misaligned


def test_lact_empty_batch_is_a_no_op(lib):
    st, size = _lact(lib, _lp(B=0))
    assert st == ttt.TTT_OK
    assert _lact(lib, _lp(B=0), ws=ctypes.c_void_p(0x100000), size=max(size, 256))[0] == ttt.TTT_OK


def test_lact_loop_variant_fields(lib):
    # the struct's tail: flags pointer, inner steps, eta per matrix (a zero tail is the plain loop)
    assert ctypes.sizeof(ttt.LactParams) == 88
    st, plain = _lact(lib, _lp())
    assert st == ttt.TTT_OK
    st, flagged = _lact(lib, _lp(chunk_flags=0x2000))
    # apply-only chunks hold the state and momentum of every pair: 2 x 32 pairs x 3 x 128 x 256 fp32
    assert st == ttt.TTT_OK and flagged == plain + 2 * 32 * 3 * 128 * 256 * 4
    assert _lact(lib, _lp(inner_steps=4)) == (ttt.TTT_OK, plain)
    for bad in (dict(inner_steps=-1), dict(inner_steps=65), dict(eta_per_matrix=2), dict(eta_per_matrix=-1)):
        assert _lact(lib, _lp(**bad))[0] == ttt.TTT_ERR_ARG, bad


def _lin(lib, W0=FAKE, W2=FAKE, ws=None, size=0, **kw):
    base = dict(B=4, H=8, N=8192, h=64, r=2, chunk=512, order=0, dtype=ttt.BF16, w_batch_stride=0)
    base.update(kw)
    p = ttt.LinattnParams(**base)
    sz = ctypes.c_size_t(size)
    st = lib.ttt_linattn_forward(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, W0, W2, FAKE, FAKE, None,
                                 ws, ctypes.byref(sz), None)
    return st, sz.value


def test_linattn_query_and_validation(lib):
    st, size = _lin(lib)
    assert st == ttt.TTT_OK and size > 0
    assert _lin(lib, N=8000)[0] == ttt.TTT_ERR_SHAPE
    assert _lin(lib, h=48)[0] == ttt.TTT_ERR_SHAPE
    assert _lin(lib, chunk=0)[0] == ttt.TTT_ERR_ARG
    assert _lin(lib, dtype=ttt.FP32, h=256)[0] == ttt.TTT_ERR_UNSUPPORTED


def test_linattn_momentum_validation(lib):
    for bad in (-0.1, 1.0, 1.5, float("nan"), float("inf")):
        assert _lin(lib, momentum=bad)[0] == ttt.TTT_ERR_ARG, bad
    st0, single_pass = _lin(lib)
    st1, multi = _lin(lib, momentum=0.9)
    assert st0 == st1 == ttt.TTT_OK
    # with momentum the single-pass workspace holds the momentum of each inclusive prefix too
    assert multi == single_pass + 4 * 8 * 16 * 128 * 64 * 4
    assert ctypes.sizeof(ttt.LinattnParams) == 56


def test_linattn_identity_feature_map_validation(lib):
    ID = ttt.FEATURE_MAPS["identity"]
    st, size = _lin(lib, r=1, feature_map=ID)
    # single-pass workspace only: aggregates and inclusive prefixes of 64 x 64 states
    assert st == ttt.TTT_OK and 2 * 32 * 16 * 64 * 64 * 4 <= size < _lin(lib)[1]
    assert _lin(lib, r=1, feature_map=ID, W0=None, W2=None) == (ttt.TTT_OK, size)  # W0/W2 not read
    assert _lin(lib, W0=None)[0] == ttt.TTT_ERR_ARG                                   # but required by SwiGLU
    assert _lin(lib, r=2, feature_map=ID)[0] == ttt.TTT_ERR_ARG                       # state must be h x h
    for bad in (-1, 2, 7):
        assert _lin(lib, feature_map=bad)[0] == ttt.TTT_ERR_ARG
    for kw in (dict(h=96), dict(h=32), dict(h=256), dict(dtype=ttt.FP32)):
        assert _lin(lib, r=1, feature_map=ID, **kw)[0] == ttt.TTT_ERR_UNSUPPORTED, kw
    # no 8-XCD device here: a real call is refused before any launch, with a reason
    assert _lin(lib, r=1, feature_map=ID, ws=FAKE, size=size)[0] == ttt.TTT_ERR_UNSUPPORTED
    assert "single-pass" in ttt.last_error()


def test_linattn_flags_take_the_multi_launch_path(lib):
    st, plain = _lin(lib)
    st2, flagged = _lin(lib, chunk_flags=0x6000)
    assert st == st2 == ttt.TTT_OK
    # the multi-launch plan: W0/W2 shadows, chunk aggregates (fp32) and per-chunk states (fp16)
    P, nch, n = 32, 16, 128 * 64
    assert flagged >= P * 2 * n * 2 + P * nch * n * 4 + P * nch * n * 2
    assert _lin(lib, r=1, feature_map=ttt.FEATURE_MAPS["identity"], chunk_flags=0x6000)[0] == ttt.TTT_ERR_UNSUPPORTED


def test_linattn_backward_query_and_validation(lib):
    def q(**kw):
        base = dict(B=4, H=8, N=8192, h=64, r=2, chunk=512, order=0, dtype=ttt.BF16, w_batch_stride=0)
        base.update(kw)
        p = ttt.LinattnParams(**base)
        sz = ctypes.c_size_t(0)
        st = lib.ttt_linattn_backward(ctypes.byref(p), *([FAKE] * 15), None, ctypes.byref(sz), None)
        return st, sz.value
    st, size = q()
    assert st == ttt.TTT_OK and size > 0
    assert q(momentum=0.9, order=1)[0] == ttt.TTT_OK
    for kw in (dict(dtype=ttt.FP32), dict(h=128, r=2), dict(h=64, r=1), dict(r=1, feature_map=1)):
        assert q(**kw)[0] == ttt.TTT_ERR_UNSUPPORTED, kw
    assert q(N=8000)[0] == ttt.TTT_ERR_SHAPE
    assert q(momentum=1.0)[0] == ttt.TTT_ERR_ARG
    assert q(feature_map=3)[0] == ttt.TTT_ERR_ARG
    assert q(chunk_flags=0x6000)[0] == ttt.TTT_ERR_UNSUPPORTED


def _inp(lib, Vbar=FAKE, **kw):
    base = dict(B=1, N=32768, d_model=4096, d_hidden=14336, chunk=1024, eta=1e-3, dtype=ttt.BF16,
                wdown_batch_stride=0)
    base.update(kw)
    p = ttt.InplaceParams(**base)
    sz = ctypes.c_size_t(0)
    st = lib.ttt_inplace_down_forward(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, Vbar, FAKE, None, None,
                                      ctypes.byref(sz), None)
    return st, sz.value


def test_inplace_lm_aligned_target_fields(lib):
    assert ctypes.sizeof(ttt.InplaceParams) == 72
    st, given = _inp(lib)
    tgt = dict(Vbar=None, X0=0x3000, conv_taps=0x4000, conv_k=2)
    assert _inp(lib, **tgt) == (ttt.TTT_OK, given)  # the convolution is written straight into Vbar^T
    st, proj = _inp(lib, **tgt, W_target=0x5000)
    assert st == ttt.TTT_OK and proj == given + 32768 * 4096 * 2  # Conv1D(X0) before the projection
    assert _inp(lib, **{**tgt, "Vbar": FAKE})[0] == ttt.TTT_ERR_ARG  # target given twice
    for bad in (dict(conv_k=0), dict(conv_k=17), dict(conv_taps=None)):
        assert _inp(lib, **{**tgt, **bad})[0] == ttt.TTT_ERR_ARG, bad
    assert _inp(lib, Vbar=None)[0] == ttt.TTT_ERR_ARG  # no target at all


def test_inplace_query_and_validation(lib):
    st, size = _inp(lib)
    assert st == ttt.TTT_OK and size > 0
    assert _inp(lib, dtype=ttt.FP32)[0] == ttt.TTT_ERR_UNSUPPORTED
    assert _inp(lib, N=32768 + 512)[0] == ttt.TTT_ERR_SHAPE
    assert _inp(lib, d_model=4000)[0] == ttt.TTT_ERR_SHAPE
    assert _inp(lib, chunk=-4)[0] == ttt.TTT_ERR_ARG
    assert _inp(lib, chunk=64, N=32768)[0] == ttt.TTT_ERR_SHAPE  # the chunk must be a multiple of 128
    assert _inp(lib, chunk=128, N=32768)[0] == ttt.TTT_OK


def _inp_bwd(lib, **kw):
    base = dict(B=1, N=32768, d_model=4096, d_hidden=14336, chunk=1024, eta=1e-3, dtype=ttt.BF16,
                wdown_batch_stride=0)
    base.update(kw)
    p = ttt.InplaceParams(**base)
    sz = ctypes.c_size_t(0)
    st = lib.ttt_inplace_down_backward(ctypes.byref(p), *([FAKE] * 11), None, ctypes.byref(sz), None)
    return st, sz.value


def test_inplace_backward_query_and_validation(lib):
    st, size = _inp_bwd(lib)
    assert st == ttt.TTT_OK
    # every chunk's Z (both orientations), gate and up products, the transposed dA and dU, and
    # every chunk's state W_i^T, all bf16, dominate
    nch, nW = 32, 4096 * 14336
    assert size >= 6 * 32768 * 14336 * 2 + nch * nW * 2 and size < 12 << 30
    assert _inp_bwd(lib, wdown_batch_stride=4096 * 14336)[0] == ttt.TTT_OK
    assert _inp_bwd(lib, wdown_batch_stride=7)[0] == ttt.TTT_ERR_SHAPE
    assert _inp_bwd(lib, dtype=ttt.FP32)[0] == ttt.TTT_ERR_UNSUPPORTED
    assert _inp_bwd(lib, X0=0x3000, conv_taps=0x4000, conv_k=2)[0] == ttt.TTT_ERR_UNSUPPORTED
    assert _inp_bwd(lib, N=32768 + 512)[0] == ttt.TTT_ERR_SHAPE
    assert _inp_bwd(lib, d_hidden=14336 + 128)[0] == ttt.TTT_ERR_SHAPE
    assert _inp_bwd(lib, chunk=-4)[0] == ttt.TTT_ERR_ARG
    assert _inp_bwd(lib, B=0)[0] == ttt.TTT_OK


def test_inplace_target_entry_points_query_and_validation(lib):
    def q(fn, **kw):
        base = dict(B=1, N=32768, d_model=4096, d_hidden=0, chunk=1, eta=0.0, dtype=ttt.BF16, wdown_batch_stride=0,
                    X0=0x3000, conv_taps=0x4000, W_target=None, conv_k=2)
        base.update(kw)
        p = ttt.InplaceParams(**base)
        sz = ctypes.c_size_t(0)
        if fn == "fwd":
            st = lib.ttt_inplace_target_forward(ctypes.byref(p), FAKE, None, ctypes.byref(sz), None)
        else:
            st = lib.ttt_inplace_target_backward(ctypes.byref(p), FAKE, FAKE, FAKE,
                                                 FAKE if base["W_target"] else None, None, ctypes.byref(sz), None)
        return st, sz.value
    for fn in ("fwd", "bwd"):
        st, plain = q(fn)
        assert st == ttt.TTT_OK, fn
        st, proj = q(fn, W_target=0x5000)
        assert st == ttt.TTT_OK and proj > plain, fn
        assert q(fn, conv_k=0)[0] == ttt.TTT_ERR_ARG
        assert q(fn, conv_k=17)[0] == ttt.TTT_ERR_ARG
        assert q(fn, X0=None)[0] == ttt.TTT_ERR_ARG
        assert q(fn, dtype=ttt.FP32)[0] == ttt.TTT_ERR_UNSUPPORTED
        assert q(fn, d_model=4096 + 128)[0] == ttt.TTT_ERR_SHAPE
        assert q(fn, N=32768 + 64)[0] == ttt.TTT_ERR_SHAPE
    # the projection's gradient is written exactly when there is a projection
    p = ttt.InplaceParams(1, 256, 256, 0, 1, 0.0, ttt.BF16, 0, 0x3000, 0x4000, 0x5000, 2)
    sz = ctypes.c_size_t(0)
    assert lib.ttt_inplace_target_backward(ctypes.byref(p), FAKE, FAKE, FAKE, None, None, ctypes.byref(sz),
                                           None) == ttt.TTT_ERR_ARG


class _FakeCuda:
    """Stands in for a device tensor in the binding's checks (they run before any launch)."""
    is_cuda = True

    def __init__(self, shape, dtype):
        import torch
        self.shape, self.dtype, self.device = tuple(shape), dtype, torch.device("cuda:0")

    def is_contiguous(self):
        return True

    def dim(self):
        return len(self.shape)


def _fake_call_guard(monkeypatch):
    """Any attempt to reach the library after the checks fails the test."""
    def boom(*a, **k):
        raise AssertionError("the binding reached the library despite a bad argument")
    monkeypatch.setattr(ttt, "_call", boom)


@pytest.mark.parametrize("bad", ["W1 shared, W0 per sequence", "W0 wrong h", "W2 wrong heads", "W1 transposed"])
def test_linattn_binding_checks_weight_shapes_before_any_launch(monkeypatch, lib, bad):
    import torch
    _fake_call_guard(monkeypatch)
    B, H, N, h, rh = 2, 4, 256, 64, 128
    bf, f32 = torch.bfloat16, torch.float32
    Q = _FakeCuda((B, H, N, h), bf)
    eta = _FakeCuda((B, H, N), f32)
    W0, W2, W1 = _FakeCuda((H, h, rh), f32), _FakeCuda((H, h, rh), f32), _FakeCuda((H, rh, h), f32)
    if bad == "W1 shared, W0 per sequence":
        W0 = W2 = _FakeCuda((B, H, h, rh), f32)
    elif bad == "W0 wrong h":
        W0 = _FakeCuda((H, 32, rh), f32)
    elif bad == "W2 wrong heads":
        W2 = _FakeCuda((H + 1, h, rh), f32)
    else:
        W1 = _FakeCuda((H, h, rh), f32)
    with pytest.raises(ValueError):
        ttt.linattn_forward(Q, Q, Q, eta, W0, W2, W1, chunk=64)


@pytest.mark.parametrize("bad", ["W0 given", "W1 rh x h", "W1 heads", "unknown map"])
def test_identity_binding_checks_before_any_launch(monkeypatch, lib, bad):
    import torch
    _fake_call_guard(monkeypatch)
    B, H, N, h = 2, 4, 256, 64
    bf, f32 = torch.bfloat16, torch.float32
    Q = _FakeCuda((B, H, N, h), bf)
    eta = _FakeCuda((B, H, N), f32)
    W0, W1 = None, _FakeCuda((H, h, h), f32)
    fm = "identity"
    if bad == "W0 given":
        W0 = _FakeCuda((H, h, h), f32)
    elif bad == "W1 rh x h":
        W1 = _FakeCuda((H, 2 * h, h), f32)
    elif bad == "W1 heads":
        W1 = _FakeCuda((H - 1, h, h), f32)
    else:
        fm = "relu"
    with pytest.raises(ValueError):
        ttt.linattn_forward(Q, Q, Q, eta, W0, None, W1, chunk=64, feature_map=fm)


@pytest.mark.parametrize("bad", ["flags dtype", "flags shape", "inner steps 0", "eta rows"])
def test_lact_binding_checks_loop_variants_before_any_launch(monkeypatch, lib, bad):
    import torch
    _fake_call_guard(monkeypatch)
    B, H, N, h, rh = 2, 2, 256, 64, 128
    bf, f32 = torch.bfloat16, torch.float32
    Q = _FakeCuda((B, H, N, h), bf)
    eta = _FakeCuda((B, H, N), f32)
    W0, W1 = _FakeCuda((H, h, rh), f32), _FakeCuda((H, rh, h), f32)
    kw = dict(chunk_q=64)
    if bad == "flags dtype":
        kw["chunk_flags"] = _FakeCuda((B, 4), torch.int32)
    elif bad == "flags shape":
        kw["chunk_flags"] = _FakeCuda((B, 5), torch.uint8)
    elif bad == "inner steps 0":
        kw["inner_steps"] = 0
    else:
        eta = _FakeCuda((B, H, 2, N), f32)
    with pytest.raises(ValueError):
        ttt.lact_forward(Q, Q, Q, eta, W0, W1, W0, **kw)


@pytest.mark.parametrize("bad", ["M_in shape", "momentum 1", "momentum nan"])
def test_lact_binding_checks_momentum_before_any_launch(monkeypatch, lib, bad):
    import torch
    _fake_call_guard(monkeypatch)
    B, H, N, h, rh = 1, 2, 256, 64, 128
    bf, f32 = torch.bfloat16, torch.float32
    Q = _FakeCuda((B, H, N, h), bf)
    eta = _FakeCuda((B, H, N), f32)
    W0, W1 = _FakeCuda((H, h, rh), f32), _FakeCuda((H, rh, h), f32)
    kw = dict(chunk_q=64, momentum=0.9)
    if bad == "M_in shape":
        kw["M_in"] = _FakeCuda((B, H, h * rh), f32)
    else:
        kw["momentum"] = 1.0 if bad == "momentum 1" else float("nan")
    with pytest.raises(ValueError):
        ttt.lact_forward(Q, Q, Q, eta, W0, W1, W0, **kw)


def test_product_code_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "linear_attention_lact_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"\b(import|from)\s+oracle\b", text), f
                assert "oracle/" not in text, f
