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
    for name in ("ttt_lact_forward", "ttt_linattn_forward", "ttt_inplace_down_forward"):
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
    (dict(h=256, r=8), ttt.TTT_ERR_SHAPE),                 # rh > 1024
    (dict(h=256), ttt.TTT_ERR_UNSUPPORTED),
    (dict(dtype=ttt.FP32, h=128), ttt.TTT_ERR_UNSUPPORTED),
    (dict(w_batch_stride=5), ttt.TTT_ERR_SHAPE),
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


def _lin(lib, **kw):
    base = dict(B=4, H=8, N=8192, h=64, r=2, chunk=512, order=0, dtype=ttt.BF16, w_batch_stride=0)
    base.update(kw)
    p = ttt.LinattnParams(**base)
    sz = ctypes.c_size_t(0)
    st = lib.ttt_linattn_forward(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                 None, ctypes.byref(sz), None)
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
    assert ctypes.sizeof(ttt.LinattnParams) == 48


def _inp(lib, **kw):
    base = dict(B=1, N=32768, d_model=4096, d_hidden=14336, chunk=1024, eta=1e-3, dtype=ttt.BF16,
                wdown_batch_stride=0)
    base.update(kw)
    p = ttt.InplaceParams(**base)
    sz = ctypes.c_size_t(0)
    st = lib.ttt_inplace_down_forward(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None,
                                      ctypes.byref(sz), None)
    return st, sz.value


def test_inplace_query_and_validation(lib):
    st, size = _inp(lib)
    assert st == ttt.TTT_OK and size > 0
    assert _inp(lib, dtype=ttt.FP32)[0] == ttt.TTT_ERR_UNSUPPORTED
    assert _inp(lib, N=32768 + 512)[0] == ttt.TTT_ERR_SHAPE
    assert _inp(lib, d_model=4000)[0] == ttt.TTT_ERR_SHAPE
    assert _inp(lib, chunk=-4)[0] == ttt.TTT_ERR_ARG


def test_product_code_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "linear_attention_lact_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"\b(import|from)\s+oracle\b", text), f
                assert "oracle/" not in text, f
