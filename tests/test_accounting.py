"""Pins of the benchmark's FLOP and byte counters (linear_attention_lact_amd.accounting).

The roofline figures divide these counts by measured kernel times, so they are checked
against things other than themselves:

* the pages' state-size and FLOP model ("Test-Time Training Done Right" notes, section 2.5
  and Table 7: S = 3 r d^2 / n_h fast-weight elements per layer, update + apply over n tokens
  = 9 matmuls = 6 n S FLOPs), through the examples stored in tests/golden/state_size.json;
* the matrix products the oracle actually executes: the oracle runs on arrays that tally
  2 m n k for every matrix product they take part in, and the tally must equal the counter;
* the byte sizes of the arrays a call reads and writes.
"""
import json
import os
import types

import numpy as np
import pytest

from linear_attention_lact_amd import accounting as acc
from workloads import CONFIGS, LactProblem, make_lact_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "state_size.json")


class _Counted(np.ndarray):
    """ndarray that adds 2 m n k to a global tally for every 2-D matrix product."""
    flops = 0

    def __array_ufunc__(self, ufunc, method, *inputs, out=None, **kw):
        args = [i.view(np.ndarray) if isinstance(i, _Counted) else i for i in inputs]
        if out is not None:
            kw["out"] = tuple(o.view(np.ndarray) if isinstance(o, _Counted) else o for o in out)
        if ufunc is np.matmul and method == "__call__":
            a, b = args
            assert a.ndim == 2 and b.ndim == 2, "the oracle takes 2-D products only"
            _Counted.flops += 2 * a.shape[0] * a.shape[1] * b.shape[1]
        r = getattr(ufunc, method)(*args, **kw)
        if out is None and isinstance(r, np.ndarray):
            return r.view(_Counted)
        return r


def _counting_numpy():
    """A stand-in for the numpy module whose array constructors return counted arrays."""
    shim = types.SimpleNamespace()
    for name in dir(np):
        if not name.startswith("__"):
            setattr(shim, name, getattr(np, name))
    shim.asarray = lambda a, dtype=None: np.asarray(a, dtype=dtype).view(_Counted)
    shim.array = lambda a, dtype=None: np.array(a, dtype=dtype).view(_Counted)
    return shim


def _count(module, monkeypatch, fn):
    monkeypatch.setattr(module, "np", _counting_numpy())
    _Counted.flops = 0
    fn()
    return _Counted.flops


def test_state_size_examples_from_the_pages():
    g = json.load(open(GOLDEN))
    for ex in g["examples"]:
        S = acc.state_elements(ex["d"], ex["n_h"], ex["r"])
        if "state_over_d2" in ex:
            assert S / ex["d"] ** 2 == pytest.approx(ex["state_over_d2"], rel=1e-12), ex["what"]
        if "state_over_d" in ex:
            assert S / ex["d"] == pytest.approx(ex["state_over_d"], rel=1e-12), ex["what"]
        if "total_elements_approx" in ex:
            assert S * ex["layers"] == pytest.approx(ex["total_elements_approx"], rel=ex["rel_tol"]), ex["what"]


@pytest.mark.parametrize("d,n_h,r,n", [(768, 1, 2, 4096), (3072, 4, 1, 32768), (1024, 8, 2, 32768)])
def test_nine_matmuls_are_six_n_S(d, n_h, r, n):
    g = json.load(open(GOLDEN))
    S = acc.state_elements(d, n_h, r)
    assert acc.swiglu_matmul_flops(n, d, n_h, r) == pytest.approx(g["flops_per_token_over_state"] * n * S, rel=1e-12)


def test_lm_layer_total():
    """The LM workload (4 x 8 heads of h 128, r 2, 32768 tokens, 16 chunks, Muon on all three
    matrices): 6 n S per head and token plus five Newton-Schulz rounds of 4 m^2 n + 2 m^3 per
    matrix and chunk = 779.54 GFLOP."""
    p = CONFIGS[2]
    f = acc.lact_flops(p.B, p.H, p.Nq, p.Nk, p.h, p.r, p.chunk_q, p.chunk_kv, p.update_mask, p.muon)
    assert f == pytest.approx(779.54e9, rel=1e-5)
    d = p.H * p.h
    nS = p.B * p.Nk * acc.state_elements(d, p.H, p.r)
    assert f - 512 * 3 * acc.ns5_flops(p.h, p.rh) == pytest.approx(6 * nS, rel=1e-12)


@pytest.mark.parametrize("order,muon,h,r,chunk", [(0, True, 8, 2, 16), (1, True, 16, 1, 8), (0, False, 8, 3, 32)])
def test_lact_counter_equals_the_oracles_products(monkeypatch, order, muon, h, r, chunk):
    from oracle import lact as L
    N = 4 * chunk
    p = LactProblem(B=1, H=1, h=h, r=r, Nq=N, Nk=N, chunk_q=chunk, chunk_kv=chunk, order=order, muon=muon,
                    momentum=0.5)
    x = make_lact_inputs(p, 3)
    n = _count(L, monkeypatch, lambda: L.lact_pair(
        x["Q"][0, 0], x["K"][0, 0], x["V"][0, 0], x["eta"][0, 0], x["W0"][0], x["W1"][0], x["W2"][0],
        chunk_q=chunk, chunk_kv=chunk, order=order, muon=muon, momentum=0.5))
    assert n == acc.lact_flops(1, 1, N, N, h, r, chunk, chunk, 7, muon)


def test_ns5_counter_equals_the_oracles_products(monkeypatch):
    from oracle import lact as L
    G = np.random.default_rng(0).standard_normal((24, 40))
    for shape in ((24, 40), (40, 24)):
        n = _count(L, monkeypatch, lambda: L.newton_schulz5(np.asarray(G.reshape(shape)).view(_Counted), 1e-7))
        assert n == acc.ns5_flops(*shape)


def test_linattn_counter_equals_the_oracles_products(monkeypatch):
    from oracle import linattn as LA
    p = LactProblem(B=1, H=1, h=8, r=2, Nq=64, Nk=64, chunk_q=16, chunk_kv=16)
    x = make_lact_inputs(p, 4)
    n = _count(LA, monkeypatch, lambda: LA.linattn_pair(
        x["Q"][0, 0], x["K"][0, 0], x["V"][0, 0], x["eta"][0, 0], x["W0"][0], x["W1"][0], x["W2"][0], chunk=16))
    assert n == acc.linattn_flops(1, 1, 64, 8, 2)


def test_linattn_backward_counter_equals_the_oracles_products(monkeypatch):
    from oracle import linattn as LA
    p = LactProblem(B=1, H=1, h=8, r=2, Nq=64, Nk=64, chunk_q=16, chunk_kv=16)
    x = make_lact_inputs(p, 7)
    dO = np.random.default_rng(8).standard_normal((64, 8))
    n = _count(LA, monkeypatch, lambda: LA.linattn_backward_pair(
        x["Q"][0, 0], x["K"][0, 0], x["V"][0, 0], x["eta"][0, 0], x["W0"][0], x["W1"][0], x["W2"][0], dO, chunk=16))
    assert n == acc.linattn_backward_flops(1, 1, 64, 8, 2)


def test_linattn_identity_counter_equals_the_oracles_products(monkeypatch):
    from oracle import linattn as LA
    p = LactProblem(B=1, H=1, h=8, r=1, Nq=64, Nk=64, chunk_q=16, chunk_kv=16)
    x = make_lact_inputs(p, 6)
    n = _count(LA, monkeypatch, lambda: LA.linattn_pair(
        x["Q"][0, 0], x["K"][0, 0], x["V"][0, 0], x["eta"][0, 0], None, x["W1"][0], None, chunk=16,
        feature_map="identity"))
    assert n == acc.linattn_identity_flops(1, 1, 64, 8)


def test_inplace_counter_equals_the_oracles_products(monkeypatch):
    from oracle import inplace as IP
    rng = np.random.default_rng(5)
    N, dm, dh, C = 64, 16, 24, 16
    Hs, Vb = rng.standard_normal((N, dm)), rng.standard_normal((N, dm))
    Wg, Wu, Wd = rng.standard_normal((dh, dm)), rng.standard_normal((dh, dm)), rng.standard_normal((dm, dh))
    n = _count(IP, monkeypatch, lambda: IP.inplace_sequence(Hs, Wg, Wu, Wd, Vb, 1e-3, chunk=C))
    assert n == acc.inplace_flops(1, N, dm, dh)


def test_linattn_bytes_are_the_calls_arrays():
    """Compulsory traffic = the bytes of every array the scan call reads or writes once:
    Q, K, V, O in bf16, eta, W0, W1, W2 and the final state in fp32."""
    B, H, N, h, r = 2, 3, 64, 16, 2
    rh = r * h
    tok = np.zeros((B, H, N, h), np.uint16)
    arrays = [tok, tok, tok, tok, np.zeros((B, H, N), np.float32)]
    per_pair_w = [np.zeros((h, rh), np.float32), np.zeros((rh, h), np.float32), np.zeros((h, rh), np.float32),
                  np.zeros((rh, h), np.float32)]
    total = sum(a.nbytes for a in arrays) + B * H * sum(a.nbytes for a in per_pair_w)
    assert acc.linattn_bytes(B, H, N, h, r) == total


def test_linattn_identity_bytes_are_the_calls_arrays():
    """Identity map: Q, K, V, O in bf16, eta, the initial and the final h x h state in fp32."""
    B, H, N, h = 2, 3, 64, 16
    tok = np.zeros((B, H, N, h), np.uint16)
    arrays = [tok, tok, tok, tok, np.zeros((B, H, N), np.float32), np.zeros((B, H, h, h), np.float32),
              np.zeros((B, H, h, h), np.float32)]
    assert acc.linattn_identity_bytes(B, H, N, h) == sum(a.nbytes for a in arrays)
