"""Pins of the In-Place TTT oracle (CPU only).

* eta = 0 gives the plain gated MLP of Eq. 2 (written here with torch);
* chunk 0 always sees the initial W_down, so its rows equal the plain MLP;
* the sequential chunk loop equals the context-parallel prefix form
  (section 3.4), which is what associativity of Eq. 4 promises;
* the last target row never affects O (causal next-token target);
* the In-Place update is the linear-attention scan at MLP dimensions:
  Q = K = H, W0 = W_gate^T, W2 = W_up^T, W1 = W_down^T, constant eta, V = Vbar;
* the sampled evaluators (final W_down columns, selected output rows) agree
  with the full recurrence.
"""
import numpy as np
import pytest
import torch

from oracle import inplace as IP
from oracle import linattn as LA
from workloads import InplaceProblem, make_inplace_inputs


def _inputs(seed=2, **kw):
    base = dict(B=2, N=48, d_model=12, d_hidden=20, chunk=8, eta=0.05)
    base.update(kw)
    p = InplaceProblem(**base)
    return p, make_inplace_inputs(p, seed)


def _mlp(Hs, Wg, Wu, Wd):
    t = lambda a: torch.tensor(np.asarray(a), dtype=torch.float64)
    return ((torch.nn.functional.silu(t(Hs) @ t(Wg).T) * (t(Hs) @ t(Wu).T)) @ t(Wd).T).numpy()


def test_zero_eta_is_the_plain_mlp():
    p, x = _inputs()
    y = IP.inplace_forward(x["Hs"], x["W_gate"], x["W_up"], x["W_down"], x["Vbar"], 0.0, chunk=p.chunk)
    for b in range(p.B):
        np.testing.assert_allclose(y["O"][b], _mlp(x["Hs"][b], x["W_gate"], x["W_up"], x["W_down"]),
                                   rtol=1e-12, atol=1e-13)


def test_first_chunk_is_the_plain_mlp():
    p, x = _inputs()
    y = IP.inplace_forward(x["Hs"], x["W_gate"], x["W_up"], x["W_down"], x["Vbar"], p.eta, chunk=p.chunk)
    ref = _mlp(x["Hs"][0, :p.chunk], x["W_gate"], x["W_up"], x["W_down"])
    np.testing.assert_allclose(y["O"][0, :p.chunk], ref, rtol=1e-12, atol=1e-13)
    assert not np.allclose(y["O"][0, p.chunk:2 * p.chunk],
                           _mlp(x["Hs"][0, p.chunk:2 * p.chunk], x["W_gate"], x["W_up"], x["W_down"]))


def test_sequential_equals_prefix_form():
    p, x = _inputs()
    for b in range(p.B):
        o1, w1 = IP.inplace_sequence(x["Hs"][b], x["W_gate"], x["W_up"], x["W_down"], x["Vbar"][b],
                                     p.eta, chunk=p.chunk)
        o2, w2 = IP.inplace_prefix_form(x["Hs"][b], x["W_gate"], x["W_up"], x["W_down"], x["Vbar"][b],
                                        p.eta, chunk=p.chunk)
        np.testing.assert_allclose(o1, o2, rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(w1, w2, rtol=1e-11, atol=1e-13)


def test_last_target_row_does_not_reach_the_output():
    p, x = _inputs()
    y1 = IP.inplace_forward(x["Hs"], x["W_gate"], x["W_up"], x["W_down"], x["Vbar"], p.eta, chunk=p.chunk)
    x["Vbar"][:, -1] = 123.0
    y2 = IP.inplace_forward(x["Hs"], x["W_gate"], x["W_up"], x["W_down"], x["Vbar"], p.eta, chunk=p.chunk)
    assert np.array_equal(y1["O"], y2["O"])


def test_inplace_is_the_linear_attention_scan_at_mlp_dimensions():
    p, x = _inputs(B=1)
    o, w = IP.inplace_sequence(x["Hs"][0], x["W_gate"], x["W_up"], x["W_down"], x["Vbar"][0],
                               p.eta, chunk=p.chunk)
    eta = np.full(p.N, p.eta)
    ol, S = LA.linattn_pair(x["Hs"][0], x["Hs"][0], x["Vbar"][0], eta, x["W_gate"].T,
                            x["W_down"].T, x["W_up"].T, chunk=p.chunk, order=0)
    np.testing.assert_allclose(o, ol, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(w, S.T, rtol=1e-11, atol=1e-13)


def test_sampled_evaluators_agree_with_the_full_recurrence():
    p, x = _inputs(B=1, N=64)
    o, w = IP.inplace_sequence(x["Hs"][0], x["W_gate"], x["W_up"], x["W_down"], x["Vbar"][0],
                               p.eta, chunk=p.chunk)
    cols = [0, 5, 19]
    np.testing.assert_allclose(
        IP.final_wdown_columns(x["Hs"][0], x["W_gate"], x["W_up"], x["W_down"], x["Vbar"][0], p.eta, cols),
        w[:, cols], rtol=1e-11, atol=1e-13)
    rows = [0, 7, 8, 15, 30, 63]
    np.testing.assert_allclose(
        IP.output_rows(x["Hs"][0], x["W_gate"], x["W_up"], x["W_down"], x["Vbar"][0], p.eta,
                       chunk=p.chunk, rows=rows),
        o[rows], rtol=1e-11, atol=1e-13)
