"""Pins of the linear-attention oracle (CPU only).

* the recurrent last-layer-only LaCT layer (W1 written, no renormalisation,
  no momentum, no Muon) equals the scan form -- Theorem 5.2 of the summary
  page; apply-then-update <-> exclusive prefix, update-then-apply <-> inclusive;
* the masked quadratic ("dual") matrix form of the press article, section 4;
* one chunk over the whole sequence with update-then-apply is textbook linear
  attention o = phi(q)(S0 + sum phi(k)^T (eta v)), written here token by token;
* the zero-initialised single-state case (W1 = 0);
* with momentum (Theorem 5.3, constant alpha): the recurrent layer's heavy-ball
  path (M <- alpha M + G per chunk, W <- W - M) equals the scan form with the
  cumulative coefficients, which are the geometric sums (1 - alpha^n) / (1 - alpha).
"""
import numpy as np
import pytest

from oracle import lact as L
from oracle import linattn as LA
from workloads import LactProblem, make_lact_inputs, UPD_W1


def _inputs(seed, **kw):
    base = dict(B=2, H=2, h=8, r=2, Nq=64, Nk=64, chunk_q=16, chunk_kv=16)
    base.update(kw)
    p = LactProblem(**base)
    return p, make_lact_inputs(p, seed)


@pytest.mark.parametrize("order", [0, 1])
def test_recurrent_last_layer_only_equals_scan(order):
    p, x = _inputs(3)
    x["eta"] = x["eta"] * 20
    rec = L.lact_forward(x["Q"], x["K"], x["V"], x["eta"], x["W0"], x["W1"], x["W2"],
                         chunk_q=16, chunk_kv=16, order=order, update_mask=UPD_W1,
                         weight_norm=False, muon=False, momentum=0.0)
    lin = LA.linattn_forward(x["Q"], x["K"], x["V"], x["eta"], x["W0"], x["W1"], x["W2"],
                             chunk=16, order=order)
    np.testing.assert_allclose(lin["O"], rec["O"], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(lin["S"], rec["W1"], rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("chunk", [1, 4, 16, 64])
def test_scan_equals_masked_quadratic_form(order, chunk):
    p, x = _inputs(4, chunk_q=chunk, chunk_kv=chunk)
    for b in range(p.B):
        for hd in range(p.H):
            args = [x[k][b, hd] for k in ("Q", "K", "V", "eta")] + [x[k][hd] for k in ("W0", "W1", "W2")]
            o, _ = LA.linattn_pair(*args, chunk=chunk, order=order)
            q = LA.linattn_masked_quadratic(*args, chunk=chunk, order=order)
            np.testing.assert_allclose(o, q, rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("w1_zero", [False, True])
def test_single_chunk_update_then_apply_is_textbook_linear_attention(w1_zero):
    p = LactProblem(B=1, H=1, h=8, r=2, Nq=20, Nk=20, chunk_q=20, chunk_kv=20)
    x = make_lact_inputs(p, 9, w1_zero=w1_zero)
    Q, K, V, eta = (x[k][0, 0].astype(np.float64) for k in ("Q", "K", "V", "eta"))
    W0, W1, W2 = (x[k][0].astype(np.float64) for k in ("W0", "W1", "W2"))
    o, S = LA.linattn_pair(Q, K, V, eta, W0, W1, W2, chunk=20, order=1)
    # token-by-token state accumulation, with the feature map from torch
    import torch
    t = lambda a: torch.tensor(a, dtype=torch.float64)
    feat = lambda X: (torch.nn.functional.silu(t(X) @ t(W0)) * (t(X) @ t(W2))).numpy()
    state = W1.copy()
    fk = feat(K)
    for i in range(20):
        state += np.outer(fk[i], eta[i] * V[i])
    np.testing.assert_allclose(S, state, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(o, feat(Q) @ state, rtol=1e-12, atol=1e-14)


def test_per_sequence_weights():
    p, x = _inputs(6)
    shared = LA.linattn_forward(x["Q"], x["K"], x["V"], x["eta"], x["W0"], x["W1"], x["W2"], chunk=16)
    per = {k: np.stack([x[k]] * p.B) for k in ("W0", "W1", "W2")}
    ps = LA.linattn_forward(x["Q"], x["K"], x["V"], x["eta"], per["W0"], per["W1"], per["W2"], chunk=16)
    assert np.array_equal(shared["O"], ps["O"])


@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("alpha", [0.5, 0.9])
def test_momentum_scan_equals_recurrent_heavy_ball(order, alpha):
    p, x = _inputs(11)
    x["eta"] = x["eta"] * 20
    rec = L.lact_forward(x["Q"], x["K"], x["V"], x["eta"], x["W0"], x["W1"], x["W2"],
                         chunk_q=16, chunk_kv=16, order=order, update_mask=UPD_W1,
                         weight_norm=False, muon=False, momentum=alpha)
    lin = LA.linattn_forward(x["Q"], x["K"], x["V"], x["eta"], x["W0"], x["W1"], x["W2"],
                             chunk=16, order=order, momentum=alpha)
    np.testing.assert_allclose(lin["O"], rec["O"], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(lin["S"], rec["W1"], rtol=1e-11, atol=1e-13)
    plain = LA.linattn_forward(x["Q"], x["K"], x["V"], x["eta"], x["W0"], x["W1"], x["W2"],
                               chunk=16, order=order)
    assert np.abs(lin["O"] - plain["O"]).max() > 1e-3  # momentum changes the outputs


@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("chunk", [4, 16])
def test_momentum_scan_equals_masked_quadratic_form(order, chunk):
    p, x = _inputs(12, chunk_q=chunk, chunk_kv=chunk)
    args = [x[k][1, 0] for k in ("Q", "K", "V", "eta")] + [x[k][0] for k in ("W0", "W1", "W2")]
    o, _ = LA.linattn_pair(*args, chunk=chunk, order=order, momentum=0.8)
    q = LA.linattn_masked_quadratic(*args, chunk=chunk, order=order, momentum=0.8)
    np.testing.assert_allclose(o, q, rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("order", [0, 1])
def test_momentum_weight_is_geometric_sum(order):
    for alpha in (0.0, 0.3, 0.9):
        for c in range(6):
            for i in range(6):
                n = c - i + (1 if order == 1 else 0)
                want = 0.0 if n <= 0 else (float(n) if alpha == 1.0 else (1 - alpha ** n) / (1 - alpha))
                assert abs(LA.momentum_weight(c, i, alpha, order) - want) < 1e-14, (alpha, c, i)
