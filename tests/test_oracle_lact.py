"""Pins of the LaCT oracle against things other than itself (CPU only).

* gradients: central finite differences of the loss, and torch autograd;
* Newton-Schulz-5: the singular-value polynomial via LAPACK SVD, and the
  rank-1 closed form;
* the chunk recurrence: an independent per-token unroll (torch autograd
  gradients, SVD-based orthogonalisation) equals the chunked oracle at b = 1;
* momentum: closed form when only W1 is written (its gradient then does not
  depend on the state);
* invariants the pages state: ascent == negated values, Muon's insensitivity
  to a global eta scale, renormalisation keeps the column norms, causality of
  the two orders, update-then-apply == delayed apply-then-update, eta = 0 is a
  static apply, resume from a saved state.
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch

from oracle import lact as L
from workloads import LactProblem, make_lact_inputs, UPD_ALL, UPD_W0, UPD_W1, UPD_W2

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _tiny(seed, b=3, h=4, rh=8):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((b, h))
    V = rng.standard_normal((b, h))
    eta = 0.1 + rng.random(b)
    W0 = rng.standard_normal((h, rh)) / np.sqrt(h)
    W2 = rng.standard_normal((h, rh)) / np.sqrt(h)
    W1 = rng.standard_normal((rh, h)) / np.sqrt(rh)
    return K, V, eta, W0, W1, W2


# ---------------------------------------------------------------- gradients --
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_gradients_match_central_finite_differences(seed):
    K, V, eta, W0, W1, W2 = _tiny(seed)
    G = L.chunk_gradients(K, V, eta, W0, W1, W2)
    step = 1e-6
    for which in range(3):
        Ws = [W0.copy(), W1.copy(), W2.copy()]
        num = np.zeros_like(Ws[which])
        for idx in np.ndindex(num.shape):
            for sgn in (1, -1):
                Wp = [w.copy() for w in Ws]
                Wp[which][idx] += sgn * step
                num[idx] += sgn * L.chunk_loss(K, V, eta, Wp[0], Wp[1], Wp[2])
            num[idx] /= 2 * step
        err = np.max(np.abs(num - G[which])) / np.max(np.abs(num))
        assert err < 1e-6, (which, err)


def _torch_grads(K, V, eta, W0, W1, W2):
    t = [torch.tensor(a, dtype=torch.float64, requires_grad=(i >= 3))
         for i, a in enumerate((K, V, eta, W0, W1, W2))]
    Kt, Vt, et, w0, w1, w2 = t
    F = (torch.nn.functional.silu(Kt @ w0) * (Kt @ w2)) @ w1
    loss = -(et[:, None] * F * Vt).sum()
    g0, g1, g2 = torch.autograd.grad(loss, (w0, w1, w2))
    return g0.numpy(), g1.numpy(), g2.numpy()


@pytest.mark.parametrize("seed", [3, 4])
def test_gradients_match_torch_autograd(seed):
    K, V, eta, W0, W1, W2 = _tiny(seed, b=17, h=8, rh=16)
    G = L.chunk_gradients(K, V, eta, W0, W1, W2)
    T = _torch_grads(K, V, eta, W0, W1, W2)
    for g, t in zip(G, T):
        np.testing.assert_allclose(g, t, rtol=1e-12, atol=1e-14)


def test_silu_prime_is_the_derivative_of_silu():
    a = np.linspace(-8, 8, 101)
    h = 1e-6
    num = (L.silu(a + h) - L.silu(a - h)) / (2 * h)
    np.testing.assert_allclose(L.silu_prime(a), num, rtol=1e-7, atol=1e-9)  # FD error ~ eps/h


# ------------------------------------------------------------ Newton-Schulz --
def _p5(s, a=L.NS_A, b=L.NS_B, c=L.NS_C, steps=5):
    for _ in range(steps):
        s = a * s + b * s ** 3 + c * s ** 5
    return s


def ns5_svd(G, eps):
    """Orthogonalisation through the SVD: each singular value s of the
    normalised matrix maps to p^5(s) with p(s) = a s + b s^3 + c s^5."""
    nrm = np.linalg.norm(G)
    U, S, Vt = np.linalg.svd(G, full_matrices=False)
    return (U * _p5(S / (nrm + eps))) @ Vt


def test_ns5_constants_match_the_pages():
    with open(os.path.join(GOLD, "ns5_coefficients.json")) as f:
        g = json.load(f)
    assert (L.NS_A, L.NS_B, L.NS_C, L.NS_STEPS) == (g["a"], g["b"], g["c"], g["steps"])


@pytest.mark.parametrize("shape", [(8, 16), (16, 8), (32, 64), (12, 12)])
def test_ns5_equals_singular_value_polynomial(shape):
    rng = np.random.default_rng(sum(shape))
    G = rng.standard_normal(shape)
    np.testing.assert_allclose(L.newton_schulz5(G, 1e-7), ns5_svd(G, 1e-7), rtol=1e-9, atol=1e-11)


def test_ns5_rank_one_closed_form():
    rng = np.random.default_rng(7)
    u, v = rng.standard_normal(8), rng.standard_normal(24)
    G = 3.7 * np.outer(u, v)
    out = L.newton_schulz5(G, 0.0)
    expect = _p5(1.0) * G / np.linalg.norm(G)
    np.testing.assert_allclose(out, expect, rtol=1e-12, atol=1e-14)
    # the scalar value of five rounds from s = 1
    assert abs(_p5(1.0) - 0.6964364094697522) < 1e-13


def test_ns5_of_zero_is_zero():
    assert not np.any(L.newton_schulz5(np.zeros((4, 6)), 1e-7))


# ------------------------------------------------------------ per-token unroll
def unroll_per_token(Q, K, V, eta, W0, W1, W2, *, order, update_mask, weight_norm, muon,
                     momentum, eps_norm, eps_ns):
    """Token-by-token recurrence written independently of the chunked oracle:
    per-token gradients by torch autograd, orthogonalisation via SVD."""
    W = [W0.copy(), W1.copy(), W2.copy()]
    upd = [bool(update_mask & m) for m in (UPD_W0, UPD_W1, UPD_W2)]
    nu = [np.sqrt((w ** 2).sum(0)) for w in W]
    M = [np.zeros_like(w) for w in W]
    O = np.zeros((Q.shape[0], W1.shape[1]))

    def f(q):
        a, bm = q @ W[0], q @ W[2]
        return (a / (1 + np.exp(-a)) * bm) @ W[1]

    for t in range(K.shape[0]):
        if order == 0:
            O[t] = f(Q[t])
        g = _torch_grads(K[t:t + 1], V[t:t + 1], eta[t:t + 1], W[0], W[1], W[2])
        for i in range(3):
            if not upd[i]:
                continue
            u = g[i]
            if momentum:
                M[i] = momentum * M[i] + g[i]
                u = M[i]
            if muon:
                u = ns5_svd(u, eps_ns)
            W[i] = W[i] - u
            if weight_norm:
                W[i] = W[i] * (nu[i] / (np.sqrt((W[i] ** 2).sum(0)) + eps_norm))
        if order == 1:
            O[t] = f(Q[t])
    return O, W, M


FLAG_SETS = [
    dict(update_mask=UPD_ALL, weight_norm=True, muon=False, momentum=0.0),
    dict(update_mask=UPD_ALL, weight_norm=True, muon=True, momentum=0.0),
    dict(update_mask=UPD_ALL, weight_norm=True, muon=True, momentum=0.9),
    dict(update_mask=UPD_ALL, weight_norm=False, muon=False, momentum=0.5),
    dict(update_mask=UPD_W1, weight_norm=False, muon=False, momentum=0.0),
    dict(update_mask=UPD_W0 | UPD_W2, weight_norm=True, muon=True, momentum=0.3),
]


@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("flags", FLAG_SETS)
def test_chunked_oracle_at_b1_equals_per_token_unroll(order, flags):
    p = LactProblem(B=1, H=1, h=4, r=2, Nq=6, Nk=6, chunk_q=1, chunk_kv=1)
    x = make_lact_inputs(p, 11)
    x["eta"] = x["eta"] * 30  # make the writes visible
    args = [x[k][0, 0].astype(np.float64) for k in ("Q", "K", "V", "eta")]
    ws = [x[k][0].astype(np.float64) for k in ("W0", "W1", "W2")]
    O, W0, W1, W2, M = L.lact_pair(*args, *ws, chunk_q=1, chunk_kv=1, order=order,
                                   eps_norm=1e-5, eps_ns=1e-7, **flags)
    Ou, Wu, Mu = unroll_per_token(*args, *ws, order=order, eps_norm=1e-5, eps_ns=1e-7, **flags)
    np.testing.assert_allclose(O, Ou, rtol=1e-9, atol=1e-12)
    for a, b in zip((W0, W1, W2), Wu):
        np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-12)


def test_momentum_closed_form_when_only_w1_is_written():
    """With W1 the only written matrix, its gradient -phi(K)^T diag(eta) V does
    not depend on the state, so heavy-ball momentum unrolls to
    W1_c = W1_0 - sum_{i<c} G_i (1 - alpha^(c-i)) / (1 - alpha)."""
    p = LactProblem(B=1, H=1, h=8, r=2, Nq=40, Nk=40, chunk_q=8, chunk_kv=8)
    x = make_lact_inputs(p, 5)
    Q, K, V, eta = (x[k][0, 0].astype(np.float64) for k in ("Q", "K", "V", "eta"))
    W0, W1, W2 = (x[k][0].astype(np.float64) for k in ("W0", "W1", "W2"))
    alpha = 0.9
    O, *_ = L.lact_pair(Q, K, V, eta, W0, W1, W2, chunk_q=8, chunk_kv=8, order=0,
                        update_mask=UPD_W1, weight_norm=False, muon=False, momentum=alpha)
    G = [_torch_grads(K[c * 8:(c + 1) * 8], V[c * 8:(c + 1) * 8], eta[c * 8:(c + 1) * 8],
                      W0, W1, W2)[1] for c in range(5)]
    for c in range(5):
        Wc = W1 - sum(G[i] * (1 - alpha ** (c - i)) / (1 - alpha) for i in range(c))
        a = Q[c * 8:(c + 1) * 8] @ W0
        ref = (a / (1 + np.exp(-a)) * (Q[c * 8:(c + 1) * 8] @ W2)) @ Wc
        np.testing.assert_allclose(O[c * 8:(c + 1) * 8], ref, rtol=1e-10, atol=1e-13)


# ------------------------------------------------------------------ invariants
def _small(seed=1, **kw):
    base = dict(B=1, H=2, h=8, r=2, Nq=48, Nk=48, chunk_q=12, chunk_kv=12)
    base.update(kw)
    p = LactProblem(**base)
    return p, make_lact_inputs(p, seed)


def _run(p, x, **kw):
    args = dict(chunk_q=p.chunk_q, chunk_kv=p.chunk_kv, order=p.order, update_mask=p.update_mask,
                weight_norm=p.weight_norm, muon=p.muon, momentum=p.momentum,
                eps_norm=p.eps_norm, eps_ns=p.eps_ns)
    args.update(kw)
    return L.lact_forward(x["Q"], x["K"], x["V"], x["eta"], x["W0"], x["W1"], x["W2"], **args)


@pytest.mark.parametrize("muon,momentum,wn", list(itertools.product([False, True], [0.0, 0.9], [False, True])))
def test_gradient_ascent_equals_negated_values(muon, momentum, wn):
    p, x = _small(muon=muon, momentum=momentum, weight_norm=wn)
    asc = _run(p, x, ascent=True)
    y = dict(x)
    y["V"] = -x["V"]
    neg = _run(p, y)
    for k in ("O", "W0", "W1", "W2"):
        assert np.array_equal(asc[k], neg[k]), k


def test_muon_is_insensitive_to_a_global_eta_scale():
    p, x = _small(muon=True, momentum=0.9, eps_ns=0.0)
    a = _run(p, x)
    y = dict(x)
    y["eta"] = x["eta"].astype(np.float64) * 7.0  # exact scale (float32 rounding would be amplified by NS5)
    b = _run(p, y)
    for k in ("O", "W0", "W1", "W2"):
        np.testing.assert_allclose(a[k], b[k], rtol=1e-9, atol=1e-12)


def test_renorm_keeps_initial_column_norms():
    p, x = _small(muon=True, momentum=0.5, eps_norm=0.0)
    y = _run(p, x)
    for n in ("W0", "W1", "W2"):
        for hd in range(p.H):
            np.testing.assert_allclose(np.linalg.norm(y[n][0, hd], axis=0),
                                       np.linalg.norm(x[n][hd].astype(np.float64), axis=0), rtol=1e-12)


@pytest.mark.parametrize("order", [0, 1])
def test_resume_from_saved_state_equals_one_call(order):
    p, x = _small(muon=True, momentum=0.9, eps_norm=0.0, order=order)
    full = _run(p, x)
    half = p.Nk // 2
    first = L.lact_forward(x["Q"][:, :, :half], x["K"][:, :, :half], x["V"][:, :, :half],
                           x["eta"][:, :, :half], x["W0"], x["W1"], x["W2"], chunk_q=p.chunk_q,
                           chunk_kv=p.chunk_kv, order=order, muon=True, momentum=0.9, eps_norm=0.0)
    second = L.lact_forward(x["Q"][:, :, half:], x["K"][:, :, half:], x["V"][:, :, half:],
                            x["eta"][:, :, half:], first["W0"], first["W1"], first["W2"],
                            chunk_q=p.chunk_q, chunk_kv=p.chunk_kv, order=order, muon=True,
                            momentum=0.9, eps_norm=0.0,
                            M_in={"W0": first["M0"], "W1": first["M1"], "W2": first["M2"]})
    np.testing.assert_allclose(np.concatenate([first["O"], second["O"]], axis=2), full["O"],
                               rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(second["W1"], full["W1"], rtol=1e-9, atol=1e-12)


@pytest.mark.parametrize("order", [0, 1])
def test_causality_of_the_two_orders(order):
    p, x = _small(muon=True, momentum=0.9, order=order, H=1)
    base = _run(p, x)
    c = 2
    y = {k: v.copy() for k, v in x.items()}
    y["K"][0, 0, c * 12 + 3] += 0.5
    y["V"][0, 0, c * 12 + 5] -= 0.5
    y["eta"][0, 0, c * 12 + 7] *= 3
    pert = _run(p, y)
    keep = (c + 1) * 12 if order == 0 else c * 12
    assert np.array_equal(base["O"][..., :keep, :], pert["O"][..., :keep, :])
    assert not np.allclose(base["O"][..., keep:, :], pert["O"][..., keep:, :])
    # a query perturbation changes only its own chunk's rows
    z = {k: v.copy() for k, v in x.items()}
    z["Q"][0, 0, c * 12 + 1] += 0.5
    qp = _run(p, z)
    diff = np.any(base["O"] != qp["O"], axis=-1)[0, 0]
    assert np.array_equal(np.nonzero(diff)[0], [c * 12 + 1])


def test_update_then_apply_is_delayed_apply_then_update():
    p, x = _small(muon=True, momentum=0.9, order=1, H=1)
    ua = _run(p, x)
    cq = p.chunk_q
    Q2 = np.concatenate([np.zeros_like(x["Q"][:, :, :cq]), x["Q"]], axis=2)
    K2 = np.concatenate([x["K"], x["K"][:, :, :cq]], axis=2)
    V2 = np.concatenate([x["V"], x["V"][:, :, :cq]], axis=2)
    e2 = np.concatenate([x["eta"], np.zeros_like(x["eta"][:, :, :cq])], axis=2)
    au = L.lact_forward(Q2, K2, V2, e2, x["W0"], x["W1"], x["W2"], chunk_q=cq, chunk_kv=cq,
                        order=0, muon=True, momentum=0.9)
    np.testing.assert_allclose(au["O"][:, :, cq:], ua["O"], rtol=1e-12, atol=1e-14)


def test_zero_eta_is_a_static_apply():
    p, x = _small(muon=True, momentum=0.9, eps_norm=0.0)
    x["eta"][:] = 0
    y = _run(p, x)
    for hd in range(p.H):
        q = x["Q"][0, hd].astype(np.float64)
        w0, w1, w2 = (x[k][hd].astype(np.float64) for k in ("W0", "W1", "W2"))
        a = q @ w0
        ref = (a / (1 + np.exp(-a)) * (q @ w2)) @ w1
        np.testing.assert_allclose(y["O"][0, hd], ref, rtol=1e-12, atol=1e-14)


def test_per_sequence_weights_match_shared_weights():
    p, x = _small(B=2, muon=True, momentum=0.9)
    shared = _run(p, x)
    per = {k: np.broadcast_to(x[k][None], (2,) + x[k].shape).copy() for k in ("W0", "W1", "W2")}
    y = L.lact_forward(x["Q"], x["K"], x["V"], x["eta"], per["W0"], per["W1"], per["W2"],
                       chunk_q=p.chunk_q, chunk_kv=p.chunk_kv, muon=True, momentum=0.9)
    assert np.array_equal(shared["O"], y["O"])
