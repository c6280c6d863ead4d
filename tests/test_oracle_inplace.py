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


# ---- the LM-aligned target (section 3.2, Eq. 3) ----

def _target_inputs(seed, N=40, d=12, k=3):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((N, d)), rng.standard_normal((k, d)), rng.standard_normal((d, d)) / np.sqrt(d)


def test_next_token_taps_with_identity_projection_are_the_next_token_shift():
    X0, _, _ = _target_inputs(1)
    taps = np.zeros((2, X0.shape[1]))
    taps[1] = 1.0
    V = IP.lm_aligned_target(X0, taps)
    np.testing.assert_array_equal(V[:-1], X0[1:])
    np.testing.assert_array_equal(V[-1], 0.0)
    from workloads import InplaceProblem, make_inplace_inputs
    p = InplaceProblem(B=1, N=64, d_model=16, d_hidden=32, chunk=16, eta=1e-3)
    x = make_inplace_inputs(p, 3)
    # the generator's next-token target is this case of the general target
    np.testing.assert_array_equal(IP.lm_aligned_target(x["X0"][0], np.stack([np.zeros(16), np.ones(16)])),
                                  x["Vbar"][0])


def test_target_conv_equals_torch_depthwise_conv1d():
    """The convolution is torch's grouped (depthwise) conv1d over the sequence, right-padded with
    k - 1 zeros, with the taps in cross-correlation order; the projection is torch's linear."""
    import torch
    X0, taps, W = _target_inputs(2)
    k, d = taps.shape
    x = torch.tensor(X0.T[None], dtype=torch.float64)                   # [1, d, N]
    x = torch.nn.functional.pad(x, (0, k - 1))
    w = torch.tensor(taps.T[:, None, :], dtype=torch.float64)            # [d, 1, k]
    conv = torch.nn.functional.conv1d(x, w, groups=d)[0].T               # [N, d]
    ref = torch.nn.functional.linear(conv, torch.tensor(W, dtype=torch.float64)).numpy()
    np.testing.assert_allclose(IP.lm_aligned_target(X0, taps, W), ref, rtol=1e-12, atol=1e-12)


def test_target_row_sees_only_its_window():
    """Vbar_t depends on X0_t .. X0_{t+k-1} and on nothing else (the window the taps cover)."""
    X0, taps, W = _target_inputs(3, k=4)
    base = IP.lm_aligned_target(X0, taps, W)
    for s in (0, 7, 20, 39):
        Y = X0.copy()
        Y[s] += 1.0
        moved = np.any(IP.lm_aligned_target(Y, taps, W) != base, axis=1)
        expect = np.zeros(X0.shape[0], bool)
        expect[max(0, s - 3):s + 1] = True
        np.testing.assert_array_equal(moved, expect)


# ---- backward, pinned against torch autograd of an independent torch forward ----

@pytest.mark.parametrize("per_seq", [False, True])
def test_backward_equals_torch_autograd(per_seq):
    import torch
    rng = np.random.default_rng(51)
    B, N, d, dh, C, eta = 2, 48, 8, 12, 12, 0.3
    Hs, Vb, dO = rng.standard_normal((B, N, d)), rng.standard_normal((B, N, d)), rng.standard_normal((B, N, d))
    Wg, Wu = rng.standard_normal((dh, d)) / 3, rng.standard_normal((dh, d)) / 3
    Wd = rng.standard_normal((B, d, dh) if per_seq else (d, dh)) / 3
    t = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    th, tg, tu, td, tv = t(Hs), t(Wg), t(Wu), t(Wd), t(Vb)
    outs = []
    for b in range(B):
        W = td[b] if per_seq else td
        for i in range(N // C):
            s = slice(i * C, (i + 1) * C)
            Z = torch.nn.functional.silu(th[b, s] @ tg.T) * (th[b, s] @ tu.T)
            outs.append(Z @ W.T)
            W = W + eta * (tv[b, s].T @ Z)
    O = torch.stack(outs).reshape(B, N, d)
    grads = torch.autograd.grad((O * torch.tensor(dO)).sum(), (th, tg, tu, td, tv))
    got = IP.inplace_backward(Hs, Wg, Wu, Wd, Vb, eta, dO, chunk=C)
    for k, g in zip(("dH", "dW_gate", "dW_up", "dW_down", "dVbar"), grads):
        np.testing.assert_allclose(got[k], g.numpy(), rtol=1e-10, atol=1e-11, err_msg=k)


def test_hidden_unit_gradients_equal_the_full_backward():
    """The per-unit evaluator used at full size against the full backward (itself pinned to
    autograd above), on units at both ends and in the middle."""
    rng = np.random.default_rng(52)
    N, d, dh, C, eta = 60, 10, 14, 12, 0.2
    Hs, Vb, dO = rng.standard_normal((N, d)), rng.standard_normal((N, d)), rng.standard_normal((N, d))
    Wg, Wu, Wd = rng.standard_normal((dh, d)) / 3, rng.standard_normal((dh, d)) / 3, rng.standard_normal((d, dh)) / 3
    full = IP.inplace_backward_sequence(Hs, Wg, Wu, Wd, Vb, eta, dO, chunk=C)
    units = [0, 5, dh - 1]
    got = IP.backward_hidden_units(Hs, Wg, Wu, Wd, Vb, eta, dO, units, chunk=C)
    np.testing.assert_allclose(got["dW_gate"], full["dW_gate"][units], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(got["dW_up"], full["dW_up"][units], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(got["dW_down"], full["dW_down"][:, units].T, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("proj", [False, True])
def test_target_backward_equals_torch_autograd(proj):
    """The target's gradients against torch autograd of torch's depthwise conv1d and linear."""
    import torch
    X0, taps, W = _target_inputs(4, k=3)
    W = W if proj else None
    dV = np.random.default_rng(9).standard_normal(X0.shape)
    k, d = taps.shape
    tx = torch.tensor(X0, dtype=torch.float64, requires_grad=True)
    tt = torch.tensor(taps, dtype=torch.float64, requires_grad=True)
    xin = torch.nn.functional.pad(tx.T[None], (0, k - 1))
    conv = torch.nn.functional.conv1d(xin, tt.T[:, None, :], groups=d)[0].T
    leaves = [tx, tt]
    if proj:
        tw = torch.tensor(W, dtype=torch.float64, requires_grad=True)
        leaves.append(tw)
        conv = torch.nn.functional.linear(conv, tw)
    grads = torch.autograd.grad((conv * torch.tensor(dV)).sum(), leaves)
    dX0, dtaps, dW = IP.lm_aligned_target_backward(X0, taps, W, dV)
    np.testing.assert_allclose(dX0, grads[0].numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dtaps, grads[1].numpy(), rtol=1e-12, atol=1e-12)
    if proj:
        np.testing.assert_allclose(dW, grads[2].numpy(), rtol=1e-12, atol=1e-12)
    else:
        assert dW is None
