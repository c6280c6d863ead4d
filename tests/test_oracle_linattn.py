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


# ---- Variant 3: phi = identity, one linear fast-weight layer with an h x h state ----

def _identity_inputs(seed, h=8, N=48, B=2, H=2):
    p = LactProblem(B=B, H=H, h=h, r=1, Nq=N, Nk=N, chunk_q=N, chunk_kv=N)
    x = make_lact_inputs(p, seed)
    x["eta"] = x["eta"] * 20
    return p, x


def _recurrent_linear_fast_weight(Q, K, V, eta, S0, chunk, order, momentum):
    """Variant 3 as test-time training, written without the scan: the fast weight is the single
    linear layer f(x) = x W; each chunk takes one gradient step on
    L_c(W) = -sum_t eta_t <k_t W, v_t> at the chunk-start W (gradient from torch autograd), through
    the heavy-ball buffer M <- alpha M + G, W <- W - M; apply-then-update reads W before the step,
    update-then-apply after it."""
    import torch
    t = lambda a: torch.tensor(np.asarray(a), dtype=torch.float64)
    Q, K, V, eta = t(Q), t(K), t(V), t(eta)
    W = t(S0)
    M = torch.zeros_like(W)
    O = torch.zeros(Q.shape[0], W.shape[1], dtype=torch.float64)
    for c in range(K.shape[0] // chunk):
        sl = slice(c * chunk, (c + 1) * chunk)
        if order == 0:
            O[sl] = Q[sl] @ W
        Wv = W.clone().requires_grad_(True)
        loss = -(eta[sl, None] * (K[sl] @ Wv) * V[sl]).sum()
        (G,) = torch.autograd.grad(loss, Wv)
        M = momentum * M + G
        W = W - M
        if order == 1:
            O[sl] = Q[sl] @ W
    return O.numpy(), W.numpy()


@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("momentum", [0.0, 0.6])
@pytest.mark.parametrize("chunk", [1, 8, 48])
def test_identity_scan_equals_recurrent_linear_fast_weight(order, momentum, chunk):
    p, x = _identity_inputs(21)
    for b in range(p.B):
        for hd in range(p.H):
            args = [x[k][b, hd] for k in ("Q", "K", "V", "eta")]
            o, s = LA.linattn_pair(*args, None, x["W1"][hd], None, chunk=chunk, order=order,
                                   momentum=momentum, feature_map="identity")
            ro, rs = _recurrent_linear_fast_weight(*args, x["W1"][hd], chunk, order, momentum)
            np.testing.assert_allclose(o, ro, rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(s, rs, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("momentum", [0.0, 0.7])
@pytest.mark.parametrize("chunk", [1, 4, 16])
def test_identity_scan_equals_masked_quadratic_form(order, momentum, chunk):
    p, x = _identity_inputs(22)
    args = [x[k][0, 1] for k in ("Q", "K", "V", "eta")]
    o, _ = LA.linattn_pair(*args, None, x["W1"][1], None, chunk=chunk, order=order, momentum=momentum,
                           feature_map="identity")
    q = LA.linattn_masked_quadratic(*args, None, x["W1"][1], None, chunk=chunk, order=order,
                                    momentum=momentum, feature_map="identity")
    np.testing.assert_allclose(o, q, rtol=1e-11, atol=1e-12)


def test_identity_token_chunks_update_then_apply_is_causal_linear_attention():
    """Chunks of one token with update-then-apply: textbook causal linear attention,
    o_t = q_t (S0 + sum_{s <= t} k_s^T (eta_s v_s)), accumulated token by token."""
    p, x = _identity_inputs(23, h=16, N=40, B=1, H=1)
    Q, K, V, eta = (x[k][0, 0].astype(np.float64) for k in ("Q", "K", "V", "eta"))
    S0 = x["W1"][0].astype(np.float64)
    out = LA.linattn_forward(x["Q"], x["K"], x["V"], x["eta"], None, x["W1"], None, chunk=1, order=1,
                             feature_map="identity")
    state = S0.copy()
    for t in range(40):
        state += eta[t] * np.outer(K[t], V[t])
        np.testing.assert_allclose(out["O"][0, 0, t], Q[t] @ state, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(out["S"][0, 0], state, rtol=1e-12, atol=1e-13)
    assert out["S"].shape == (1, 1, 16, 16)


# ---- backward of the scan form, pinned against torch autograd ----

def _torch_scan_forward(Q, K, V, eta, W0, W1, W2, chunk, order, momentum, ident):
    """The scan form written with torch ops and the heavy-ball recurrence (m <- alpha m + dS_c,
    S <- S + m), independent of the oracle's coefficient form."""
    import torch
    feat = (lambda X: X) if ident else (lambda X: torch.nn.functional.silu(X @ W0) * (X @ W2))
    S = W1.clone()
    m = torch.zeros_like(W1)
    outs = []
    for c in range(K.shape[0] // chunk):
        s = slice(c * chunk, (c + 1) * chunk)
        dS = feat(K[s]).T @ (eta[s, None] * V[s])
        if order == 1:
            m = momentum * m + dS
            S = S + m
        outs.append(feat(Q[s]) @ S)
        if order == 0:
            m = momentum * m + dS
            S = S + m
    return torch.cat(outs)


@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("momentum", [0.0, 0.7])
@pytest.mark.parametrize("ident", [False, True])
def test_backward_equals_torch_autograd(order, momentum, ident):
    import torch
    h, r = 8, (1 if ident else 2)
    p = LactProblem(B=1, H=1, h=h, r=r, Nq=48, Nk=48, chunk_q=12, chunk_kv=12)
    x = make_lact_inputs(p, 31)
    x["eta"] = x["eta"] * 30
    dO = np.random.default_rng(32).standard_normal((48, h))
    t = lambda a: torch.tensor(np.asarray(a, np.float64), requires_grad=True)
    args = [t(x[k][0, 0]) for k in ("Q", "K", "V", "eta")] + [t(x[k][0]) for k in ("W0", "W1", "W2")]
    O = _torch_scan_forward(*args, 12, order, momentum, ident)
    grads = torch.autograd.grad((O * torch.tensor(dO)).sum(), args, allow_unused=True)
    ref = dict(zip(("dQ", "dK", "dV", "deta", "dW0", "dW1", "dW2"), grads))
    w0, w2 = (None, None) if ident else (x["W0"][0], x["W2"][0])
    got = LA.linattn_backward_pair(x["Q"][0, 0], x["K"][0, 0], x["V"][0, 0], x["eta"][0, 0], w0, x["W1"][0], w2, dO,
                                   chunk=12, order=order, momentum=momentum,
                                   feature_map="identity" if ident else "swiglu")
    for k, v in ref.items():
        if ident and k in ("dW0", "dW2"):
            assert got[k] is None
            continue
        np.testing.assert_allclose(got[k], v.numpy(), rtol=1e-10, atol=1e-12, err_msg=k)


def test_backward_batch_layouts():
    """Shared weights: the weight gradients are summed over the batch; per-sequence weights keep
    one gradient per sequence, equal to the single-pair gradients."""
    p = LactProblem(B=2, H=2, h=8, r=2, Nq=24, Nk=24, chunk_q=8, chunk_kv=8)
    x = make_lact_inputs(p, 33)
    dO = np.random.default_rng(34).standard_normal((2, 2, 24, 8))
    shared = LA.linattn_backward(x["Q"], x["K"], x["V"], x["eta"], x["W0"], x["W1"], x["W2"], dO, chunk=8)
    per = {k: np.stack([x[k]] * 2) for k in ("W0", "W1", "W2")}
    ps = LA.linattn_backward(x["Q"], x["K"], x["V"], x["eta"], per["W0"], per["W1"], per["W2"], dO, chunk=8)
    for k in ("dW0", "dW1", "dW2"):
        np.testing.assert_allclose(shared[k], ps[k].sum(axis=0), rtol=1e-12, atol=1e-14)
        one = LA.linattn_backward_pair(x["Q"][1, 0], x["K"][1, 0], x["V"][1, 0], x["eta"][1, 0], x["W0"][0],
                                       x["W1"][0], x["W2"][0], dO[1, 0], chunk=8)
        np.testing.assert_allclose(ps[k][1, 0], one[k], rtol=1e-12, atol=1e-14)
    for k in ("dQ", "dK", "dV", "deta"):
        assert np.array_equal(shared[k], ps[k])


# ---- per-chunk flags in the scan form ----

def _flag_inputs(seed):
    p = LactProblem(B=1, H=2, h=8, r=2, Nq=60, Nk=60, chunk_q=12, chunk_kv=12)
    x = make_lact_inputs(p, seed)
    x["eta"] = x["eta"] * 20
    return p, x


def _lin(x, sl=None, **kw):
    take = (lambda a: a[:, :, sl]) if sl is not None else (lambda a: a)
    return LA.linattn_forward(take(x["Q"]), take(x["K"]), take(x["V"]), take(x["eta"]), x["W0"], x["W1"], x["W2"],
                              chunk=12, **kw)


@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("momentum", [0.0, 0.8])
def test_scan_flags_clear_equal_the_coefficient_form(order, momentum):
    p, x = _flag_inputs(41)
    a = _lin(x, order=order, momentum=momentum)
    b = _lin(x, order=order, momentum=momentum, chunk_flags=np.zeros((1, 5), np.uint8))
    np.testing.assert_allclose(b["O"], a["O"], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(b["S"], a["S"], rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("momentum", [0.0, 0.8])
def test_scan_reset_equals_a_fresh_call(order, momentum):
    p, x = _flag_inputs(42)
    flags = np.zeros((1, 5), np.uint8)
    flags[0, [2, 4]] = LA.CHUNK_RESET
    full = _lin(x, order=order, momentum=momentum, chunk_flags=flags)
    for s0, s1 in ((0, 2), (2, 4), (4, 5)):
        seg = _lin(x, sl=slice(12 * s0, 12 * s1), order=order, momentum=momentum)
        np.testing.assert_allclose(full["O"][:, :, 12 * s0:12 * s1], seg["O"], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(full["S"], seg["S"], rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("momentum", [0.0, 0.8])
def test_scan_apply_only_chunk_equals_removing_its_write(order, momentum):
    p, x = _flag_inputs(43)
    flags = np.zeros((1, 5), np.uint8)
    flags[0, [1, 3]] = LA.CHUNK_NO_UPDATE
    full = _lin(x, order=order, momentum=momentum, chunk_flags=flags)
    kept = np.concatenate([np.arange(12 * c, 12 * c + 12) for c in (0, 2, 4)])
    rest = _lin(x, sl=kept, order=order, momentum=momentum)
    for i, c in enumerate((0, 2, 4)):
        np.testing.assert_allclose(full["O"][:, :, 12 * c:12 * c + 12], rest["O"][:, :, 12 * i:12 * i + 12],
                                   rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(full["S"], rest["S"], rtol=1e-11, atol=1e-12)
    for c, before in ((1, [0]), (3, [0, 2])):  # its queries read the state the earlier writes left
        prev = _lin(x, sl=np.concatenate([np.arange(12 * k, 12 * k + 12) for k in before]), order=order,
                    momentum=momentum)
        for hd in range(2):
            o = LA.phi(x["Q"][0, hd, 12 * c:12 * c + 12].astype(np.float64), x["W0"][hd], x["W2"][hd]) @ prev["S"][0, hd]
            np.testing.assert_allclose(full["O"][0, hd, 12 * c:12 * c + 12], o, rtol=1e-11, atol=1e-12)
