"""Pins of the LaCT oracle's loop variants (CPU only): per-chunk write masks and resets, eta per
matrix and several inner steps per chunk.

* a reset at chunk c equals a fresh call on the tokens from c on (the definition of a document
  boundary), and the outputs before c equal a call on the tokens before c;
* an apply-only chunk equals removing its keys and values from the sequence, with its queries
  applied to the weights the earlier chunks left;
* k inner steps equal a call in which every chunk appears k times in a row (outputs read at the
  first copy for apply-then-update, at the last for update-then-apply), for every flag;
* k inner steps writing only W1 (no renorm, momentum or Muon) equal one step with k eta, since
  W1's gradient does not depend on W1;
* eta per matrix: three equal rows equal the shared eta; each matrix's one-step write equals
  the autograd gradient of the loss weighted by its own row; zero rows freeze their matrices.
"""
import itertools

import numpy as np
import pytest
import torch

from oracle import lact as L
from workloads import LactProblem, UPD_W1, make_lact_inputs

NO_UPD, RESET = L.CHUNK_NO_UPDATE, L.CHUNK_RESET


def _small(seed=1, **kw):
    base = dict(B=2, H=2, h=8, r=2, Nq=48, Nk=48, chunk_q=12, chunk_kv=12, muon=True, momentum=0.9)
    base.update(kw)
    p = LactProblem(**base)
    x = make_lact_inputs(p, seed)
    x["eta"] = x["eta"] * 10  # writes large enough that a wrong state shows
    return p, x


def _call(p, x, sl=None, b=None, **kw):
    """The oracle on sequence b's tokens sl (a slice or an index array over tokens), all heads."""
    take = lambda a: a[b:b + 1][:, :, sl] if sl is not None else a[b:b + 1]
    args = dict(chunk_q=p.chunk_q, chunk_kv=p.chunk_kv, order=p.order, update_mask=p.update_mask,
                weight_norm=p.weight_norm, muon=p.muon, momentum=p.momentum, eps_norm=p.eps_norm,
                eps_ns=p.eps_ns)
    args.update(kw)
    return L.lact_forward(take(x["Q"]), take(x["K"]), take(x["V"]), take(x["eta"]), x["W0"], x["W1"], x["W2"],
                          **args)


def _tokens(chunks, size):
    return np.concatenate([np.arange(c * size, (c + 1) * size) for c in chunks]) if chunks else np.arange(0)


TOL = dict(rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("order", [0, 1])
def test_reset_equals_a_fresh_call(order):
    p, x = _small(order=order)
    nch = p.Nk // p.chunk_kv
    flags = np.zeros((p.B, nch), np.uint8)
    flags[0, 2] = RESET
    flags[1, 1] = flags[1, 3] = RESET
    full = _call(p, x, chunk_flags=flags[0:1], b=0), _call(p, x, chunk_flags=flags[1:2], b=1)
    for b, starts in ((0, [0, 2]), (1, [0, 1, 3])):
        bounds = starts + [nch]
        for s0, s1 in zip(bounds[:-1], bounds[1:]):
            seg = _call(p, x, sl=slice(s0 * p.chunk_kv, s1 * p.chunk_kv), b=b)
            np.testing.assert_allclose(full[b]["O"][:, :, s0 * p.chunk_q:s1 * p.chunk_q], seg["O"], **TOL)
        for k in ("W0", "W1", "W2", "M0", "M1", "M2"):
            np.testing.assert_allclose(full[b][k], seg[k], **TOL)


@pytest.mark.parametrize("order", [0, 1])
def test_apply_only_chunk_equals_removing_its_writes(order):
    p, x = _small(order=order)
    nch = p.Nk // p.chunk_kv
    for b, masked in ((0, [1]), (1, [0, 3])):
        flags = np.zeros((1, nch), np.uint8)
        flags[0, masked] = NO_UPD
        full = _call(p, x, chunk_flags=flags, b=b)
        kept = [c for c in range(nch) if c not in masked]
        rest = _call(p, x, sl=_tokens(kept, p.chunk_kv), b=b)
        for i, c in enumerate(kept):
            np.testing.assert_allclose(full["O"][:, :, c * p.chunk_q:(c + 1) * p.chunk_q],
                                       rest["O"][:, :, i * p.chunk_q:(i + 1) * p.chunk_q], **TOL)
        for k in ("W0", "W1", "W2", "M0", "M1", "M2"):
            np.testing.assert_allclose(full[k], rest[k], **TOL)
        for c in masked:  # its queries see the weights the earlier written chunks left
            before = _call(p, x, sl=_tokens([k for k in kept if k < c], p.chunk_kv), b=b)
            for hd in range(p.H):
                o = L.swiglu_apply(x["Q"][b, hd, c * p.chunk_q:(c + 1) * p.chunk_q].astype(np.float64),
                                   before["W0"][0, hd], before["W1"][0, hd], before["W2"][0, hd])
                np.testing.assert_allclose(full["O"][0, hd, c * p.chunk_q:(c + 1) * p.chunk_q], o, **TOL)


@pytest.mark.parametrize("order,steps", list(itertools.product([0, 1], [2, 3])))
def test_inner_steps_equal_repeated_chunks(order, steps):
    p, x = _small(order=order)
    nch = p.Nk // p.chunk_kv
    for b in range(p.B):
        full = _call(p, x, b=b, inner_steps=steps)
        rep = _call(p, x, sl=_tokens([c for c in range(nch) for _ in range(steps)], p.chunk_kv), b=b)
        pick = 0 if order == 0 else steps - 1  # the copy whose output the loop reports
        for c in range(nch):
            r = (c * steps + pick) * p.chunk_q
            np.testing.assert_allclose(full["O"][:, :, c * p.chunk_q:(c + 1) * p.chunk_q],
                                       rep["O"][:, :, r:r + p.chunk_q], **TOL)
        for k in ("W0", "W1", "W2", "M0", "M1", "M2"):
            np.testing.assert_allclose(full[k], rep[k], **TOL)


def test_inner_steps_of_w1_only_sgd_equal_a_scaled_eta():
    p, x = _small(muon=False, momentum=0.0, weight_norm=False, update_mask=UPD_W1)
    three = _call(p, x, b=0, inner_steps=3)
    y = dict(x)
    y["eta"] = 3 * x["eta"].astype(np.float64)  # exact: the float32 draws scaled in float64
    one = _call(p, y, b=0)
    np.testing.assert_allclose(three["O"], one["O"], **TOL)
    np.testing.assert_allclose(three["W1"], one["W1"], **TOL)


def test_eta_per_matrix_with_equal_rows_is_the_shared_eta():
    p, x = _small()
    shared = _call(p, x, b=1)
    y = dict(x)
    y["eta"] = np.stack([x["eta"]] * 3, axis=2)  # [B, H, 3, Nk]
    per = _call(p, y, b=1)
    for k in ("O", "W0", "W1", "W2", "M0", "M1", "M2"):
        assert np.array_equal(shared[k], per[k]), k


def test_eta_per_matrix_write_is_each_rows_autograd_gradient():
    """One chunk of plain gradient descent: W_X moves by minus the gradient of the loss weighted
    by eta_X, taken by torch autograd at the initial weights."""
    p, x = _small(B=1, H=1, Nq=12, Nk=12, muon=False, momentum=0.0, weight_norm=False)
    rng = np.random.default_rng(5)
    eta3 = 0.05 + 0.5 * rng.random((3, p.Nk))
    out = L.lact_pair(x["Q"][0, 0], x["K"][0, 0], x["V"][0, 0], eta3, x["W0"][0], x["W1"][0], x["W2"][0],
                      chunk_q=12, chunk_kv=12, weight_norm=False)
    t = lambda a, g=False: torch.tensor(np.asarray(a, np.float64), requires_grad=g)
    K, V = t(x["K"][0, 0]), t(x["V"][0, 0])
    for i, name in enumerate(("W0", "W1", "W2")):
        w = [t(x[n][0], g=True) for n in ("W0", "W1", "W2")]
        F = (torch.nn.functional.silu(K @ w[0]) * (K @ w[2])) @ w[1]
        loss = -(t(eta3[i])[:, None] * F * V).sum()
        (g,) = torch.autograd.grad(loss, w[i])
        np.testing.assert_allclose(out[1 + i], x[name][0] - g.numpy(), rtol=1e-12, atol=1e-13)


def test_eta_per_matrix_zero_rows_freeze_their_matrices():
    p, x = _small(muon=False, momentum=0.0, weight_norm=False)
    y = dict(x)
    z = np.zeros_like(x["eta"])
    y["eta"] = np.stack([z, x["eta"], z], axis=2)
    per = _call(p, y, b=0)
    only_w1 = _call(p, x, b=0, update_mask=UPD_W1)
    for k in ("O", "W0", "W1", "W2"):
        np.testing.assert_allclose(per[k], only_w1[k], **TOL)
