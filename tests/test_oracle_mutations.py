"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible mistake into the oracle (a dropped term, a flipped sign, a
wrong operand, a wrong coefficient or round count, the wrong normalisation axis, a dampened
momentum, swapped update/apply order, an off-by-one in the scan boundary) and runs the pin
that is meant to see it. The pin must fail: a pin that passes on a broken oracle pins
nothing. The mistakes are planted by monkeypatching the oracle modules inside the test, so
the oracle itself is untouched.
"""
import numpy as np
import pytest

from oracle import inplace as IP
from oracle import lact as L
from oracle import linattn as LA
from tests import test_oracle_inplace as TI
from tests import test_oracle_lact as TL
from tests import test_oracle_lact_variants as TLV
from tests import test_oracle_linattn as TLA


def _flip_g0(orig):
    def f(*a):
        G0, G1, G2 = orig(*a)
        return -G0, G1, G2
    return f


def _g1_wrong_operand(orig):
    def f(K, V, eta, W0, W1, W2):
        G0, _, G2 = orig(K, V, eta, W0, W1, W2)
        A, Bm = K @ W0, K @ W2
        return G0, -((L.silu(A) * Bm).T @ V), G2  # eta dropped from the value
    return f


def _silu_prime_dropped_term(orig):
    return lambda a: L.sigmoid(a)  # s (1 + a (1 - s)) -> s


def _ns5_coefficient(orig):
    def f(G, eps):
        X = G / (np.linalg.norm(G) + eps)
        t = X.shape[0] > X.shape[1]
        X = X.T if t else X
        for _ in range(5):
            A = X @ X.T
            X = 3.4445 * X + (-4.70 * A + 2.0315 * (A @ A)) @ X
        return X.T if t else X
    return f


def _ns5_four_rounds(orig):
    def f(G, eps):
        X = G / (np.linalg.norm(G) + eps)
        t = X.shape[0] > X.shape[1]
        X = X.T if t else X
        for _ in range(4):
            A = X @ X.T
            X = 3.4445 * X + (-4.7750 * A + 2.0315 * (A @ A)) @ X
        return X.T if t else X
    return f


def _ns5_spectral_norm(orig):
    return lambda G, eps: orig(G * (np.linalg.norm(G) / np.linalg.norm(G, 2)), eps)


def _renorm_output_axis(orig):
    # norms of the rows (over the output axis), recycled to one factor per column
    return lambda W: np.resize(np.sqrt(np.sum(W * W, axis=1)), W.shape[1])


def _dampened_momentum(orig):
    def f(Q, K, V, eta, *a, momentum=0.0, **k):
        e = np.asarray(eta, dtype=np.float64) * ((1.0 - momentum) if momentum else 1.0)
        return orig(Q, K, V, e, *a, momentum=momentum, **k)
    return f


def _swapped_order(orig):
    return lambda *a, order=0, **k: orig(*a, order=1 - order, **k)


def _inclusive_prefix(orig):
    return lambda c, i, alpha, order: orig(c + (1 if order == 0 else 0), i, alpha, order) if i <= c else 0.0


def _momentum_exponent(orig):
    def f(c, i, alpha, order):
        last = c - 1 if order == 0 else c
        return float(sum(alpha ** (j - i + 1) for j in range(i, last + 1)))
    return f


def _update_before_apply(orig):
    def f(Hs, W_gate, W_up, W_down, Vbar, eta, *, chunk, dtype=np.float64):
        Hs, W_gate, W_up, W, Vbar = (np.asarray(a, dtype=dtype) for a in (Hs, W_gate, W_up, W_down, Vbar))
        W = W.copy()
        O = np.zeros((Hs.shape[0], W.shape[0]), dtype=dtype)
        for i in range(Hs.shape[0] // chunk):
            sl = slice(i * chunk, (i + 1) * chunk)
            Z = IP.gated_activation(Hs[sl], W_gate, W_up)
            W = W + eta * (Vbar[sl].T @ Z)
            O[sl] = Z @ W.T
        return O, W
    return f


def _drop_flag(bit):
    def mutate(orig):
        def f(*a, chunk_flags=None, **k):
            flags = None if chunk_flags is None else (np.asarray(chunk_flags).astype(np.int64) & ~bit)
            return orig(*a, chunk_flags=flags, **k)
        return f
    return mutate


def _one_inner_step(orig):
    def f(*a, inner_steps=1, **k):
        return orig(*a, **k)
    return f


def _eta_rows_swapped(orig):
    def f(Q, K, V, eta, *a, **k):
        eta = np.asarray(eta)
        return orig(Q, K, V, eta[[2, 1, 0]] if eta.ndim == 2 else eta, *a, **k)
    return f


def _target_taps_backward(orig):
    def f(X0, taps, W_target=None, dtype=np.float64):  # tap tau on X0_{t - tau} instead of X0_{t + tau}
        X0, taps = np.asarray(X0, dtype=dtype), np.asarray(taps, dtype=dtype)
        conv = np.zeros_like(X0)
        for tau in range(taps.shape[0]):
            conv[tau:] += taps[tau][None, :] * X0[:X0.shape[0] - tau]
        return conv if W_target is None else conv @ np.asarray(W_target, dtype=dtype).T
    return f


def _backward_silu_prime_dropped(orig):
    def f(A):
        sil, _ = orig(A)
        return sil, 0.5 * (1.0 + np.tanh(0.5 * A))  # silu' -> sigmoid
    return f


def _inplace_backward_no_write_term(orig):
    def f(Hs, W_gate, W_up, W_down, Vbar, eta, dO, *, chunk, dtype=np.float64):
        return orig(Hs, W_gate, W_up, W_down, np.zeros_like(np.asarray(Vbar)), eta, dO, chunk=chunk, dtype=dtype)
    return f


def _identity_scaled(orig):
    return lambda X, W0=None, W2=None: X / np.sqrt(X.shape[1])  # an attention-style 1/sqrt(h)


MUTATIONS = [
    # (label, module, attribute, mutation, pin that must fail)
    ("G0 sign flipped", L, "chunk_gradients", _flip_g0, lambda: TL.test_gradients_match_torch_autograd(3)),
    ("eta dropped from G1", L, "chunk_gradients", _g1_wrong_operand,
     lambda: TL.test_gradients_match_torch_autograd(4)),
    ("silu' term dropped", L, "silu_prime", _silu_prime_dropped_term,
     lambda: TL.test_gradients_match_central_finite_differences(0)),
    ("NS5 coefficient b", L, "newton_schulz5", _ns5_coefficient,
     lambda: TL.test_ns5_equals_singular_value_polynomial((8, 16))),
    ("NS5 four rounds", L, "newton_schulz5", _ns5_four_rounds, lambda: TL.test_ns5_rank_one_closed_form()),
    ("NS5 spectral pre-normalisation", L, "newton_schulz5", _ns5_spectral_norm,
     lambda: TL.test_ns5_equals_singular_value_polynomial((16, 8))),
    ("renorm over the output axis", L, "input_dim_norms", _renorm_output_axis,
     lambda: TL.test_renorm_keeps_initial_column_norms()),
    ("dampened momentum", L, "lact_pair", _dampened_momentum,
     lambda: TL.test_momentum_closed_form_when_only_w1_is_written()),
    ("update/apply order swapped", L, "lact_pair", _swapped_order,
     lambda: TL.test_causality_of_the_two_orders(0)),
    ("scan boundary inclusive", LA, "momentum_weight", _inclusive_prefix,
     lambda: TLA.test_scan_equals_masked_quadratic_form(0, 4)),
    ("momentum coefficient exponent", LA, "momentum_weight", _momentum_exponent,
     lambda: TLA.test_momentum_scan_equals_recurrent_heavy_ball(1, 0.5)),
    ("reset flag ignored", L, "lact_pair", _drop_flag(L.CHUNK_RESET),
     lambda: TLV.test_reset_equals_a_fresh_call(0)),
    ("apply-only flag ignored", L, "lact_pair", _drop_flag(L.CHUNK_NO_UPDATE),
     lambda: TLV.test_apply_only_chunk_equals_removing_its_writes(1)),
    ("inner steps ignored", L, "lact_pair", _one_inner_step,
     lambda: TLV.test_inner_steps_equal_repeated_chunks(0, 2)),
    ("eta rows of W0 and W2 swapped", L, "lact_pair", _eta_rows_swapped,
     lambda: TLV.test_eta_per_matrix_write_is_each_rows_autograd_gradient()),
    ("scan reset flag ignored", LA, "linattn_pair", _drop_flag(LA.CHUNK_RESET),
     lambda: TLA.test_scan_reset_equals_a_fresh_call(0, 0.8)),
    ("scan apply-only flag ignored", LA, "linattn_pair", _drop_flag(LA.CHUNK_NO_UPDATE),
     lambda: TLA.test_scan_apply_only_chunk_equals_removing_its_write(1, 0.0)),
    ("backward silu' term dropped", LA, "_silu_parts", _backward_silu_prime_dropped,
     lambda: TLA.test_backward_equals_torch_autograd(0, 0.0, False)),
    ("identity kernel rescaled", LA, "phi_identity", _identity_scaled,
     lambda: TLA.test_identity_scan_equals_recurrent_linear_fast_weight(0, 0.0, 8)),
    ("target taps on past tokens", IP, "lm_aligned_target", _target_taps_backward,
     lambda: TI.test_next_token_taps_with_identity_projection_are_the_next_token_shift()),
    ("In-Place backward without the writes' terms", IP, "inplace_backward_sequence",
     _inplace_backward_no_write_term, lambda: TI.test_backward_equals_torch_autograd(False)),
    ("target backward without the projection's transpose", IP, "lm_aligned_target_backward",
     lambda orig: (lambda X0, taps, Wt, dV, **k: orig(X0, taps, None if Wt is None else np.asarray(Wt).T, dV, **k)),
     lambda: TI.test_target_backward_equals_torch_autograd(True)),
    ("In-Place per-unit gradients without the writes", IP, "backward_hidden_units",
     lambda orig: (lambda Hs, Wg, Wu, Wd, Vb, eta, dO, units, **k: orig(Hs, Wg, Wu, Wd, Vb, 0.0, dO, units, **k)),
     lambda: TI.test_hidden_unit_gradients_equal_the_full_backward()),
    ("In-Place update before apply", IP, "inplace_sequence", _update_before_apply,
     lambda: TI.test_first_chunk_is_the_plain_mlp()),
]


@pytest.mark.parametrize("label,module,attr,mutate,pin", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pin_catches_planted_mistake(monkeypatch, label, module, attr, mutate, pin):
    pin()  # the pin passes on the oracle as it is
    monkeypatch.setattr(module, attr, mutate(getattr(module, attr)))
    with pytest.raises(AssertionError):
        pin()
