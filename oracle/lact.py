"""Oracle for the chunked LaCT fast-weight layer (test infrastructure only).

Sources (cited by page title and section):

* "Test-Time Training with KV Binding Is Secretly Linear Attention" summary
  page, section "Prerequisites -> LaCT": the fast weight is a bias-free SwiGLU
  MLP f(x) = (silu(x W0) * (x W2)) W1 in row-vector form, the inner loss is the
  negative Frobenius inner product -<f(k), v>, with per-token learning rate
  eta_t, momentum and a Muon-style orthogonalisation of the update.
* "Test-Time Training Done Right" reading notes:
  - section 2.1 (symbols): per-token positive update weights eta_i, chunk size b;
  - section 2.2 (from gradient write to Muon write): each matrix is
    renormalised along its input dimension back to the original weight's norm;
    Muon approximates U V^T of g = U S V^T with five Newton-Schulz rounds with
    coefficients 3.4445, -4.7750, 2.0315; with momentum, M is fed to the
    update operator;
  - section 2.3 (update order): language models apply the history state to
    the current chunk and then update with it; sets / view synthesis update
    first and then apply.
* "In-Place Test-Time Training" notes, TTT review (Eq. 1): W <- W - eta grad L,
  then apply; section 3.1: all tokens of a chunk take their gradient at the
  chunk-start weights.

Readings (the pages' formulas for the loss, the update operators and the
momentum are lost in extraction; these are the plainest readings the rest
supports):

1. Row form, W0/W2 h x rh, W1 rh x h (the summary page's notation).
2. Loss of a chunk: L = -sum_i eta_i <f(k_i), v_i>; descent W <- W - U.
3. One eta per token and head, shared by the three matrices.
4. All tokens of a chunk use the chunk-start weights; the three matrices are
   updated simultaneously from one gradient of the same loss.
5. Momentum is heavy ball per chunk: M <- alpha M + G, M0 = 0, U = M.
6. Newton-Schulz-5: X = G / (||G||_F + eps); work on the wide orientation;
   five times A = X X^T, B = b A + c A A, X = a X + B X.
7. Pipeline: G -> momentum -> NS5 -> subtract -> renorm. The momentum buffer
   is not renormalised.
8. Renorm target nu = column norms of the weights at the start of the call;
   W[:, j] <- W[:, j] * nu_j / (||W[:, j]||_2 + eps_norm), only for updated
   matrices.
9. Input axis = axis 0 of the row-form matrices (each output column is
   normalised over its inputs).

Variants of the same loop (the reading notes' section 2.3 update-order table
and section 2.4; the In-Place notes, section 3.4; the notes' section 2.1 symbol
table; the KV-binding summary page, "Motivation", on more inner-loop
iterations):

10. Per-chunk write mask: an apply-only chunk (the autoregressive-video row's
    noisy chunks) is applied with the current weights and writes nothing:
    weights and momentum are left as they are.
11. Per-chunk reset (a document boundary inside a packed sequence): before the
    chunk is applied or written, the weights return to the call's initial
    weights and the momentum to zero, as if a new call started there.
12. eta per matrix ("may be predicted separately for the three matrices"): the
    gradient of matrix X is that of the chunk loss weighted by eta_X,
    L_X = -sum_i eta_{X,i} <f(k_i), v_i>; one eta shared by the three is the
    default.
13. Several inner steps per chunk: the chunk's write (gradient at the current
    weights, momentum, Newton-Schulz, subtract, renorm) is repeated that many
    times on the same tokens; apply-then-update applies before the first step,
    update-then-apply after the last.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

NS_A, NS_B, NS_C = 3.4445, -4.7750, 2.0315
NS_STEPS = 5

APPLY_THEN_UPDATE = 0
UPDATE_THEN_APPLY = 1
UPD_W0, UPD_W1, UPD_W2 = 1, 2, 4
CHUNK_NO_UPDATE, CHUNK_RESET = 1, 2  # per-chunk flags (readings 10, 11)


def sigmoid(a: np.ndarray) -> np.ndarray:
    return 0.5 * (1.0 + np.tanh(0.5 * a))


def silu(a: np.ndarray) -> np.ndarray:
    """silu(a) = a * sigmoid(a)."""
    return a * sigmoid(a)


def silu_prime(a: np.ndarray) -> np.ndarray:
    """d silu / da = s + a s (1 - s) with s = sigmoid(a)."""
    s = sigmoid(a)
    return s * (1.0 + a * (1.0 - s))


def swiglu_apply(X: np.ndarray, W0: np.ndarray, W1: np.ndarray, W2: np.ndarray) -> np.ndarray:
    """f(X) = (silu(X W0) * (X W2)) W1, row-wise over the tokens of X.

    Summary page, "Prerequisites -> LaCT": the bias-free SwiGLU fast weight.
    """
    return (silu(X @ W0) * (X @ W2)) @ W1


def chunk_gradients(K: np.ndarray, V: np.ndarray, eta: np.ndarray,
                    W0: np.ndarray, W1: np.ndarray, W2: np.ndarray):
    """Gradients of L = -sum_i eta_i <f(k_i), v_i> w.r.t. W0, W1, W2.

    Reading 2 of the loss (summary page, "Prerequisites -> LaCT" and the
    step-detail passage: the value of the linear-attention form is
    g = -eta dL/df = eta v). With F = H W1, H = silu(A) * Bm, A = K W0,
    Bm = K W2 and Vt = diag(eta) V, the chain rule gives
        dL/dF  = -Vt
        dL/dW1 = -H^T Vt
        dL/dH  = -Vt W1^T              (=: -D)
        dL/dA  = -D * Bm * silu'(A)    (=: -X0)
        dL/dBm = -D * silu(A)          (=: -X2)
        dL/dW0 = -K^T X0,  dL/dW2 = -K^T X2.
    Returns (G0, G1, G2) with the shapes of (W0, W1, W2).
    """
    A = K @ W0
    Bm = K @ W2
    Vt = eta[:, None] * V
    D = Vt @ W1.T
    Hm = silu(A) * Bm
    X0 = D * Bm * silu_prime(A)
    X2 = D * silu(A)
    G1 = -(Hm.T @ Vt)
    G0 = -(K.T @ X0)
    G2 = -(K.T @ X2)
    return G0, G1, G2


def chunk_loss(K, V, eta, W0, W1, W2) -> float:
    """L = -sum_i eta_i <f(k_i), v_i> (used by the finite-difference pin)."""
    F = swiglu_apply(K, W0, W1, W2)
    return float(-np.sum(eta[:, None] * F * V))


def newton_schulz5(G: np.ndarray, eps: float) -> np.ndarray:
    """Five Newton-Schulz rounds approximating the orthogonal factor of G.

    "Test-Time Training Done Right" notes, section 2.2 (Appendix A of the
    paper): coefficients (3.4445, -4.7750, 2.0315), five rounds. Reading 6:
    Frobenius pre-normalisation with eps, iteration on the wide orientation.
    """
    X = G / (np.linalg.norm(G) + eps)
    transposed = X.shape[0] > X.shape[1]
    if transposed:
        X = X.T
    for _ in range(NS_STEPS):
        A = X @ X.T
        Bq = NS_B * A + NS_C * (A @ A)
        X = NS_A * X + Bq @ X
    return X.T if transposed else X


def input_dim_norms(W: np.ndarray) -> np.ndarray:
    """Column norms over the input axis (axis 0) of a row-form weight."""
    return np.sqrt(np.sum(W * W, axis=0))


def renorm_input_dim(W: np.ndarray, nu: np.ndarray, eps: float) -> np.ndarray:
    """W[:, j] * nu_j / (||W[:, j]|| + eps) -- notes section 2.2 (reading 8, 9)."""
    return W * (nu / (input_dim_norms(W) + eps))[None, :]


def lact_pair(Q: np.ndarray, K: np.ndarray, V: np.ndarray, eta: np.ndarray,
              W0: np.ndarray, W1: np.ndarray, W2: np.ndarray, *,
              chunk_q: int, chunk_kv: int, order: int = APPLY_THEN_UPDATE,
              update_mask: int = 7, weight_norm: bool = True, muon: bool = False,
              momentum: float = 0.0, eps_norm: float = 1e-5, eps_ns: float = 1e-7,
              M_in: Optional[Dict[str, np.ndarray]] = None, ascent: bool = False,
              chunk_flags=None, inner_steps: int = 1, dtype=np.float64):
    """The chunk recurrence for one (sequence, head) pair.

    Steps per chunk c (notes section 2.3 for the order; section 2.2 for the
    update operators; In-Place notes section 3.1 for chunk-start gradients):
      AU: O_c = f_W(Q_c), then update W with (K_c, V_c, eta_c);
      UA: update first, then O_c = f_W(Q_c).
    ``ascent`` flips the sign of the write (summary page, "Experimental
    results": gradient ascent in the inner loop). ``eta`` is [Nk] (shared) or
    [3, Nk] (one row per matrix W0, W1, W2; reading 12). ``chunk_flags`` holds
    one CHUNK_NO_UPDATE / CHUNK_RESET bit set per chunk (readings 10, 11);
    ``inner_steps`` writes per chunk (reading 13).
    Returns (O, W0, W1, W2, M) with M = {"W0":..., "W1":..., "W2":...}.
    """
    Q, K, V, eta = (np.asarray(a, dtype=dtype) for a in (Q, K, V, eta))
    init = {"W0": np.array(W0, dtype=dtype), "W1": np.array(W1, dtype=dtype),
            "W2": np.array(W2, dtype=dtype)}
    W = {n: w.copy() for n, w in init.items()}
    bits = {"W0": UPD_W0, "W1": UPD_W1, "W2": UPD_W2}
    updated = [n for n in ("W0", "W1", "W2") if update_mask & bits[n]]
    nu = {n: input_dim_norms(W[n]) for n in updated}
    M = {n: (np.array(M_in[n], dtype=dtype) if M_in is not None else np.zeros_like(W[n]))
         for n in ("W0", "W1", "W2")}
    n_chunks = K.shape[0] // chunk_kv
    assert Q.shape[0] // chunk_q == n_chunks
    O = np.zeros((Q.shape[0], W["W1"].shape[1]), dtype=dtype)

    def apply(c):
        q = Q[c * chunk_q:(c + 1) * chunk_q]
        O[c * chunk_q:(c + 1) * chunk_q] = swiglu_apply(q, W["W0"], W["W1"], W["W2"])

    def gradients(sl):
        """The chunk loss's gradients; with one eta row per matrix, each matrix's gradient of
        the loss weighted by its own eta (reading 12)."""
        if eta.ndim == 1:
            return dict(zip(("W0", "W1", "W2"), chunk_gradients(K[sl], V[sl], eta[sl], W["W0"], W["W1"], W["W2"])))
        per = [chunk_gradients(K[sl], V[sl], eta[x, sl], W["W0"], W["W1"], W["W2"]) for x in range(3)]
        return {"W0": per[0][0], "W1": per[1][1], "W2": per[2][2]}

    for c in range(n_chunks):
        flag = 0 if chunk_flags is None else int(chunk_flags[c])
        if flag & CHUNK_RESET:
            W = {n: w.copy() for n, w in init.items()}
            M = {n: np.zeros_like(w) for n, w in init.items()}
        if order == APPLY_THEN_UPDATE:
            apply(c)
        sl = slice(c * chunk_kv, (c + 1) * chunk_kv)
        for _ in range(0 if flag & CHUNK_NO_UPDATE else inner_steps):
            G = gradients(sl)
            for n in updated:
                U = G[n]
                if momentum != 0.0:
                    M[n] = momentum * M[n] + G[n]
                    U = M[n]
                if muon:
                    U = newton_schulz5(U, eps_ns)
                W[n] = W[n] + U if ascent else W[n] - U
                if weight_norm:
                    W[n] = renorm_input_dim(W[n], nu[n], eps_norm)
        if order == UPDATE_THEN_APPLY:
            apply(c)
    return O, W["W0"], W["W1"], W["W2"], M


def lact_forward(Q, K, V, eta, W0, W1, W2, *, chunk_q, chunk_kv, order=APPLY_THEN_UPDATE,
                 update_mask=7, weight_norm=True, muon=False, momentum=0.0,
                 eps_norm=1e-5, eps_ns=1e-7, M_in=None, pairs=None, ascent=False,
                 chunk_flags=None, inner_steps=1, dtype=np.float64) -> Dict[str, np.ndarray]:
    """All (sequence, head) pairs of a call; each pair is independent.

    Q [B,H,Nq,h], K/V [B,H,Nk,h], eta [B,H,Nk] (or [B,H,3,Nk], one row per
    matrix); W0/W2 [H,h,rh] and W1 [H,rh,h] shared across the batch, or
    [B,H,...] per sequence. ``M_in`` (optional) is a dict of [B,H,...] momentum
    buffers. ``chunk_flags`` (optional) is [B, n_chunks]: one flag set per
    sequence and chunk, shared by its heads. ``pairs`` restricts the computation
    to a list of (b, head) pairs; the outputs of other pairs are left as NaN.
    """
    B, H, Nq, h = Q.shape
    per_seq = np.ndim(W0) == 4
    rh = W0.shape[-1]
    O = np.full((B, H, Nq, h), np.nan, dtype=dtype)
    Wout = {n: np.full((B, H) + np.shape(w)[-2:], np.nan, dtype=dtype)
            for n, w in (("W0", W0), ("W1", W1), ("W2", W2))}
    Mout = {n: np.full_like(Wout[n], np.nan) for n in Wout}
    todo = pairs if pairs is not None else [(b, hd) for b in range(B) for hd in range(H)]
    for (b, hd) in todo:
        w = [(w4[b, hd] if per_seq else w4[hd]) for w4 in (W0, W1, W2)]
        m_in = None if M_in is None else {n: M_in[n][b, hd] for n in ("W0", "W1", "W2")}
        o, w0, w1, w2, m = lact_pair(
            Q[b, hd], K[b, hd], V[b, hd], eta[b, hd], w[0], w[1], w[2],
            chunk_q=chunk_q, chunk_kv=chunk_kv, order=order, update_mask=update_mask,
            weight_norm=weight_norm, muon=muon, momentum=momentum, eps_norm=eps_norm,
            eps_ns=eps_ns, M_in=m_in, ascent=ascent,
            chunk_flags=None if chunk_flags is None else chunk_flags[b], inner_steps=inner_steps, dtype=dtype)
        O[b, hd] = o
        Wout["W0"][b, hd], Wout["W1"][b, hd], Wout["W2"][b, hd] = w0, w1, w2
        for n in Mout:
            Mout[n][b, hd] = m[n]
    assert rh == Wout["W0"].shape[-1]
    return dict(O=O, W0=Wout["W0"], W1=Wout["W1"], W2=Wout["W2"],
                M0=Mout["W0"], M1=Mout["W1"], M2=Mout["W2"])
