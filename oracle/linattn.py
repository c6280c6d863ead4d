"""Oracle for the last-layer-only linear-attention form (test infrastructure only).

Sources (cited by page title and section):

* "Test-Time Training with KV Binding Is Secretly Linear Attention" summary
  page, "Prerequisites -> Linear attention": o = phi(q) S with state
  S = S0 + sum_i phi(k_i)^T v_i; "Method step details" (Theorem 5.2): unrolled,
  W_{t+1} = W_0 + sum_i phi_i(k_i)^T g_i(k_i) with value g = -eta dL/df.
* Press article on the same paper, section 4 (parallelisation): when only the
  last layer is updated and there is no weight normalisation the kernel phi is
  static and the state update is associative, so a prefix scan replaces the
  sequential recurrence.

For the LaCT fast weight, phi(x) = silu(x W0) * (x W2) and the last layer is
W1, so with the loss -eta <f(k), v> the value is g = eta v and a chunk adds
dS_c = phi(K_c)^T diag(eta_c) V_c. Apply-then-update sees the exclusive prefix
(S_c = W1 + sum_{j<c} dS_j); update-then-apply the inclusive one (j <= c).
"""
from __future__ import annotations

from typing import Dict

import numpy as np

APPLY_THEN_UPDATE = 0
UPDATE_THEN_APPLY = 1


def phi(X: np.ndarray, W0: np.ndarray, W2: np.ndarray) -> np.ndarray:
    """The static feature map silu(X W0) * (X W2)."""
    A = X @ W0
    return A * (0.5 * (1.0 + np.tanh(0.5 * A))) * (X @ W2)


def linattn_pair(Q, K, V, eta, W0, W1, W2, *, chunk: int, order: int = APPLY_THEN_UPDATE,
                 dtype=np.float64):
    """Chunked linear attention for one pair. Returns (O, S_final)."""
    Q, K, V, eta, W0, W1, W2 = (np.asarray(a, dtype=dtype) for a in (Q, K, V, eta, W0, W1, W2))
    n_chunks = K.shape[0] // chunk
    dS = []
    for c in range(n_chunks):
        sl = slice(c * chunk, (c + 1) * chunk)
        dS.append(phi(K[sl], W0, W2).T @ (eta[sl, None] * V[sl]))
    O = np.zeros((Q.shape[0], W1.shape[1]), dtype=dtype)
    S = W1.copy()
    for c in range(n_chunks):
        sl = slice(c * chunk, (c + 1) * chunk)
        if order == UPDATE_THEN_APPLY:
            S = S + dS[c]
        O[sl] = phi(Q[sl], W0, W2) @ S
        if order == APPLY_THEN_UPDATE:
            S = S + dS[c]
    return O, S


def linattn_forward(Q, K, V, eta, W0, W1, W2, *, chunk: int, order: int = APPLY_THEN_UPDATE,
                    pairs=None, dtype=np.float64) -> Dict[str, np.ndarray]:
    """All pairs. Q/K/V [B,H,N,h], eta [B,H,N], W0/W2 [H,h,rh], W1 [H,rh,h]
    (or [B,H,...] per sequence). Returns O [B,H,N,h] and S [B,H,rh,h]."""
    B, H, N, h = Q.shape
    per_seq = np.ndim(W0) == 4
    rh = W0.shape[-1]
    O = np.full((B, H, N, h), np.nan, dtype=dtype)
    S = np.full((B, H, rh, h), np.nan, dtype=dtype)
    todo = pairs if pairs is not None else [(b, hd) for b in range(B) for hd in range(H)]
    for (b, hd) in todo:
        w0, w1, w2 = ((w[b, hd] if per_seq else w[hd]) for w in (W0, W1, W2))
        O[b, hd], S[b, hd] = linattn_pair(Q[b, hd], K[b, hd], V[b, hd], eta[b, hd], w0, w1, w2,
                                          chunk=chunk, order=order, dtype=dtype)
    return dict(O=O, S=S)


def linattn_masked_quadratic(Q, K, V, eta, W0, W1, W2, *, chunk: int, order: int = APPLY_THEN_UPDATE,
                             dtype=np.float64) -> np.ndarray:
    """The parallel matrix form for one pair on small N:
    O = phi(Q) W1 + (M * phi(Q) phi(K)^T) diag(eta) V with the chunk mask
    M[t, s] = 1 iff chunk(s) < chunk(t) (apply-then-update) or <= (update-then-apply).

    Press article, section 4: the parallel form built from a block mask, a
    learning-rate vector and scaled values.
    """
    Q, K, V, eta, W0, W1, W2 = (np.asarray(a, dtype=dtype) for a in (Q, K, V, eta, W0, W1, W2))
    ct = np.arange(Q.shape[0]) // chunk
    cs = np.arange(K.shape[0]) // chunk
    mask = (cs[None, :] < ct[:, None]) if order == APPLY_THEN_UPDATE else (cs[None, :] <= ct[:, None])
    pq, pk = phi(Q, W0, W2), phi(K, W0, W2)
    return pq @ W1 + (mask * (pq @ pk.T)) @ (eta[:, None] * V)
