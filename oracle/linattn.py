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

With momentum (same summary page, Theorem 5.3) the value written at step i is
carried into every later state with the cumulative coefficient
beta_{ji}, so the effective write is dS_i * sum_{j=i}^{t} beta_{ji}. Reading:
one heavy-ball step per chunk with a constant coefficient alpha, so
beta_{ji} = alpha^(j-i) and the state that chunk c reads is
S_c = W1 + sum_{i<c} dS_i sum_{j=i}^{c-1} alpha^(j-i) (apply-then-update; the
inner sums run to c, and i <= c, for update-then-apply). alpha = 0 gives the
plain prefix above.

Variant 3 of the same summary page's simplification ladder ("Method step
details", step 3: the multi-layer fast weight becomes one linear layer) has
f(x) = x W with W in R^{h x h}: the kernel is the identity, phi(x) = x, and the
state S (= W) is h x h. The form above holds with phi(K_c) = K_c; the
feature_map="identity" option computes it (W0 and W2 are then unused).
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


def phi_identity(X: np.ndarray, W0=None, W2=None) -> np.ndarray:
    """Variant 3's kernel: the input itself (a single linear fast-weight layer)."""
    return X


def feature_map_fn(name: str):
    """The kernel named by feature_map: "swiglu" (phi above) or "identity"."""
    return {"swiglu": phi, "identity": phi_identity}[name]


def momentum_weight(c: int, i: int, alpha: float, order: int) -> float:
    """Theorem 5.3's cumulative coefficient of chunk i's write in the state chunk c reads:
    sum_{j=i}^{last} alpha^(j-i) with last = c-1 (apply-then-update) or c (update-then-apply);
    zero when chunk i comes after that."""
    last = c - 1 if order == APPLY_THEN_UPDATE else c
    return float(sum(alpha ** (j - i) for j in range(i, last + 1)))


def _as(a, dtype):
    return None if a is None else np.asarray(a, dtype=dtype)


def linattn_pair(Q, K, V, eta, W0, W1, W2, *, chunk: int, order: int = APPLY_THEN_UPDATE,
                 momentum: float = 0.0, feature_map: str = "swiglu", dtype=np.float64):
    """Chunked linear attention for one pair. Returns (O, S_final); S_final is the state
    after the last chunk's write. feature_map "identity": phi(x) = x, W1 is h x h."""
    Q, K, V, eta, W0, W1, W2 = (_as(a, dtype) for a in (Q, K, V, eta, W0, W1, W2))
    feat = feature_map_fn(feature_map)
    n_chunks = K.shape[0] // chunk
    dS = []
    for c in range(n_chunks):
        sl = slice(c * chunk, (c + 1) * chunk)
        dS.append(feat(K[sl], W0, W2).T @ (eta[sl, None] * V[sl]))

    def state(c, ord_):
        S = W1.copy()
        for i in range(n_chunks):
            w = momentum_weight(c, i, momentum, ord_)
            if w != 0.0:
                S = S + w * dS[i]
        return S

    O = np.zeros((Q.shape[0], W1.shape[1]), dtype=dtype)
    for c in range(n_chunks):
        sl = slice(c * chunk, (c + 1) * chunk)
        O[sl] = feat(Q[sl], W0, W2) @ state(c, order)
    return O, state(n_chunks - 1, UPDATE_THEN_APPLY) if n_chunks else W1.copy()


def linattn_forward(Q, K, V, eta, W0, W1, W2, *, chunk: int, order: int = APPLY_THEN_UPDATE,
                    momentum: float = 0.0, feature_map: str = "swiglu", pairs=None,
                    dtype=np.float64) -> Dict[str, np.ndarray]:
    """All pairs. Q/K/V [B,H,N,h], eta [B,H,N], W0/W2 [H,h,rh], W1 [H,rh,h]
    (or [B,H,...] per sequence). Returns O [B,H,N,h] and S [B,H,rh,h]. With
    feature_map "identity" W0/W2 are unused (None) and W1 is [(B,)H,h,h]."""
    B, H, N, h = Q.shape
    per_seq = np.ndim(W1) == 4
    rh = W1.shape[-2]
    O = np.full((B, H, N, h), np.nan, dtype=dtype)
    S = np.full((B, H, rh, h), np.nan, dtype=dtype)
    todo = pairs if pairs is not None else [(b, hd) for b in range(B) for hd in range(H)]
    for (b, hd) in todo:
        w0, w1, w2 = ((None if w is None else (w[b, hd] if per_seq else w[hd])) for w in (W0, W1, W2))
        O[b, hd], S[b, hd] = linattn_pair(Q[b, hd], K[b, hd], V[b, hd], eta[b, hd], w0, w1, w2,
                                          chunk=chunk, order=order, momentum=momentum,
                                          feature_map=feature_map, dtype=dtype)
    return dict(O=O, S=S)


def linattn_masked_quadratic(Q, K, V, eta, W0, W1, W2, *, chunk: int, order: int = APPLY_THEN_UPDATE,
                             momentum: float = 0.0, feature_map: str = "swiglu",
                             dtype=np.float64) -> np.ndarray:
    """The parallel matrix form for one pair on small N:
    O = phi(Q) W1 + (M * phi(Q) phi(K)^T) diag(eta) V with the chunk mask
    M[t, s] = 1 iff chunk(s) < chunk(t) (apply-then-update) or <= (update-then-apply);
    with momentum M[t, s] is the cumulative coefficient of chunk(s) seen from chunk(t).

    Press article, section 4: the parallel form built from a block mask, a
    learning-rate vector and scaled values.
    """
    Q, K, V, eta, W0, W1, W2 = (_as(a, dtype) for a in (Q, K, V, eta, W0, W1, W2))
    feat = feature_map_fn(feature_map)
    ct = np.arange(Q.shape[0]) // chunk
    cs = np.arange(K.shape[0]) // chunk
    if momentum == 0.0:
        mask = (cs[None, :] < ct[:, None]) if order == APPLY_THEN_UPDATE else (cs[None, :] <= ct[:, None])
    else:
        mask = np.array([[momentum_weight(a, b, momentum, order) for b in cs] for a in ct])
    pq, pk = feat(Q, W0, W2), feat(K, W0, W2)
    return pq @ W1 + (mask * (pq @ pk.T)) @ (eta[:, None] * V)
