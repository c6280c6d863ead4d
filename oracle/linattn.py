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


CHUNK_NO_UPDATE, CHUNK_RESET = 1, 2  # per-chunk flags, as in the LaCT loop


def linattn_pair(Q, K, V, eta, W0, W1, W2, *, chunk: int, order: int = APPLY_THEN_UPDATE,
                 momentum: float = 0.0, feature_map: str = "swiglu", chunk_flags=None, dtype=np.float64):
    """Chunked linear attention for one pair. Returns (O, S_final); S_final is the state
    after the last chunk's write. feature_map "identity": phi(x) = x, W1 is h x h.

    chunk_flags (one per chunk; the LaCT loop's apply-only and reset flags, read for the scan
    form): an apply-only chunk writes nothing and takes no momentum step; a reset chunk starts
    from W1 with zero momentum, as a fresh call would. With flags the states follow the
    heavy-ball recurrence chunk by chunk (m <- alpha m + dS_c, S <- S + m)."""
    Q, K, V, eta, W0, W1, W2 = (_as(a, dtype) for a in (Q, K, V, eta, W0, W1, W2))
    feat = feature_map_fn(feature_map)
    n_chunks = K.shape[0] // chunk
    dS = []
    for c in range(n_chunks):
        sl = slice(c * chunk, (c + 1) * chunk)
        dS.append(feat(K[sl], W0, W2).T @ (eta[sl, None] * V[sl]))
    if chunk_flags is not None:
        O = np.zeros((Q.shape[0], W1.shape[1]), dtype=dtype)
        S, m = W1.copy(), np.zeros_like(W1)
        for c in range(n_chunks):
            f = int(chunk_flags[c])
            if f & CHUNK_RESET:
                S, m = W1.copy(), np.zeros_like(W1)
            write = not f & CHUNK_NO_UPDATE
            if order == UPDATE_THEN_APPLY and write:
                m = momentum * m + dS[c]
                S = S + m
            sl = slice(c * chunk, (c + 1) * chunk)
            O[sl] = feat(Q[sl], W0, W2) @ S
            if order == APPLY_THEN_UPDATE and write:
                m = momentum * m + dS[c]
                S = S + m
        return O, S

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
                    momentum: float = 0.0, feature_map: str = "swiglu", pairs=None, chunk_flags=None,
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
                                          feature_map=feature_map, dtype=dtype,
                                          chunk_flags=None if chunk_flags is None else chunk_flags[b])
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


# ---- backward of the scan form (the gradients the parallel form trains through) ----
# The forward above is O_c = phi(Q_c) S_c with S_c = W1 + sum_j w(c, j) dS_j,
# dS_j = phi(K_j)^T diag(eta_j) V_j and w = momentum_weight. Given dL/dO:
#   G_c = phi(Q_c)^T dO_c                       (the gradient reaching S_c)
#   dW1 = sum_c G_c
#   R_j = sum_c w(c, j) G_c                     (the gradient reaching dS_j)
#   dphi(Q_c) = dO_c S_c^T
#   dphi(K_j) = diag(eta_j) V_j R_j^T,   d(eta V)_j = phi(K_j) R_j
#   dV_t = eta_t d(eta V)_t,   deta_t = <d(eta V)_t, V_t>
# and through phi(X) = silu(A) * Bm with A = X W0, Bm = X W2:
#   dA = dphi * Bm * silu'(A),  dBm = dphi * silu(A),  dX = dA W0^T + dBm W2^T,
#   dW0 = sum X^T dA,  dW2 = sum X^T dBm  (over the queries and the keys).

def _silu_parts(A):
    s = 0.5 * (1.0 + np.tanh(0.5 * A))
    return A * s, s * (1.0 + A * (1.0 - s))  # silu(A), silu'(A)


def linattn_backward_pair(Q, K, V, eta, W0, W1, W2, dO, *, chunk: int, order: int = APPLY_THEN_UPDATE,
                          momentum: float = 0.0, feature_map: str = "swiglu", dtype=np.float64):
    """Gradients of sum(O * dO) for one pair: dict(dQ, dK, dV, deta, dW0, dW1, dW2); dW0/dW2 are
    None for the identity map."""
    Q, K, V, eta, W0, W1, W2, dO = (_as(a, dtype) for a in (Q, K, V, eta, W0, W1, W2, dO))
    ident = feature_map == "identity"
    n = K.shape[0] // chunk
    sl = [slice(c * chunk, (c + 1) * chunk) for c in range(n)]

    def feat(X):
        if ident:
            return X, None, None
        A, Bm = X @ W0, X @ W2
        sil, dsil = _silu_parts(A)
        return sil * Bm, (A, Bm, sil, dsil), X

    def feat_back(dphi, cache, X):
        if ident:
            return dphi, None, None
        A, Bm, sil, dsil = cache
        dA, dBm = dphi * Bm * dsil, dphi * sil
        return dA @ W0.T + dBm @ W2.T, X.T @ dA, X.T @ dBm

    fq = [feat(Q[s]) for s in sl]
    fk = [feat(K[s]) for s in sl]
    dS = [fk[c][0].T @ (eta[sl[c], None] * V[sl[c]]) for c in range(n)]
    S = [W1 + sum((momentum_weight(c, j, momentum, order) * dS[j] for j in range(n)), np.zeros_like(W1))
         for c in range(n)]
    G = [fq[c][0].T @ dO[sl[c]] for c in range(n)]
    R = [sum((momentum_weight(c, j, momentum, order) * G[c] for c in range(n)), np.zeros_like(W1)) for j in range(n)]
    out = dict(dQ=np.zeros_like(Q), dK=np.zeros_like(K), dV=np.zeros_like(V), deta=np.zeros_like(eta),
               dW1=sum(G, np.zeros_like(W1)),
               dW0=None if ident else np.zeros_like(W0), dW2=None if ident else np.zeros_like(W2))
    for c in range(n):
        dX, g0, g2 = feat_back(dO[sl[c]] @ S[c].T, fq[c][1], fq[c][2])
        out["dQ"][sl[c]] = dX
        dEV = fk[c][0] @ R[c]
        out["dV"][sl[c]] = eta[sl[c], None] * dEV
        out["deta"][sl[c]] = np.sum(dEV * V[sl[c]], axis=1)
        dX, h0, h2 = feat_back((eta[sl[c], None] * V[sl[c]]) @ R[c].T, fk[c][1], fk[c][2])
        out["dK"][sl[c]] = dX
        if not ident:
            out["dW0"] += g0 + h0
            out["dW2"] += g2 + h2
    return out


def linattn_backward(Q, K, V, eta, W0, W1, W2, dO, *, chunk: int, order: int = APPLY_THEN_UPDATE,
                     momentum: float = 0.0, feature_map: str = "swiglu", dtype=np.float64) -> Dict[str, np.ndarray]:
    """All pairs: dQ, dK, dV [B,H,N,h], deta [B,H,N]; the weight gradients in the weights' own
    layout, summed over the batch when the weights are shared ([H,...]) and per sequence when
    they are [B,H,...]."""
    B, H, N, h = Q.shape
    per_seq = np.ndim(W1) == 4
    res = {k: [] for k in ("dQ", "dK", "dV", "deta", "dW0", "dW1", "dW2")}
    for b in range(B):
        for hd in range(H):
            w0, w1, w2 = ((None if w is None else (w[b, hd] if per_seq else w[hd])) for w in (W0, W1, W2))
            r = linattn_backward_pair(Q[b, hd], K[b, hd], V[b, hd], eta[b, hd], w0, w1, w2, dO[b, hd], chunk=chunk,
                                      order=order, momentum=momentum, feature_map=feature_map, dtype=dtype)
            for k in res:
                res[k].append(r[k])
    out = {k: np.stack(res[k]).reshape((B, H) + res[k][0].shape) for k in ("dQ", "dK", "dV", "deta")}
    for k in ("dW0", "dW1", "dW2"):
        if res[k][0] is None:
            out[k] = None
            continue
        g = np.stack(res[k]).reshape((B, H) + res[k][0].shape)
        out[k] = g if per_seq else g.sum(axis=0)
    return out
