"""Oracle for the In-Place TTT down-projection update (test infrastructure only).

Source: "In-Place Test-Time Training" reading notes.

* Section 3.1, Eq. 2: the gated MLP output is
  O = (phi(H W_gate^T) * (H W_up^T)) W_down with phi = silu; W_gate and W_up
  are frozen slow weights and only W_down is a fast weight. Z is split into
  non-overlapping chunks of C tokens; chunk i applies O_[i] = Z_[i] W^(i)T and
  then updates W.
* Section 3.2, Eq. 4: with the loss -<., .>_F the update is
  W^(i+1) = W^(i) + eta Vbar_[i]^T Z_[i].
* Section 3.4: the update is associative, so all chunk deltas can be formed in
  parallel, prefix-summed (exclusive) and applied (the context-parallel form).

Reading of the transpose conventions (Eq. 2 writes "Z W_down", the chunk
steps and Eq. 4 write "Z W_down^T" and "Vbar^T Z"): W_down is
d_model x d_hidden, O = Z W_down^T, dW = eta Vbar^T Z -- three of the four
formulas agree on this.

* Section 3.2, Eq. 3 (the LM-aligned target): Vbar = Conv1D(X0) W_target with a
  1-D convolution over the sequence and a d_model x d_model projection; taps
  that put weight 1 on the next token and 0 elsewhere with W_target = I give
  the next-token target. Reading: the convolution is depthwise (one weight per
  channel and tap, the projection mixes the channels) and tap tau multiplies
  X0_{t+tau} (tau = 0 is the token itself, tau = 1 the next one), with zeros
  past the end of the sequence (section 3.4: the padding keeps the target
  within the sequence); W_target is given in nn.Linear layout [out, in], so
  Vbar_t = (sum_tau taps[tau] * X0_{t+tau}) W_target^T.
"""
from __future__ import annotations

from typing import Dict, Sequence

import numpy as np


def silu(a):
    return a * (0.5 * (1.0 + np.tanh(0.5 * a)))


def gated_activation(Hs, W_gate, W_up):
    """Z = silu(H W_gate^T) * (H W_up^T)  (section 3.1)."""
    return silu(Hs @ W_gate.T) * (Hs @ W_up.T)


def lm_aligned_target(X0, taps, W_target=None, dtype=np.float64):
    """Vbar [N, d_model] of one sequence from the token embeddings X0 [N, d_model], the
    depthwise taps [k, d_model] and W_target [d_model(out), d_model(in)] (None: identity)."""
    X0, taps = np.asarray(X0, dtype=dtype), np.asarray(taps, dtype=dtype)
    N = X0.shape[0]
    conv = np.zeros_like(X0)
    for tau in range(taps.shape[0]):
        conv[:N - tau] += taps[tau][None, :] * X0[tau:]
    return conv if W_target is None else conv @ np.asarray(W_target, dtype=dtype).T


def lm_aligned_target_backward(X0, taps, W_target, dVbar, dtype=np.float64):
    """Gradients of sum(Vbar * dVbar) of lm_aligned_target for one sequence: (dX0 [N, d_model],
    dtaps [k, d_model], dW_target [d_model, d_model] or None). With C = Conv1D(X0):
    dC = dVbar W_target (dVbar without a projection), dW_target = dVbar^T C,
    dX0[s] = sum_tau taps[tau] * dC[s - tau] (s - tau >= 0), dtaps[tau] = sum_t dC[t] * X0[t + tau]."""
    X0, taps, dV = (np.asarray(a, dtype=dtype) for a in (X0, taps, dVbar))
    N = X0.shape[0]
    conv = lm_aligned_target(X0, taps, None, dtype=dtype)
    if W_target is None:
        dC, dW = dV, None
    else:
        Wt = np.asarray(W_target, dtype=dtype)
        dC, dW = dV @ Wt, dV.T @ conv
    dX0 = np.zeros_like(X0)
    dtaps = np.zeros_like(taps)
    for tau in range(taps.shape[0]):
        dX0[tau:] += taps[tau][None, :] * dC[:N - tau]
        dtaps[tau] = (dC[:N - tau] * X0[tau:]).sum(axis=0)
    return dX0, dtaps, dW


def inplace_sequence(Hs, W_gate, W_up, W_down, Vbar, eta, *, chunk: int, dtype=np.float64):
    """Sequential chunk loop for one sequence. Returns (O [N,d_model], W_final)."""
    Hs, W_gate, W_up, W, Vbar = (np.asarray(a, dtype=dtype) for a in (Hs, W_gate, W_up, W_down, Vbar))
    W = W.copy()
    N = Hs.shape[0]
    O = np.zeros((N, W.shape[0]), dtype=dtype)
    for i in range(N // chunk):
        sl = slice(i * chunk, (i + 1) * chunk)
        Z = gated_activation(Hs[sl], W_gate, W_up)
        O[sl] = Z @ W.T
        W = W + eta * (Vbar[sl].T @ Z)
    return O, W


def inplace_prefix_form(Hs, W_gate, W_up, W_down, Vbar, eta, *, chunk: int, dtype=np.float64):
    """Context-parallel form (section 3.4): deltas, exclusive prefix sum, apply."""
    Hs, W_gate, W_up, W0, Vbar = (np.asarray(a, dtype=dtype) for a in (Hs, W_gate, W_up, W_down, Vbar))
    N = Hs.shape[0]
    n = N // chunk
    Z = [gated_activation(Hs[i * chunk:(i + 1) * chunk], W_gate, W_up) for i in range(n)]
    dW = [Vbar[i * chunk:(i + 1) * chunk].T @ Z[i] for i in range(n)]
    O = np.zeros((N, W0.shape[0]), dtype=dtype)
    prefix = np.zeros_like(W0)
    for i in range(n):
        O[i * chunk:(i + 1) * chunk] = Z[i] @ (W0 + eta * prefix).T
        prefix = prefix + dW[i]
    return O, W0 + eta * prefix


def inplace_forward(Hs, W_gate, W_up, W_down, Vbar, eta, *, chunk: int,
                    dtype=np.float64) -> Dict[str, np.ndarray]:
    """All sequences of a batch. Hs/Vbar [B,N,d_model]; W_down [d_model,d_hidden]
    shared (or [B,d_model,d_hidden] per sequence). Returns O and W_down final."""
    B = Hs.shape[0]
    per_seq = np.ndim(W_down) == 3
    outs, ws = [], []
    for b in range(B):
        o, w = inplace_sequence(Hs[b], W_gate, W_up, W_down[b] if per_seq else W_down, Vbar[b],
                                eta, chunk=chunk, dtype=dtype)
        outs.append(o)
        ws.append(w)
    return dict(O=np.stack(outs), W_down=np.stack(ws))


# --- sampled evaluation at sizes where the whole recurrence is too slow ------
def final_wdown_columns(Hs, W_gate, W_up, W_down, Vbar, eta, cols: Sequence[int],
                        dtype=np.float64) -> np.ndarray:
    """Columns of the final fast weight of one sequence:
    W_final[:, j] = W_down[:, j] + eta * sum_t Vbar[t] Z[t, j]  (Eq. 4 summed
    over all chunks). Only the needed hidden units of Z are formed."""
    cols = np.asarray(cols)
    Hs = np.asarray(Hs, dtype=dtype)
    Zc = gated_activation(Hs, np.asarray(W_gate[cols], dtype=dtype), np.asarray(W_up[cols], dtype=dtype))
    return np.asarray(W_down[:, cols], dtype=dtype) + eta * (np.asarray(Vbar, dtype=dtype).T @ Zc)


def output_rows(Hs, W_gate, W_up, W_down, Vbar, eta, *, chunk: int, rows: Sequence[int],
                dtype=np.float64) -> np.ndarray:
    """Selected output rows of one sequence: for t in chunk i,
    O[t] = Z[t] (W_down + eta * Vbar[:iC]^T Z[:iC])^T, evaluated as
    Z[t] W_down^T + eta * (Z[t] Z[:iC]^T) Vbar[:iC]."""
    rows = np.asarray(rows)
    last = int(rows.max()) // chunk
    Hs = np.asarray(Hs, dtype=dtype)
    Wg, Wu = np.asarray(W_gate, dtype=dtype), np.asarray(W_up, dtype=dtype)
    Zt = gated_activation(Hs[rows], Wg, Wu)
    out = Zt @ np.asarray(W_down, dtype=dtype).T
    if last > 0:
        Zp = gated_activation(Hs[:last * chunk], Wg, Wu)
        Vp = np.asarray(Vbar[:last * chunk], dtype=dtype)
        G = Zt @ Zp.T
        lim = (rows // chunk) * chunk
        G = G * (np.arange(last * chunk)[None, :] < lim[:, None])
        out = out + eta * (G @ Vp)
    return out


# ---- backward (the gradients the chunked update trains through) ----
# Forward per sequence: W_0 = W_down, Z_i = silu(A_i) * U_i with A_i = H_i W_gate^T,
# U_i = H_i W_up^T, O_i = Z_i W_i^T, W_{i+1} = W_i + eta Vbar_i^T Z_i. Given dL/dO:
#   G_i = dO_i^T Z_i            (the gradient reaching W_i through chunk i's output)
#   R_i = sum_{k > i} G_k       (the gradient reaching chunk i's write eta Vbar_i^T Z_i)
#   dW_down = sum_i G_i
#   dZ_i = dO_i W_i + eta Vbar_i R_i,   dVbar_i = eta Z_i R_i^T
#   dA = dZ * U * silu'(A),  dU = dZ * silu(A),  dH = dA W_gate + dU W_up,
#   dW_gate = sum dA^T H,  dW_up = sum dU^T H.

def inplace_backward_sequence(Hs, W_gate, W_up, W_down, Vbar, eta, dO, *, chunk: int, dtype=np.float64):
    """Gradients of sum(O * dO) for one sequence: dict(dH, dW_gate, dW_up, dW_down, dVbar)."""
    Hs, Wg, Wu, W, Vbar, dO = (np.asarray(a, dtype=dtype) for a in (Hs, W_gate, W_up, W_down, Vbar, dO))
    n = Hs.shape[0] // chunk
    sl = [slice(i * chunk, (i + 1) * chunk) for i in range(n)]
    A = [Hs[s] @ Wg.T for s in sl]
    U = [Hs[s] @ Wu.T for s in sl]
    Z = [silu(a) * u for a, u in zip(A, U)]
    Ws = [W.copy()]
    for i in range(n - 1):
        Ws.append(Ws[-1] + eta * (Vbar[sl[i]].T @ Z[i]))
    G = [dO[s].T @ z for s, z in zip(sl, Z)]
    out = dict(dH=np.zeros_like(Hs), dW_gate=np.zeros_like(Wg), dW_up=np.zeros_like(Wu),
               dW_down=sum(G, np.zeros_like(W)), dVbar=np.zeros_like(Vbar))
    R = np.zeros_like(W)
    for i in reversed(range(n)):
        dZ = dO[sl[i]] @ Ws[i] + eta * (Vbar[sl[i]] @ R)
        out["dVbar"][sl[i]] = eta * (Z[i] @ R.T)
        sg = 0.5 * (1.0 + np.tanh(0.5 * A[i]))
        dA = dZ * U[i] * sg * (1.0 + A[i] * (1.0 - sg))
        dU = dZ * A[i] * sg
        out["dH"][sl[i]] = dA @ Wg + dU @ Wu
        out["dW_gate"] += dA.T @ Hs[sl[i]]
        out["dW_up"] += dU.T @ Hs[sl[i]]
        R = R + G[i]
    return out


def inplace_backward(Hs, W_gate, W_up, W_down, Vbar, eta, dO, *, chunk: int,
                     dtype=np.float64) -> Dict[str, np.ndarray]:
    """All sequences: dH, dVbar [B,N,d_model]; dW_gate, dW_up summed over the batch; dW_down
    summed over the batch when W_down is shared ([d_model,d_hidden]), per sequence when it is
    [B,d_model,d_hidden]."""
    B = Hs.shape[0]
    per_seq = np.ndim(W_down) == 3
    res = [inplace_backward_sequence(Hs[b], W_gate, W_up, W_down[b] if per_seq else W_down, Vbar[b], eta, dO[b],
                                     chunk=chunk, dtype=dtype) for b in range(B)]
    out = {k: np.stack([r[k] for r in res]) for k in ("dH", "dVbar")}
    out["dW_gate"] = sum(r["dW_gate"] for r in res)
    out["dW_up"] = sum(r["dW_up"] for r in res)
    out["dW_down"] = np.stack([r["dW_down"] for r in res]) if per_seq else sum(r["dW_down"] for r in res)
    return out


def backward_hidden_units(Hs, W_gate, W_up, W_down, Vbar, eta, dO, units: Sequence[int], *, chunk: int,
                          dtype=np.float64) -> Dict[str, np.ndarray]:
    """dW_gate[j], dW_up[j] and dW_down[:, j] of one sequence for the hidden units j in `units`
    (dict of [len(units), d_model] arrays). Every quantity of unit j depends on column j of Z
    alone: W_i[:, j] = W_down[:, j] + eta sum_{k<i} Vbar_k^T Z_k[:, j],
    R_i[:, j] = sum_{k>i} dO_k^T Z_k[:, j], dZ_i[:, j] = dO_i W_i[:, j] + eta Vbar_i R_i[:, j],
    so sampled units cost O(N d_model) each at any d_hidden."""
    Hs, Vbar, dO = (np.asarray(a, dtype=dtype) for a in (Hs, Vbar, dO))
    n = Hs.shape[0] // chunk
    sl = [slice(i * chunk, (i + 1) * chunk) for i in range(n)]
    out = {k: np.zeros((len(units), Hs.shape[1]), dtype) for k in ("dW_gate", "dW_up", "dW_down")}
    for u_idx, j in enumerate(units):
        a = Hs @ np.asarray(W_gate[j], dtype)
        u = Hs @ np.asarray(W_up[j], dtype)
        z = silu(a) * u
        writes = [Vbar[s].T @ z[s] for s in sl]  # column j of Vbar_k^T Z_k
        g = [dO[s].T @ z[s] for s in sl]  # column j of G_k
        w = np.asarray(W_down[:, j], dtype).copy()
        r = sum(g[1:], np.zeros_like(w))
        dz = np.zeros_like(a)
        for i in range(n):
            dz[sl[i]] = dO[sl[i]] @ w + eta * (Vbar[sl[i]] @ r)
            w = w + eta * writes[i]
            if i + 1 < n:
                r = r - g[i + 1]
        sg = 0.5 * (1.0 + np.tanh(0.5 * a))
        out["dW_gate"][u_idx] = (dz * u * sg * (1.0 + a * (1.0 - sg))) @ Hs
        out["dW_up"][u_idx] = (dz * a * sg) @ Hs
        out["dW_down"][u_idx] = sum(g, np.zeros_like(w))
    return out
