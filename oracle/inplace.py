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
"""
from __future__ import annotations

from typing import Dict, Sequence

import numpy as np


def silu(a):
    return a * (0.5 * (1.0 + np.tanh(0.5 * a)))


def gated_activation(Hs, W_gate, W_up):
    """Z = silu(H W_gate^T) * (H W_up^T)  (section 3.1)."""
    return silu(Hs @ W_gate.T) * (Hs @ W_up.T)


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
