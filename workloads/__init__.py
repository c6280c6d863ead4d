"""Seeded synthetic inputs for the chunked TTT-KVB fast-weight layer.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark. It draws random numbers and shapes them; it holds none of the
method's arithmetic (no fast-weight apply, gradient, orthogonalisation, scan or
update). Everything here is input preparation:

* draws from ``numpy.random.default_rng(seed)`` (PCG64) in a fixed order;
* per-token L2 normalisation of Q/K(/V) over the head dimension;
* per-token step sizes ``eta = 0.01 * softplus(N(0, 1))``;
* round-to-nearest-even conversion to bfloat16 for bf16 problems, so that the
  oracle and the GPU consume bit-identical values.

Problem shapes follow the pages' workloads: the LaCT language-model layer
(seq 32768, chunk 2048; "Test-Time Training Done Right" notes, sections 2.3 and
3), the novel-view-synthesis scene (48 views of 512x512 with 8x8 patches plus a
~4096-token target; same notes, section 4.1 / Table 2) and the In-Place TTT MLP
(32k context, chunk 1024; "In-Place Test-Time Training" notes, section 3.1).
No dataset item is reproduced: all values are Gaussian draws.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

APPLY_THEN_UPDATE = 0
UPDATE_THEN_APPLY = 1
FP32 = 0
BF16 = 1

UPD_W0, UPD_W1, UPD_W2 = 1, 2, 4
UPD_ALL = UPD_W0 | UPD_W1 | UPD_W2


# ----------------------------------------------------------------------------
# bfloat16 conversion (round to nearest, ties to even)
# ----------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bit patterns of the nearest bfloat16 (RNE)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_from_bits(b: np.ndarray) -> np.ndarray:
    """uint16 bfloat16 bit patterns -> float32 values."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16, returned as float32."""
    return bf16_from_bits(bf16_bits(x))


# ----------------------------------------------------------------------------
# Problem descriptions
# ----------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class LactProblem:
    """One call of the chunked LaCT layer (or of its linear-attention form).

    Row-vector convention: W0, W2 are h x rh and W1 is rh x h per head.
    """
    B: int
    H: int
    h: int
    r: int
    Nq: int
    Nk: int
    chunk_q: int
    chunk_kv: int
    order: int = APPLY_THEN_UPDATE
    dtype: int = FP32
    update_mask: int = UPD_ALL
    weight_norm: bool = True
    muon: bool = False
    momentum: float = 0.0
    eps_norm: float = 1e-5
    eps_ns: float = 1e-7
    v_normalised: bool = True  # config 0/1: V L2-normalised too; configs 2/3: V ~ N(0,1)

    @property
    def rh(self) -> int:
        return self.r * self.h

    @property
    def n_chunks(self) -> int:
        return self.Nk // self.chunk_kv

    def replace(self, **kw) -> "LactProblem":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class InplaceProblem:
    """One call of the In-Place TTT down-projection update."""
    B: int
    N: int
    d_model: int
    d_hidden: int
    chunk: int
    eta: float = 1e-3
    dtype: int = BF16

    @property
    def n_chunks(self) -> int:
        return self.N // self.chunk

    def replace(self, **kw) -> "InplaceProblem":
        return dataclasses.replace(self, **kw)


# The five workloads. Index k is also the seed of its inputs.
CONFIGS = {
    0: LactProblem(B=1, H=2, h=32, r=2, Nq=256, Nk=256, chunk_q=64, chunk_kv=64,
                   order=APPLY_THEN_UPDATE, dtype=FP32, update_mask=UPD_ALL,
                   weight_norm=True, muon=False, momentum=0.0, v_normalised=True),
    1: LactProblem(B=4, H=8, h=64, r=2, Nq=8192, Nk=8192, chunk_q=512, chunk_kv=512,
                   order=APPLY_THEN_UPDATE, dtype=BF16, update_mask=UPD_W1,
                   weight_norm=False, muon=False, momentum=0.0, v_normalised=True),
    2: LactProblem(B=4, H=8, h=128, r=2, Nq=32768, Nk=32768, chunk_q=2048, chunk_kv=2048,
                   order=APPLY_THEN_UPDATE, dtype=BF16, update_mask=UPD_ALL,
                   weight_norm=True, muon=True, momentum=0.9, v_normalised=False),
    3: LactProblem(B=1, H=4, h=192, r=2, Nq=4096, Nk=196608, chunk_q=4096, chunk_kv=196608,
                   order=UPDATE_THEN_APPLY, dtype=BF16, update_mask=UPD_ALL,
                   weight_norm=True, muon=True, momentum=0.0, v_normalised=False),
    4: InplaceProblem(B=1, N=32768, d_model=4096, d_hidden=14336, chunk=1024, eta=1e-3, dtype=BF16),
}

CONFIG_NAMES = {
    0: "tiny LaCT layer fp32 (B1 H2 h32 r2 seq256 chunk64)",
    1: "last-layer-only linear-attention scan bf16 (B4 H8 h64 r2 seq8192 chunk512)",
    2: "LaCT LM layer bf16 (B4 H8 h128 r2 seq32768 chunk2048, momentum 0.9, Muon, renorm)",
    3: "LaCT NVS scene bf16 (1 scene, 4 heads h192 r2, 196608 context + 4096 query tokens, Muon)",
    4: "In-Place TTT W_down update bf16 (d_model4096 d_H14336 seq32768 chunk1024)",
}


# ----------------------------------------------------------------------------
# Generators
# ----------------------------------------------------------------------------
def _normal(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _l2_rows(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(np.square(x, dtype=np.float64), axis=-1, keepdims=True))
    return (x / n).astype(np.float32)


def _softplus(x: np.ndarray) -> np.ndarray:
    x64 = x.astype(np.float64)
    return (np.maximum(x64, 0.0) + np.log1p(np.exp(-np.abs(x64)))).astype(np.float32)


def make_lact_inputs(p: LactProblem, seed: int, *, eta_scale: float = 0.01,
                     w1_zero: bool = False) -> Dict[str, np.ndarray]:
    """Draw Q, K, V, eta, W0, W2, W1 (in that order) for problem ``p``.

    Returns float32 arrays (bf16-representable when ``p.dtype == BF16``):
      Q [B,H,Nq,h], K/V [B,H,Nk,h], eta [B,H,Nk], W0/W2 [H,h,rh], W1 [H,rh,h].
    ``eta_scale`` and ``w1_zero`` build the stress variants of the parity tests.
    """
    rng = np.random.default_rng(seed)
    B, H, h, rh = p.B, p.H, p.h, p.rh
    Q = _l2_rows(_normal(rng, (B, H, p.Nq, h)))
    K = _l2_rows(_normal(rng, (B, H, p.Nk, h)))
    V = _normal(rng, (B, H, p.Nk, h))
    if p.v_normalised:
        V = _l2_rows(V)
    eta = (np.float32(eta_scale) * _softplus(_normal(rng, (B, H, p.Nk)))).astype(np.float32)
    W0 = _normal(rng, (H, h, rh), 1.0 / math.sqrt(h))
    W2 = _normal(rng, (H, h, rh), 1.0 / math.sqrt(h))
    W1 = _normal(rng, (H, rh, h), 1.0 / math.sqrt(rh))
    if w1_zero:
        W1 = np.zeros_like(W1)
    if p.dtype == BF16:
        Q, K, V, W0, W1, W2 = (bf16_round(a) for a in (Q, K, V, W0, W1, W2))
    return dict(Q=Q, K=K, V=V, eta=eta, W0=W0, W1=W1, W2=W2)


def make_inplace_inputs(p: InplaceProblem, seed: int, *, eta: Optional[float] = None
                        ) -> Dict[str, np.ndarray]:
    """Draw H, W_gate, W_up, W_down, X0 (in that order) for problem ``p``.

    Returns float32 arrays (bf16-representable for bf16 problems):
      Hs [B,N,d_model], W_gate/W_up [d_hidden,d_model], W_down [d_model,d_hidden],
      Vbar [B,N,d_model] = next-token shift of X0 with a zero last row, X0 [B,N,d_model].
    The next-token target is the causal Conv1D with taps (0, 1) and an identity
    projection ("In-Place Test-Time Training" notes, section 3.2 / Eq. 3).
    """
    rng = np.random.default_rng(seed)
    B, N, dm, dh = p.B, p.N, p.d_model, p.d_hidden
    Hs = _normal(rng, (B, N, dm))
    Wg = _normal(rng, (dh, dm), 1.0 / math.sqrt(dm))
    Wu = _normal(rng, (dh, dm), 1.0 / math.sqrt(dm))
    Wd = _normal(rng, (dm, dh), 1.0 / math.sqrt(dh))
    X0 = _normal(rng, (B, N, dm))
    if p.dtype == BF16:
        Hs, Wg, Wu, Wd, X0 = (bf16_round(a) for a in (Hs, Wg, Wu, Wd, X0))
    Vbar = np.zeros_like(X0)
    Vbar[:, :-1] = X0[:, 1:]
    return dict(Hs=Hs, W_gate=Wg, W_up=Wu, W_down=Wd, Vbar=Vbar, X0=X0,
                eta=np.float32(p.eta if eta is None else eta))


def max_abs_rel(y: np.ndarray, ref: np.ndarray) -> float:
    """max|y - ref| / max|ref| over a whole tensor (the parity error metric)."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(y - ref))) if ref.size else 0.0
    if den == 0.0:
        return num
    return num / den
