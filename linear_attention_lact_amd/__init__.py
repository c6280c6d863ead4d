"""Python binding of the MI355X chunked TTT-KVB fast-weight library.

Argument marshalling only: every step of the computation runs in the gfx950
kernels of ``libttt_lact.so`` behind the C ABI declared in ``include/ttt_lact.h``.
PyTorch provides device memory and the stream. There is no CPU fallback: if the
shared library is missing, every entry point raises.

Entry points (same names as the C ABI, without the ``ttt_`` prefix):

* :func:`lact_forward`          -- the chunked LaCT layer
* :func:`linattn_forward`       -- the last-layer-only linear-attention scan form
* :func:`inplace_down_forward`  -- the In-Place TTT down-projection update
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libttt_lact.so")

TTT_OK, TTT_ERR_ARG, TTT_ERR_SHAPE, TTT_ERR_UNSUPPORTED, TTT_ERR_WORKSPACE, TTT_ERR_HIP = 0, -1, -2, -3, -4, -5
APPLY_THEN_UPDATE, UPDATE_THEN_APPLY = 0, 1
FP32, BF16 = 0, 1
UPD_W0, UPD_W1, UPD_W2 = 1, 2, 4

EXPORTED = ("ttt_lact_forward", "ttt_linattn_forward", "ttt_inplace_down_forward", "ttt_status_string",
            "ttt_timing_enable", "ttt_timing_collect")


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("launches", ctypes.c_int32), ("total_ms", ctypes.c_float)]


class LactParams(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("Nq", ctypes.c_int32), ("Nk", ctypes.c_int32),
                ("h", ctypes.c_int32), ("r", ctypes.c_int32), ("chunk_q", ctypes.c_int32),
                ("chunk_kv", ctypes.c_int32), ("order", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("update_mask", ctypes.c_uint32), ("weight_norm", ctypes.c_int32), ("muon", ctypes.c_int32),
                ("momentum", ctypes.c_float), ("eps_norm", ctypes.c_float), ("eps_ns", ctypes.c_float),
                ("w_batch_stride", ctypes.c_int64)]


class LinattnParams(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32), ("h", ctypes.c_int32),
                ("r", ctypes.c_int32), ("chunk", ctypes.c_int32), ("order", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("w_batch_stride", ctypes.c_int64), ("momentum", ctypes.c_float)]


class InplaceParams(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("N", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("d_hidden", ctypes.c_int32), ("chunk", ctypes.c_int32), ("eta", ctypes.c_float),
                ("dtype", ctypes.c_int32), ("wdown_batch_stride", ctypes.c_int64)]


_lib = None
_vp = ctypes.c_void_p
_szp = ctypes.POINTER(ctypes.c_size_t)


class TTTError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed with status {status} ({status_string(status)})")


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the shared library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"HIP library not built: {p} is missing (run __graft_entry__.build() "
                           "or python -m linear_attention_lact_amd.build)")
    lib = ctypes.CDLL(p)
    lib.ttt_lact_forward.argtypes = [ctypes.POINTER(LactParams)] + [_vp] * 13 + [_vp, _szp, _vp]
    lib.ttt_lact_forward.restype = ctypes.c_int32
    lib.ttt_linattn_forward.argtypes = [ctypes.POINTER(LinattnParams)] + [_vp] * 9 + [_vp, _szp, _vp]
    lib.ttt_linattn_forward.restype = ctypes.c_int32
    lib.ttt_inplace_down_forward.argtypes = [ctypes.POINTER(InplaceParams)] + [_vp] * 7 + [_vp, _szp, _vp]
    lib.ttt_inplace_down_forward.restype = ctypes.c_int32
    lib.ttt_status_string.argtypes = [ctypes.c_int32]
    lib.ttt_status_string.restype = ctypes.c_char_p
    lib.ttt_timing_enable.argtypes = [ctypes.c_int32]
    lib.ttt_timing_enable.restype = ctypes.c_int32
    lib.ttt_timing_collect.argtypes = [ctypes.POINTER(KernelTime), ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)]
    lib.ttt_timing_collect.restype = ctypes.c_int32
    _lib = lib
    return lib


def status_string(s: int) -> str:
    return load().ttt_status_string(s).decode()


def timing_enable(on: bool = True) -> None:
    """Bracket every kernel launched by the entry points with HIP events (per kernel class)."""
    st = load().ttt_timing_enable(int(bool(on)))
    if st != TTT_OK:
        raise TTTError("ttt_timing_enable", st)


def timing_collect() -> dict:
    """Wait for the recorded events; return {kernel class: (launches, total ms)} and clear."""
    lib = load()
    buf = (KernelTime * 32)()
    n = ctypes.c_int32(0)
    st = lib.ttt_timing_collect(buf, 32, ctypes.byref(n))
    if st != TTT_OK:
        raise TTTError("ttt_timing_collect", st)
    return {buf[i].name.decode(): (int(buf[i].launches), float(buf[i].total_ms)) for i in range(min(n.value, 32))}


# ----------------------------------------------------------------------------------------
# torch helpers (device memory and streams only)
# ----------------------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check(t, name, dtype, device):
    if t is None:
        return
    torch = _torch()
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    del torch


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _call(fn_name, fn, args, query_args, device, stream):
    """Query the workspace size, allocate it with torch, then launch."""
    torch = _torch()
    size = ctypes.c_size_t(0)
    st = fn(*query_args, None, ctypes.byref(size), _stream(stream))
    if st != TTT_OK:
        raise TTTError(fn_name, st)
    ws = torch.empty(max(int(size.value), 256), dtype=torch.uint8, device=device)
    if stream is not None:
        ws.record_stream(stream)
    size = ctypes.c_size_t(ws.numel())
    st = fn(*args, ctypes.c_void_p(ws.data_ptr()), ctypes.byref(size), _stream(stream))
    if st != TTT_OK:
        raise TTTError(fn_name, st)
    return ws


def _io_dtype(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return FP32
    raise ValueError(f"token tensors must be bfloat16 or float32, got {t.dtype}")


def lact_forward(Q, K, V, eta, W0, W1, W2, *, chunk_q: int, chunk_kv: Optional[int] = None,
                 order: int = APPLY_THEN_UPDATE, update_mask: int = 7, weight_norm: bool = True,
                 muon: bool = False, momentum: float = 0.0, eps_norm: float = 1e-5, eps_ns: float = 1e-7,
                 M_in=None, want_state: bool = True, stream=None):
    """Chunked LaCT layer. Q [B,H,Nq,h], K/V [B,H,Nk,h] (bf16 or fp32), eta [B,H,Nk] fp32,
    W0/W2 [H,h,rh] and W1 [H,rh,h] fp32 (or [B,H,...] per sequence), M_in [B,H,3,h*rh] or None.
    Returns (O, W0_out, W1_out, W2_out, M_out); the last four are None if not want_state."""
    torch = _torch()
    lib = load()
    chunk_kv = chunk_q if chunk_kv is None else chunk_kv
    B, H, Nq, h = Q.shape
    Nk = K.shape[2]
    per_seq = W0.dim() == 4
    rh = W0.shape[-1]
    dev = Q.device
    io = Q.dtype
    for t, n in ((Q, "Q"), (K, "K"), (V, "V")):
        _check(t, n, io, dev)
    _check(eta, "eta", torch.float32, dev)
    for t, n in ((W0, "W0"), (W1, "W1"), (W2, "W2"), (M_in, "M_in")):
        _check(t, n, torch.float32, dev)
    if K.shape != (B, H, Nk, h) or V.shape != K.shape or eta.shape != (B, H, Nk):
        raise ValueError("K/V must be [B,H,Nk,h] and eta [B,H,Nk]")
    wshape = ((B,) if per_seq else ()) + (H,)
    if W0.shape != wshape + (h, rh) or W2.shape != W0.shape or W1.shape != wshape + (rh, h):
        raise ValueError("W0/W2 must be [(B,)H,h,rh] and W1 [(B,)H,rh,h]")
    if rh % h:
        raise ValueError("rh must be a multiple of h")
    p = LactParams(B, H, Nq, Nk, h, rh // h, chunk_q, chunk_kv, order, _io_dtype(Q), update_mask,
                   int(bool(weight_norm)), int(bool(muon)), momentum, eps_norm, eps_ns,
                   H * h * rh if per_seq else 0)
    O = torch.empty_like(Q)
    outs = [None] * 4
    if want_state:
        outs = [torch.empty((B, H, h, rh), dtype=torch.float32, device=dev),
                torch.empty((B, H, rh, h), dtype=torch.float32, device=dev),
                torch.empty((B, H, h, rh), dtype=torch.float32, device=dev),
                torch.empty((B, H, 3, h * rh), dtype=torch.float32, device=dev)]
    base = [ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(eta), _ptr(W0), _ptr(W1), _ptr(W2), _ptr(M_in),
            _ptr(O)] + [_ptr(t) for t in outs]
    _call("ttt_lact_forward", lib.ttt_lact_forward, base, base, dev, stream)
    return (O, *outs)


def linattn_forward(Q, K, V, eta, W0, W2, W1, *, chunk: int, order: int = APPLY_THEN_UPDATE,
                    momentum: float = 0.0, want_state: bool = True, stream=None):
    """Last-layer-only linear-attention scan. Q/K/V [B,H,N,h], eta [B,H,N], W0/W2 [(B,)H,h,rh],
    W1 [(B,)H,rh,h]; momentum: heavy-ball coefficient per chunk (0 <= momentum < 1).
    Returns (O, S_out) with S_out [B,H,rh,h] (None if not want_state)."""
    torch = _torch()
    lib = load()
    B, H, N, h = Q.shape
    per_seq = W0.dim() == 4
    rh = W0.shape[-1]
    dev = Q.device
    for t, n in ((Q, "Q"), (K, "K"), (V, "V")):
        _check(t, n, Q.dtype, dev)
    _check(eta, "eta", torch.float32, dev)
    for t, n in ((W0, "W0"), (W1, "W1"), (W2, "W2")):
        _check(t, n, torch.float32, dev)
    if K.shape != Q.shape or V.shape != Q.shape or eta.shape != (B, H, N):
        raise ValueError("Q/K/V must share [B,H,N,h] and eta be [B,H,N]")
    if rh % h:
        raise ValueError("rh must be a multiple of h")
    p = LinattnParams(B, H, N, h, rh // h, chunk, order, _io_dtype(Q), H * h * rh if per_seq else 0,
                      float(momentum))
    O = torch.empty_like(Q)
    S = torch.empty((B, H, rh, h), dtype=torch.float32, device=dev) if want_state else None
    base = [ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(eta), _ptr(W0), _ptr(W2), _ptr(W1), _ptr(O), _ptr(S)]
    _call("ttt_linattn_forward", lib.ttt_linattn_forward, base, base, dev, stream)
    return O, S


def inplace_down_forward(Hs, W_gate, W_up, W_down, Vbar, *, chunk: int, eta: float,
                         want_state: bool = True, stream=None):
    """In-Place TTT down-projection update. Hs/Vbar [B,N,d_model] bf16, W_gate/W_up
    [d_hidden,d_model] bf16, W_down [(B,)d_model,d_hidden] fp32. Returns (O, W_down_out)."""
    torch = _torch()
    lib = load()
    B, N, dm = Hs.shape
    dh = W_gate.shape[0]
    dev = Hs.device
    for t, n in ((Hs, "Hs"), (W_gate, "W_gate"), (W_up, "W_up"), (Vbar, "Vbar")):
        _check(t, n, torch.bfloat16, dev)
    _check(W_down, "W_down", torch.float32, dev)
    per_seq = W_down.dim() == 3
    if W_gate.shape != (dh, dm) or W_up.shape != (dh, dm) or Vbar.shape != Hs.shape:
        raise ValueError("shape mismatch")
    if W_down.shape[-2:] != (dm, dh):
        raise ValueError("W_down must be [(B,)d_model,d_hidden]")
    p = InplaceParams(B, N, dm, dh, chunk, eta, BF16, dm * dh if per_seq else 0)
    O = torch.empty_like(Hs)
    Wout = torch.empty((B, dm, dh), dtype=torch.float32, device=dev) if want_state else None
    base = [ctypes.byref(p), _ptr(Hs), _ptr(W_gate), _ptr(W_up), _ptr(W_down), _ptr(Vbar), _ptr(O), _ptr(Wout)]
    _call("ttt_inplace_down_forward", lib.ttt_inplace_down_forward, base, base, dev, stream)
    return O, Wout
