"""Python binding of the MI355X chunked TTT-KVB fast-weight library.

Argument marshalling only: every step of the computation runs in the gfx950
kernels of ``libttt_lact.so`` behind the C ABI declared in ``include/ttt_lact.h``.
PyTorch provides device memory and the stream. There is no CPU fallback: if the
shared library is missing, every entry point raises.

Entry points (same names as the C ABI, without the ``ttt_`` prefix):

* :func:`lact_forward`          -- the chunked LaCT layer
* :func:`linattn_forward`       -- the last-layer-only linear-attention scan form
* :func:`inplace_down_forward`  -- the In-Place TTT down-projection update
* :func:`linattn_backward`, :func:`inplace_down_backward` -- their gradients
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libttt_lact.so")

TTT_OK, TTT_ERR_ARG, TTT_ERR_SHAPE, TTT_ERR_UNSUPPORTED, TTT_ERR_WORKSPACE, TTT_ERR_HIP = 0, -1, -2, -3, -4, -5
APPLY_THEN_UPDATE, UPDATE_THEN_APPLY = 0, 1
CHUNK_NO_UPDATE, CHUNK_RESET = 1, 2  # per-chunk flags of lact_forward
FEATURE_MAPS = {"swiglu": 0, "identity": 1}  # ttt_feature_map
FP32, BF16 = 0, 1
UPD_W0, UPD_W1, UPD_W2 = 1, 2, 4

EXPORTED = ("ttt_lact_forward", "ttt_linattn_forward", "ttt_linattn_forward_noalloc", "ttt_linattn_backward",
            "ttt_inplace_down_forward", "ttt_inplace_down_backward", "ttt_inplace_target_forward",
            "ttt_inplace_target_backward",
            "ttt_status_string", "ttt_last_error", "ttt_timing_enable", "ttt_timing_collect")
NOALLOC_SCRATCH_BYTES = 64 << 20  # TTT_NOALLOC_SCRATCH_BYTES


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("launches", ctypes.c_int32), ("total_ms", ctypes.c_float)]


class LactParams(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("Nq", ctypes.c_int32), ("Nk", ctypes.c_int32),
                ("h", ctypes.c_int32), ("r", ctypes.c_int32), ("chunk_q", ctypes.c_int32),
                ("chunk_kv", ctypes.c_int32), ("order", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("update_mask", ctypes.c_uint32), ("weight_norm", ctypes.c_int32), ("muon", ctypes.c_int32),
                ("momentum", ctypes.c_float), ("eps_norm", ctypes.c_float), ("eps_ns", ctypes.c_float),
                ("w_batch_stride", ctypes.c_int64), ("chunk_flags", ctypes.c_void_p),
                ("inner_steps", ctypes.c_int32), ("eta_per_matrix", ctypes.c_int32)]


class LinattnParams(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32), ("h", ctypes.c_int32),
                ("r", ctypes.c_int32), ("chunk", ctypes.c_int32), ("order", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("w_batch_stride", ctypes.c_int64), ("momentum", ctypes.c_float),
                ("feature_map", ctypes.c_int32), ("chunk_flags", ctypes.c_void_p)]


class InplaceParams(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("N", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("d_hidden", ctypes.c_int32), ("chunk", ctypes.c_int32), ("eta", ctypes.c_float),
                ("dtype", ctypes.c_int32), ("wdown_batch_stride", ctypes.c_int64),
                ("X0", ctypes.c_void_p), ("conv_taps", ctypes.c_void_p), ("W_target", ctypes.c_void_p),
                ("conv_k", ctypes.c_int32)]


_lib = None
_vp = ctypes.c_void_p
_szp = ctypes.POINTER(ctypes.c_size_t)


class TTTError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        detail = f": {last_error()}" if status in (TTT_ERR_HIP, TTT_ERR_WORKSPACE) and last_error() else ""
        super().__init__(f"{fn} failed with status {status} ({status_string(status)}){detail}")


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the shared library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"HIP library not built: {p} is missing (run __graft_entry__.build() "
                           "or python -m linear_attention_lact_amd.build)")
    # torch first: the library and torch's ROCm build both name their HIP runtime
    # libamdhip64.so.7, and the first one loaded serves the whole process. Loading torch's
    # first keeps one runtime, the one that owns the device memory and streams we are given.
    import torch  # noqa: F401
    lib = ctypes.CDLL(p)
    lib.ttt_lact_forward.argtypes = [ctypes.POINTER(LactParams)] + [_vp] * 13 + [_vp, _szp, _vp]
    lib.ttt_lact_forward.restype = ctypes.c_int32
    lib.ttt_linattn_forward.argtypes = [ctypes.POINTER(LinattnParams)] + [_vp] * 9 + [_vp, _szp, _vp]
    lib.ttt_linattn_forward.restype = ctypes.c_int32
    lib.ttt_linattn_forward_noalloc.argtypes = [ctypes.POINTER(LinattnParams)] + [_vp] * 9 + [_vp]
    lib.ttt_linattn_forward_noalloc.restype = ctypes.c_int32
    lib.ttt_linattn_backward.argtypes = [ctypes.POINTER(LinattnParams)] + [_vp] * 15 + [_vp, _szp, _vp]
    lib.ttt_linattn_backward.restype = ctypes.c_int32
    lib.ttt_inplace_down_forward.argtypes = [ctypes.POINTER(InplaceParams)] + [_vp] * 7 + [_vp, _szp, _vp]
    lib.ttt_inplace_down_forward.restype = ctypes.c_int32
    lib.ttt_inplace_down_backward.argtypes = [ctypes.POINTER(InplaceParams)] + [_vp] * 11 + [_vp, _szp, _vp]
    lib.ttt_inplace_down_backward.restype = ctypes.c_int32
    lib.ttt_inplace_target_forward.argtypes = [ctypes.POINTER(InplaceParams), _vp, _vp, _szp, _vp]
    lib.ttt_inplace_target_forward.restype = ctypes.c_int32
    lib.ttt_inplace_target_backward.argtypes = [ctypes.POINTER(InplaceParams)] + [_vp] * 4 + [_vp, _szp, _vp]
    lib.ttt_inplace_target_backward.restype = ctypes.c_int32
    lib.ttt_status_string.argtypes = [ctypes.c_int32]
    lib.ttt_status_string.restype = ctypes.c_char_p
    lib.ttt_last_error.argtypes = []
    lib.ttt_last_error.restype = ctypes.c_char_p
    lib.ttt_timing_enable.argtypes = [ctypes.c_int32]
    lib.ttt_timing_enable.restype = ctypes.c_int32
    lib.ttt_timing_collect.argtypes = [ctypes.POINTER(KernelTime), ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)]
    lib.ttt_timing_collect.restype = ctypes.c_int32
    _lib = lib
    return lib


def status_string(s: int) -> str:
    return load().ttt_status_string(s).decode()


def last_error() -> str:
    """The last HIP failure the library met on this thread (empty if none)."""
    return load().ttt_last_error().decode()


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


def _check_weights(W0, W1, W2, B, H, h):
    """W0/W2 [H,h,rh] and W1 [H,rh,h] shared by the batch, or all three [B,H,...] per
    sequence; rh a multiple of h. Checked before any launch: a wrong shape would make the
    kernels read past the end of a buffer."""
    per_seq = W0.dim() == 4
    lead = (B, H) if per_seq else (H,)
    rh = W0.shape[-1]
    if tuple(W0.shape) != lead + (h, rh) or tuple(W2.shape) != lead + (h, rh) or tuple(W1.shape) != lead + (rh, h):
        raise ValueError(f"W0/W2 must be {'[B,H,h,rh]' if per_seq else '[H,h,rh]'} and W1 "
                         f"{'[B,H,rh,h]' if per_seq else '[H,rh,h]'} with h={h}, all shared or all per sequence; "
                         f"got {tuple(W0.shape)}, {tuple(W1.shape)}, {tuple(W2.shape)}")
    if rh % h:
        raise ValueError("rh must be a multiple of h")


def lact_forward(Q, K, V, eta, W0, W1, W2, *, chunk_q: int, chunk_kv: Optional[int] = None,
                 order: int = APPLY_THEN_UPDATE, update_mask: int = 7, weight_norm: bool = True,
                 muon: bool = False, momentum: float = 0.0, eps_norm: float = 1e-5, eps_ns: float = 1e-7,
                 M_in=None, chunk_flags=None, inner_steps: int = 1, want_state: bool = True, stream=None):
    """Chunked LaCT layer. Q [B,H,Nq,h], K/V [B,H,Nk,h] (bf16 or fp32), eta [B,H,Nk] fp32
    (or [B,H,3,Nk]: one row per matrix W0, W1, W2), W0/W2 [H,h,rh] and W1 [H,rh,h] fp32 (or
    [B,H,...] per sequence), M_in [B,H,3,h*rh] or None. chunk_flags: None or a uint8 device
    tensor [B, Nk/chunk_kv] of CHUNK_NO_UPDATE / CHUNK_RESET bits; inner_steps: writes per chunk.
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
    eta3 = eta.dim() == 4
    if K.shape != (B, H, Nk, h) or V.shape != K.shape or tuple(eta.shape) != ((B, H, 3, Nk) if eta3 else (B, H, Nk)):
        raise ValueError("K/V must be [B,H,Nk,h] and eta [B,H,Nk] (or [B,H,3,Nk], one row per matrix)")
    if chunk_flags is not None:
        _check(chunk_flags, "chunk_flags", torch.uint8, dev)
        if chunk_kv <= 0 or tuple(chunk_flags.shape) != (B, Nk // chunk_kv):
            raise ValueError("chunk_flags must be uint8 [B, Nk/chunk_kv]")
    if not (1 <= inner_steps <= 64):
        raise ValueError("inner_steps must lie in [1, 64]")
    _check_weights(W0, W1, W2, B, H, h)
    if M_in is not None and tuple(M_in.shape) != (B, H, 3, h * rh):
        raise ValueError("M_in must be [B,H,3,h*rh]")
    if not (0.0 <= momentum < 1.0):
        raise ValueError("momentum must lie in [0, 1)")
    p = LactParams(B, H, Nq, Nk, h, rh // h, chunk_q, chunk_kv, order, _io_dtype(Q), update_mask,
                   int(bool(weight_norm)), int(bool(muon)), momentum, eps_norm, eps_ns,
                   H * h * rh if per_seq else 0, _ptr(chunk_flags), int(inner_steps), int(eta3))
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
                    momentum: float = 0.0, feature_map: str = "swiglu", chunk_flags=None, want_state: bool = True,
                    stream=None):
    """Last-layer-only linear-attention scan. Q/K/V [B,H,N,h], eta [B,H,N], W0/W2 [(B,)H,h,rh],
    W1 [(B,)H,rh,h]; momentum: heavy-ball coefficient per chunk (0 <= momentum < 1).
    feature_map "identity": phi(x) = x (one linear fast-weight layer), W0/W2 None, W1 [(B,)H,h,h].
    chunk_flags: None or a uint8 device tensor [B, N/chunk] of CHUNK_NO_UPDATE / CHUNK_RESET bits.
    Returns (O, S_out) with S_out [B,H,rh,h] (None if not want_state)."""
    return _linattn(Q, K, V, eta, W0, W2, W1, chunk, order, momentum, feature_map, want_state, stream,
                    noalloc=False, chunk_flags=chunk_flags)


def linattn_forward_noalloc(Q, K, V, eta, W0, W2, W1, *, chunk: int, order: int = APPLY_THEN_UPDATE,
                            momentum: float = 0.0, feature_map: str = "swiglu", want_state: bool = True,
                            stream=None):
    """linattn_forward without a workspace: the library's per-device scratch array
    (NOALLOC_SCRATCH_BYTES) serves as the workspace, so the call allocates no device memory
    besides the outputs it returns. Calls on one GPU share the array: do not overlap them."""
    return _linattn(Q, K, V, eta, W0, W2, W1, chunk, order, momentum, feature_map, want_state, stream,
                    noalloc=True)


def _linattn(Q, K, V, eta, W0, W2, W1, chunk, order, momentum, feature_map, want_state, stream, noalloc,
             chunk_flags=None):
    torch = _torch()
    lib = load()
    B, H, N, h = Q.shape
    if feature_map not in FEATURE_MAPS:
        raise ValueError(f"feature_map must be one of {sorted(FEATURE_MAPS)}")
    ident = feature_map == "identity"
    per_seq = W1.dim() == 4
    rh = W1.shape[-2]
    dev = Q.device
    for t, n in ((Q, "Q"), (K, "K"), (V, "V")):
        _check(t, n, Q.dtype, dev)
    _check(eta, "eta", torch.float32, dev)
    if K.shape != Q.shape or V.shape != Q.shape or eta.shape != (B, H, N):
        raise ValueError("Q/K/V must share [B,H,N,h] and eta be [B,H,N]")
    if ident:
        _check(W1, "W1", torch.float32, dev)
        if W0 is not None or W2 is not None:
            raise ValueError("the identity feature map takes no W0/W2")
        if tuple(W1.shape) != ((B, H) if per_seq else (H,)) + (h, h):
            raise ValueError(f"W1 must be [(B,)H,h,h] with h={h} for the identity feature map; got {tuple(W1.shape)}")
    else:
        for t, n in ((W0, "W0"), (W1, "W1"), (W2, "W2")):
            _check(t, n, torch.float32, dev)
        _check_weights(W0, W1, W2, B, H, h)
    if not (0.0 <= momentum < 1.0):
        raise ValueError("momentum must lie in [0, 1)")
    if chunk_flags is not None:
        _check(chunk_flags, "chunk_flags", torch.uint8, dev)
        if chunk <= 0 or tuple(chunk_flags.shape) != (B, N // chunk):
            raise ValueError("chunk_flags must be uint8 [B, N/chunk]")
    p = LinattnParams(B, H, N, h, rh // h, chunk, order, _io_dtype(Q), H * h * rh if per_seq else 0,
                      float(momentum), FEATURE_MAPS[feature_map], _ptr(chunk_flags))
    O = torch.empty_like(Q)
    S = torch.empty((B, H, rh, h), dtype=torch.float32, device=dev) if want_state else None
    base = [ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(eta), _ptr(W0), _ptr(W2), _ptr(W1), _ptr(O), _ptr(S)]
    if noalloc:
        st = lib.ttt_linattn_forward_noalloc(*base, _stream(stream))
        if st != TTT_OK:
            raise TTTError("ttt_linattn_forward_noalloc", st)
    else:
        _call("ttt_linattn_forward", lib.ttt_linattn_forward, base, base, dev, stream)
    return O, S


def linattn_backward(Q, K, V, eta, W0, W2, W1, dO, *, chunk: int, order: int = APPLY_THEN_UPDATE,
                     momentum: float = 0.0, stream=None):
    """Gradients of sum(O * dO) of linattn_forward (SwiGLU map). Returns dict(dQ, dK, dV, deta,
    dW0, dW2, dW1); the weight gradients have the weights' shape (summed over the batch when the
    weights are shared)."""
    torch = _torch()
    lib = load()
    B, H, N, h = Q.shape
    dev = Q.device
    for t, n in ((Q, "Q"), (K, "K"), (V, "V"), (dO, "dO")):
        _check(t, n, Q.dtype, dev)
    _check(eta, "eta", torch.float32, dev)
    for t, n in ((W0, "W0"), (W1, "W1"), (W2, "W2")):
        _check(t, n, torch.float32, dev)
    if K.shape != Q.shape or V.shape != Q.shape or dO.shape != Q.shape or eta.shape != (B, H, N):
        raise ValueError("Q/K/V/dO must share [B,H,N,h] and eta be [B,H,N]")
    _check_weights(W0, W1, W2, B, H, h)
    if not (0.0 <= momentum < 1.0):
        raise ValueError("momentum must lie in [0, 1)")
    per_seq = W0.dim() == 4
    rh = W0.shape[-1]
    p = LinattnParams(B, H, N, h, rh // h, chunk, order, _io_dtype(Q), H * h * rh if per_seq else 0,
                      float(momentum), 0)
    out = dict(dQ=torch.empty_like(Q), dK=torch.empty_like(K), dV=torch.empty_like(V),
               deta=torch.empty_like(eta), dW0=torch.empty_like(W0), dW2=torch.empty_like(W2),
               dW1=torch.empty_like(W1))
    base = [ctypes.byref(p)] + [_ptr(t) for t in (Q, K, V, eta, W0, W2, W1, dO)] + \
        [_ptr(out[k]) for k in ("dQ", "dK", "dV", "deta", "dW0", "dW2", "dW1")]
    _call("ttt_linattn_backward", lib.ttt_linattn_backward, base, base, dev, stream)
    return out


def inplace_down_forward(Hs, W_gate, W_up, W_down, Vbar, *, chunk: int, eta: float,
                         X0=None, conv_taps=None, W_target=None, want_state: bool = True, stream=None):
    """In-Place TTT down-projection update. Hs/Vbar [B,N,d_model] bf16, W_gate/W_up
    [d_hidden,d_model] bf16, W_down [(B,)d_model,d_hidden] fp32. Returns (O, W_down_out).
    LM-aligned target: pass Vbar=None with X0 [B,N,d_model] bf16, conv_taps [k,d_model] fp32
    (tap tau weights the token tau positions ahead) and optionally W_target [d_model,d_model] bf16
    (nn.Linear layout); the library then builds Vbar = Conv1D(X0) W_target^T."""
    torch = _torch()
    lib = load()
    B, N, dm = Hs.shape
    dh = W_gate.shape[0]
    dev = Hs.device
    for t, n in ((Hs, "Hs"), (W_gate, "W_gate"), (W_up, "W_up"), (Vbar, "Vbar"), (X0, "X0"),
                 (W_target, "W_target")):
        _check(t, n, torch.bfloat16, dev)
    _check(conv_taps, "conv_taps", torch.float32, dev)
    _check(W_down, "W_down", torch.float32, dev)
    per_seq = W_down.dim() == 3
    if W_gate.shape != (dh, dm) or W_up.shape != (dh, dm):
        raise ValueError("shape mismatch")
    if (Vbar is None) == (X0 is None):
        raise ValueError("give either Vbar or X0 (with conv_taps) for the target")
    if Vbar is not None and Vbar.shape != Hs.shape:
        raise ValueError("Vbar must be [B,N,d_model]")
    if X0 is not None:
        if X0.shape != Hs.shape or conv_taps is None or conv_taps.dim() != 2 or conv_taps.shape[1] != dm \
                or not (1 <= conv_taps.shape[0] <= 16):
            raise ValueError("X0 must be [B,N,d_model] and conv_taps [k,d_model] with 1 <= k <= 16")
        if W_target is not None and tuple(W_target.shape) != (dm, dm):
            raise ValueError("W_target must be [d_model,d_model]")
    if W_down.shape[-2:] != (dm, dh):
        raise ValueError("W_down must be [(B,)d_model,d_hidden]")
    p = InplaceParams(B, N, dm, dh, chunk, eta, BF16, dm * dh if per_seq else 0, _ptr(X0), _ptr(conv_taps),
                      _ptr(W_target), 0 if conv_taps is None else conv_taps.shape[0])
    O = torch.empty_like(Hs)
    Wout = torch.empty((B, dm, dh), dtype=torch.float32, device=dev) if want_state else None
    base = [ctypes.byref(p), _ptr(Hs), _ptr(W_gate), _ptr(W_up), _ptr(W_down), _ptr(Vbar), _ptr(O), _ptr(Wout)]
    _call("ttt_inplace_down_forward", lib.ttt_inplace_down_forward, base, base, dev, stream)
    return O, Wout


def inplace_down_backward(Hs, W_gate, W_up, W_down, Vbar, dO, *, chunk: int, eta: float, stream=None):
    """Gradients of sum(O * dO) of inplace_down_forward (explicit Vbar, bf16). Returns dict(dHs,
    dW_gate, dW_up, dW_down, dVbar): dHs/dVbar bf16 [B,N,d_model]; dW_gate/dW_up fp32
    [d_hidden,d_model] summed over the batch; dW_down fp32 with W_down's shape (summed over the
    batch when W_down is shared)."""
    torch = _torch()
    lib = load()
    B, N, dm = Hs.shape
    dh = W_gate.shape[0]
    dev = Hs.device
    for t, n in ((Hs, "Hs"), (W_gate, "W_gate"), (W_up, "W_up"), (Vbar, "Vbar"), (dO, "dO")):
        _check(t, n, torch.bfloat16, dev)
    _check(W_down, "W_down", torch.float32, dev)
    if Vbar is None or dO is None:
        raise ValueError("Vbar and dO are required")
    if W_gate.shape != (dh, dm) or W_up.shape != (dh, dm):
        raise ValueError("shape mismatch")
    if Vbar.shape != Hs.shape or dO.shape != Hs.shape:
        raise ValueError("Vbar and dO must be [B,N,d_model]")
    if W_down.shape[-2:] != (dm, dh) or W_down.dim() not in (2, 3) or (W_down.dim() == 3 and W_down.shape[0] != B):
        raise ValueError("W_down must be [(B,)d_model,d_hidden]")
    per_seq = W_down.dim() == 3
    p = InplaceParams(B, N, dm, dh, chunk, eta, BF16, dm * dh if per_seq else 0, None, None, None, 0)
    out = dict(dHs=torch.empty_like(Hs), dW_gate=torch.empty((dh, dm), dtype=torch.float32, device=dev),
               dW_up=torch.empty((dh, dm), dtype=torch.float32, device=dev), dW_down=torch.empty_like(W_down),
               dVbar=torch.empty_like(Vbar))
    base = [ctypes.byref(p)] + [_ptr(t) for t in (Hs, W_gate, W_up, W_down, Vbar, dO)] + \
        [_ptr(out[k]) for k in ("dHs", "dW_gate", "dW_up", "dW_down", "dVbar")]
    _call("ttt_inplace_down_backward", lib.ttt_inplace_down_backward, base, base, dev, stream)
    return out


def _target_params(X0, conv_taps, W_target):
    torch = _torch()
    B, N, dm = X0.shape
    dev = X0.device
    _check(X0, "X0", torch.bfloat16, dev)
    _check(W_target, "W_target", torch.bfloat16, dev)
    _check(conv_taps, "conv_taps", torch.float32, dev)
    if conv_taps is None or conv_taps.dim() != 2 or conv_taps.shape[1] != dm or not (1 <= conv_taps.shape[0] <= 16):
        raise ValueError("conv_taps must be [k,d_model] with 1 <= k <= 16")
    if W_target is not None and tuple(W_target.shape) != (dm, dm):
        raise ValueError("W_target must be [d_model,d_model]")
    return InplaceParams(B, N, dm, 0, 1, 0.0, BF16, 0, _ptr(X0), _ptr(conv_taps), _ptr(W_target),
                         conv_taps.shape[0]), dev


def inplace_target_forward(X0, conv_taps, W_target=None, stream=None):
    """The LM-aligned target Vbar = Conv1D(X0) W_target^T, token-major [B,N,d_model] bf16."""
    torch = _torch()
    lib = load()
    p, dev = _target_params(X0, conv_taps, W_target)
    Vbar = torch.empty_like(X0)
    base = [ctypes.byref(p), _ptr(Vbar)]
    _call("ttt_inplace_target_forward", lib.ttt_inplace_target_forward, base, base, dev, stream)
    return Vbar


def inplace_target_backward(X0, conv_taps, dVbar, W_target=None, stream=None):
    """Gradients of sum(Vbar * dVbar) of inplace_target_forward: dict(dX0 [B,N,d_model] bf16,
    dtaps [k,d_model] fp32, dW_target [d_model,d_model] fp32 or None), summed over the batch."""
    torch = _torch()
    lib = load()
    p, dev = _target_params(X0, conv_taps, W_target)
    _check(dVbar, "dVbar", torch.bfloat16, dev)
    if dVbar is None or dVbar.shape != X0.shape:
        raise ValueError("dVbar must be [B,N,d_model]")
    out = dict(dX0=torch.empty_like(X0), dtaps=torch.empty_like(conv_taps),
               dW_target=None if W_target is None else torch.empty((X0.shape[2],) * 2, dtype=torch.float32,
                                                                    device=dev))
    base = [ctypes.byref(p), _ptr(dVbar), _ptr(out["dX0"]), _ptr(out["dtaps"]), _ptr(out["dW_target"])]
    _call("ttt_inplace_target_backward", lib.ttt_inplace_target_backward, base, base, dev, stream)
    return out
