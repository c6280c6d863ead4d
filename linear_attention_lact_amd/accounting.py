"""Algorithmic FLOP and byte counts of the three forms (host-side bookkeeping for the
benchmark's roofline figures).

FLOPs count multiply-adds of the matrix products only (2 per MAC), as the LaCT paper's
FLOP model does ("Test-Time Training Done Right" notes, section 2.5: update + apply over n
tokens is 9 matmuls = 18 n r d^2 / n_h = 6 n S with state S = 3 r d^2 / n_h per layer).
Newton-Schulz products are counted on top because the method computes them; elementwise
work (silu, norms, scans) is not counted.
"""
from __future__ import annotations


def state_elements(d: int, n_h: int, r: float) -> float:
    """Fast-weight elements per layer: three matrices of h x rh per head, S = 3 r d^2 / n_h."""
    return 3.0 * r * d * d / n_h


def swiglu_matmul_flops(tokens: int, d: int, n_h: int, r: float) -> float:
    """Update + apply over `tokens` tokens: 9 products of 2 * tokens * h * rh each per head."""
    h = d // n_h
    return 9 * 2.0 * tokens * h * (r * h) * n_h


def ns5_flops(m: int, n: int, steps: int = 5) -> float:
    """Newton-Schulz on an m x n matrix (m <= n): per step X X^T (2 m^2 n), A A (2 m^3),
    B X (2 m^2 n)."""
    m, n = min(m, n), max(m, n)
    return steps * (4.0 * m * m * n + 2.0 * m ** 3)


def lact_flops(B, H, Nq, Nk, h, r, chunk_q, chunk_kv, update_mask=7, muon=False) -> float:
    rh = r * h
    n_ch = Nk // chunk_kv
    pairs = B * H
    apply = 3 * 2.0 * Nq * h * rh
    n_upd = bin(update_mask & 7).count("1")
    if update_mask == 7:
        grads = 6 * 2.0 * Nk * h * rh          # A, Bm, D and the three token contractions
    elif update_mask == 2:
        grads = 3 * 2.0 * Nk * h * rh          # A, Bm and H^T V
    else:
        grads = 6 * 2.0 * Nk * h * rh
    ns = n_ch * n_upd * ns5_flops(h, rh) if muon else 0.0
    return pairs * (apply + grads + ns)


def lact_bytes(B, H, Nq, Nk, h, r, io_bytes=2) -> float:
    """Compulsory HBM traffic: Q, K, V, O once, eta once, initial and final fp32 state."""
    pairs = B * H
    rh = r * h
    return pairs * ((2 * Nq + 2 * Nk) * h * io_bytes + 4 * Nk + 2 * 3 * h * rh * 4)


def linattn_flops(B, H, N, h, r) -> float:
    """phi(K) (2 products), dS (1), phi(Q) (2), phi(Q) S (1): 6 products of 2 N h rh."""
    return B * H * 6 * 2.0 * N * h * (r * h)


def linattn_bytes(B, H, N, h, r, io_bytes=2) -> float:
    """Q, K, V read and O written once, eta once, W0/W1/W2 read once per head (fp32) and the
    final state written (fp32)."""
    rh = r * h
    return B * H * (4 * N * h * io_bytes + 4 * N + 4 * h * rh * 4)


def linattn_backward_flops(B, H, N, h, r) -> float:
    """Backward of the scan form: phi(Q), phi(K) (4 products), dS (1), G = phi(Q)^T dO (1),
    dphi(Q) = dO S^T (1), dphi(K) and d(eta V) (2), and through each feature map dX (2) and the
    weight gradients (2), i.e. 17 products of 2 N h rh (the GPU recomputes phi(Q) and phi(K)
    once more: 21)."""
    return B * H * 17 * 2.0 * N * h * (r * h)


def linattn_identity_flops(B, H, N, h) -> float:
    """Identity feature map (h x h state): dS = K^T diag(eta) V and O = Q S, 2 products of 2 N h h."""
    return B * H * 2 * 2.0 * N * h * h


def linattn_identity_bytes(B, H, N, h, io_bytes=2) -> float:
    """Q, K, V read and O written once, eta once, the initial state read and the final state
    written (fp32)."""
    return B * H * (4 * N * h * io_bytes + 4 * N + 2 * h * h * 4)


def inplace_flops(B, N, d_model, d_hidden) -> float:
    """Z (2 products), apply (1), update (1): 4 products of 2 N d_model d_hidden."""
    return B * 4 * 2.0 * N * d_model * d_hidden


def inplace_backward_flops(B, N, d_model, d_hidden) -> float:
    """The products the gradients need, each 2 N d_model d_hidden: the forward's Z (2) and the
    chunk states (1) recomputed, dZ (2: through the chunk's own output and through the later
    chunks' reads of its write), dVbar (1), the summed output gradient G (1), dHs (2) and the two
    frozen projections' gradients (2): 11 per chunk. The last chunk needs three fewer (no later
    chunk reads its state or its write); the count keeps them (under 1 % at 32 chunks)."""
    return B * 11 * 2.0 * N * d_model * d_hidden


PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 / fp16 MFMA (AMD public figure)
PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def kernel_source_hash(root: str) -> str:
    """sha1 over the kernel sources and the C header (identifies the build a profile was taken on)."""
    import glob
    import hashlib
    import os
    h = hashlib.sha1()
    files = sorted(glob.glob(os.path.join(root, "linear_attention_lact_amd", "csrc", "*")))
    files.append(os.path.join(root, "include", "ttt_lact.h"))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


KERNEL_SYMBOLS = {"lact_update": ("lact_update_kernel",), "lact_grad": ("grad_ws_kernel", "grad_rd_kernel", "grad_kernel"),
                  "lact_apply": ("apply_rd_kernel",), "linattn_delta": ("grad_rd_kernel",),
                  "linattn_apply": ("apply_rd_kernel", "linattn_bwd_tok_kernel"), "linattn_scan": ("linattn_scan_kernel",),
                  "lact_update_apply": ("lact_update_apply_kernel",), "linattn_fused": ("linattn_fused_kernel",),
                  "inplace_apply_z": ("gemm_big_pair_kernel",), "inplace_update": ("gemm_rmw_pp_kernel",),
                  "inplace_swiglu_bwd": ("gemm_big_kernelILi4E",), "inplace_wgrad": ("gemm_rmw_pp_kernel",)}


def profiled_avg_us(root: str, kernel_class: str, stem: str):
    """Average duration (us) of a kernel class's dispatches in the committed rocprofv3 kernel
    statistics profiles/<stem>_kernel_stats.txt (the call-weighted mean over the matching
    kernels), or None when there is none or the kernel sources changed since it was taken."""
    import os
    syms = KERNEL_SYMBOLS.get(kernel_class)
    path = os.path.join(root, "profiles", stem + "_kernel_stats.txt")
    if syms is None or not os.path.exists(path):
        return None
    lines = open(path).read().splitlines()
    tag = [l for l in lines if l.startswith("# kernel sources sha1:")]
    if not tag or tag[0].split(":", 1)[1].strip() != kernel_source_hash(root):
        return None
    calls = tot = 0.0
    for l in lines:
        if l.startswith("#") or not l.strip() or not any(sym in l for sym in syms):
            continue
        parts = l.split()
        try:
            calls += float(parts[0])
            tot += float(parts[4]) * 1e3  # total ms -> us
        except (ValueError, IndexError):
            return None
    return tot / calls if calls else None


def profiled_traffic(root: str, kernel_class: str, stem: str):
    """HBM bytes per launch (read + write) of a kernel class from the committed counter profile
    profiles/<stem>_hbm_counters.txt, or None when there is none for this class or the kernel
    sources changed since it was taken."""
    import glob
    import os
    syms = KERNEL_SYMBOLS.get(kernel_class)
    if syms is None:
        return None
    cur = kernel_source_hash(root)
    for path in glob.glob(os.path.join(root, "profiles", stem + "_hbm_counters.txt")):
        lines = open(path).read().splitlines()
        tag = [l for l in lines if l.startswith("# kernel sources sha1:")]
        if not tag or tag[0].split(":", 1)[1].strip() != cur:
            continue
        for l in lines:
            if l.startswith("#") or not any(sym in l for sym in syms):
                continue
            parts = l.split()
            try:
                return (float(parts[3]) + float(parts[4])) * 1e6
            except (ValueError, IndexError):
                return None
    return None
