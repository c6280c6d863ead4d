"""GPU parity of the LaCT loop variants against the CPU oracle: per-chunk apply-only and reset
flags, several inner steps per chunk, both together, and one step-size row per matrix. Same tolerances as the plain loop
(max-abs-relative 2e-2 in bf16 mode, 1e-4 in fp32 mode); every output is compared: O, the final
fast weights and the final momentum."""
import numpy as np
import pytest

from tests._helpers import BF16_TOL, FP32_TOL, announce, dev, host, lact_on_gpu, lact_oracle
from tests.test_gpu_lact import _compare
from workloads import BF16, FP32, LactProblem, make_lact_inputs, max_abs_rel

pytestmark = pytest.mark.gpu

NO_UPD, RESET = 1, 2


def _flags(B, nch, seed):
    """Every sequence gets a different mix: resets, apply-only chunks and both on one chunk."""
    rng = np.random.default_rng(seed)
    f = np.zeros((B, nch), np.uint8)
    for b in range(B):
        for c in rng.choice(nch, size=min(3, nch), replace=False):
            f[b, c] = (NO_UPD, RESET, NO_UPD | RESET)[(b + int(c)) % 3]
    f[0, :] = 0
    f[0, nch // 2] = RESET  # the first sequence: one document boundary only
    return f


CASES = [
    # (label, problem kwargs, flags?, inner steps, seed)
    ("bf16 AU muon mom h128 flags", dict(h=128, N=2048, chunk=256, muon=True, momentum=0.9), True, 1, 1),
    ("bf16 UA muon h128 flags", dict(h=128, N=2048, chunk=256, muon=True, order=1), True, 1, 2),
    ("bf16 AU muon mom h64 two steps", dict(h=64, N=1024, chunk=128, muon=True, momentum=0.9), False, 2, 3),
    ("bf16 UA mom h128 three steps", dict(h=128, N=1024, chunk=256, momentum=0.5, order=1), False, 3, 4),
    ("bf16 AU muon mom h128 flags two steps", dict(h=128, N=2048, chunk=256, muon=True, momentum=0.9), True, 2, 5),
    ("bf16 AU h192 flags (tiled update)", dict(h=192, N=512, chunk=128, muon=True), True, 2, 6),
    ("fp32 AU muon mom h64 flags two steps", dict(h=64, N=512, chunk=64, muon=True, momentum=0.9, dtype=FP32),
     True, 2, 7),
    ("fp32 UA h32 flags three steps", dict(h=32, N=256, chunk=32, momentum=0.9, order=1, dtype=FP32), True, 3, 8),
]


@pytest.mark.parametrize("label,kw,use_flags,steps,seed", CASES, ids=[c[0] for c in CASES])
def test_loop_variants(lib, label, kw, use_flags, steps, seed):
    import torch
    kw = dict(kw)
    N, chunk = kw.pop("N"), kw.pop("chunk")
    base = dict(B=3, H=2, h=64, r=2, Nq=N, Nk=N, chunk_q=chunk, chunk_kv=chunk, dtype=BF16, v_normalised=False)
    base.update(kw)
    p = LactProblem(**base)
    nch = N // chunk
    x = make_lact_inputs(p, 900 + seed)
    flags = _flags(p.B, nch, seed) if use_flags else None
    announce(f"lact variants {label}: flags {None if flags is None else flags.tolist()} steps {steps}")
    gpu = lact_on_gpu(lib, p, x, chunk_flags=None if flags is None else dev(flags, torch.uint8),
                      inner_steps=steps)
    ref = lact_oracle(p, x, chunk_flags=flags, inner_steps=steps)
    _compare(gpu, ref, BF16_TOL if p.dtype == BF16 else FP32_TOL, label=label)


def test_all_flags_clear_is_bitwise_the_plain_loop(lib):
    """A flag array of zeros (the flag kernels run but select no pair) gives the plain loop's
    results bit for bit."""
    import torch
    p = LactProblem(B=2, H=4, h=128, r=2, Nq=1024, Nk=1024, chunk_q=256, chunk_kv=256, dtype=BF16, muon=True,
                    momentum=0.9, v_normalised=False)
    announce("lact variants: zero flags vs plain")
    x = make_lact_inputs(p, 950)
    plain = lact_on_gpu(lib, p, x)
    zero = lact_on_gpu(lib, p, x, chunk_flags=dev(np.zeros((2, 4), np.uint8), torch.uint8))
    for a, b in zip(plain, zero):
        assert torch.equal(a, b)


def test_lm_shape_with_document_boundaries(lib):
    """The LM layer's shape (B4 H8 h128 r2, chunk 2048) over 8 chunks with document boundaries and
    apply-only chunks; sampled pairs against the oracle."""
    import torch
    p = LactProblem(B=4, H=8, h=128, r=2, Nq=16384, Nk=16384, chunk_q=2048, chunk_kv=2048, dtype=BF16, muon=True,
                    momentum=0.9, v_normalised=False)
    nch = 8
    flags = np.zeros((4, nch), np.uint8)
    flags[1, 3] = RESET
    flags[2, [2, 5]] = NO_UPD
    flags[3, 4] = RESET | NO_UPD
    announce(f"lact variants LM shape flags {flags.tolist()}")
    x = make_lact_inputs(p, 960)
    gpu = lact_on_gpu(lib, p, x, chunk_flags=dev(flags, torch.uint8))
    pairs = [(1, 2), (2, 5), (3, 7)]
    ref = lact_oracle(p, x, pairs=pairs, chunk_flags=flags)
    _compare(gpu, ref, BF16_TOL, pairs=pairs, label="LM shape flags")


ETA3_CASES = [
    # (label, problem kwargs, seed): the role-split gradient kernel (h 64, 128), the register-direct
    # one (h 32, fp32) and the LDS one (h 192)
    ("bf16 AU muon mom h128", dict(h=128, N=1024, chunk=256, muon=True, momentum=0.9), 11),
    ("bf16 UA muon h64", dict(h=64, N=512, chunk=128, muon=True, order=1), 12),
    ("bf16 AU mom h32", dict(h=32, N=384, chunk=96, momentum=0.5), 13),
    ("bf16 AU muon h192", dict(h=192, N=512, chunk=256, muon=True), 14),
    ("fp32 AU muon mom h64", dict(h=64, N=256, chunk=64, muon=True, momentum=0.9, dtype=FP32), 15),
]


@pytest.mark.parametrize("label,kw,seed", ETA3_CASES, ids=[c[0] for c in ETA3_CASES])
def test_eta_per_matrix(lib, label, kw, seed):
    """One step-size row per matrix (eta [B,H,3,Nk]): rows of different scales, so that a row
    applied to the wrong matrix shows."""
    kw = dict(kw)
    N, chunk = kw.pop("N"), kw.pop("chunk")
    base = dict(B=2, H=2, h=64, r=2, Nq=N, Nk=N, chunk_q=chunk, chunk_kv=chunk, dtype=BF16, v_normalised=False)
    base.update(kw)
    p = LactProblem(**base)
    x = make_lact_inputs(p, 980 + seed)
    rng = np.random.default_rng(seed)
    e = x["eta"]
    x["eta"] = np.stack([0.25 * e, 2.0 * e, e * rng.uniform(0.5, 1.5, e.shape).astype(np.float32)], axis=2)
    announce(f"lact eta per matrix {label}")
    gpu = lact_on_gpu(lib, p, x)
    ref = lact_oracle(p, x)
    _compare(gpu, ref, BF16_TOL if p.dtype == BF16 else FP32_TOL, label=label)


@pytest.mark.parametrize("h,dtype", [(128, BF16), (32, BF16), (192, BF16), (64, FP32)])
def test_eta_per_matrix_with_equal_rows_matches_shared_eta(lib, h, dtype):
    """Three equal rows give the shared-eta results. The per-matrix kernels do the same
    arithmetic, but the compiler may round an epilogue product to fp16 once (a fused multiply
    and convert) where the shared-eta build rounds it to fp32 first, so single intermediates can
    differ by one fp16 unit. Bounds: the fp32 states within 1e-4 max-abs-relative, O (bf16)
    within one bf16 unit (2^-8 of the largest output); a row applied to the wrong matrix moves
    them by the rows' ratio, here x1."""
    p = LactProblem(B=2, H=4, h=h, r=2, Nq=512, Nk=512, chunk_q=128, chunk_kv=128, dtype=dtype, muon=False,
                    momentum=0.9, v_normalised=False)
    announce(f"lact eta per matrix: equal rows vs shared h{h} dtype {dtype}")
    x = make_lact_inputs(p, 990)
    shared = lact_on_gpu(lib, p, x)
    y = dict(x)
    y["eta"] = np.stack([x["eta"]] * 3, axis=2)
    per = lact_on_gpu(lib, p, y)
    errs = {n: max_abs_rel(host(b), host(a)) for n, a, b in zip(("O", "W0", "W1", "W2", "M"), shared, per)}
    print("equal rows vs shared:", errs, flush=True)
    assert errs["O"] <= 2.0 ** -8 and all(errs[k] <= 1e-4 for k in ("W0", "W1", "W2", "M")), errs
