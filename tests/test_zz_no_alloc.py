"""ttt_linattn_forward_noalloc (the allocation-free variant of the scan form) against
ttt_linattn_forward: same bits on two calls in a row, the second with a smaller input; a call
beyond the scratch size is rejected before any launch."""
import ctypes

import numpy as np
import pytest

from tests._helpers import announce, dev, host
from workloads import BF16, CONFIGS, LactProblem, make_lact_inputs

pytestmark = pytest.mark.gpu


def _run(lib, p, x, noalloc, momentum=0.0):
    import torch
    args = [dev(x[k], torch.bfloat16) for k in ("Q", "K", "V")] + [dev(x[k], torch.float32)
                                                                    for k in ("eta", "W0", "W2", "W1")]
    fn = lib.linattn_forward_noalloc if noalloc else lib.linattn_forward
    O, S = fn(*args, chunk=p.chunk_kv, order=p.order, momentum=momentum)
    torch.cuda.synchronize()
    return host(O), host(S)


@pytest.mark.parametrize("momentum", [0.0, 0.9])
def test_noalloc_matches_workspace_entry_point(lib, momentum):
    big = CONFIGS[1]  # B4 H8 h64 r2, 8192 tokens, chunk 512 (the scan workload)
    small = LactProblem(B=1, H=2, h=64, r=2, Nq=1024, Nk=1024, chunk_q=256, chunk_kv=256, dtype=BF16, order=1)
    for p, seed in ((big, 71), (small, 72)):  # second call smaller than the first
        announce(f"noalloc scan {p} momentum {momentum}")
        x = make_lact_inputs(p, seed)
        ref = _run(lib, p, x, noalloc=False, momentum=momentum)
        got = _run(lib, p, x, noalloc=True, momentum=momentum)
        for a, b in zip(got, ref):
            assert np.array_equal(a, b)


def test_noalloc_rejects_a_call_beyond_its_scratch(lib):
    import torch
    p = lib.LinattnParams(4, 8, 65536, 64, 2, 512, 0, lib.BF16, 0, 0.0)
    need = ctypes.c_size_t(0)
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: the call must stop at the size check
    assert lib.load().ttt_linattn_forward(ctypes.byref(p), *[fake] * 8, None, None, ctypes.byref(need), None) == 0
    assert need.value > lib.NOALLOC_SCRATCH_BYTES
    st = lib.load().ttt_linattn_forward_noalloc(ctypes.byref(p), *[fake] * 8, None, None)
    assert st == lib.TTT_ERR_WORKSPACE
    assert "scratch" in lib.last_error()
    torch.cuda.synchronize()
