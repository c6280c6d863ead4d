"""GPU parity of ttt_inplace_down_forward against the CPU oracle: full recurrence at small
sizes; at the full In-Place size (d_model 4096, d_hidden 14336, seq 32768, chunk 1024) sampled
final fast-weight columns and output rows of the first two, a middle and the last chunk."""
import numpy as np
import pytest

from tests._helpers import BF16_TOL, announce, dev, host
from workloads import CONFIGS, InplaceProblem, make_inplace_inputs, max_abs_rel

pytestmark = pytest.mark.gpu


def _gpu(lib, p, x):
    import torch
    return lib.inplace_down_forward(dev(x["Hs"], torch.bfloat16), dev(x["W_gate"], torch.bfloat16),
                                    dev(x["W_up"], torch.bfloat16), dev(x["W_down"], torch.float32),
                                    dev(x["Vbar"], torch.bfloat16), chunk=p.chunk, eta=float(x["eta"]))


@pytest.mark.parametrize("kw", [
    dict(B=2, N=512, d_model=256, d_hidden=512, chunk=128, eta=1e-3),
    dict(B=1, N=1024, d_model=512, d_hidden=768, chunk=256, eta=1e-2),
    dict(B=1, N=256, d_model=256, d_hidden=256, chunk=256, eta=1e-3),
    # apply product 256 x 512 over K = 2048: the large-tile kernel with a four-way K split
    dict(B=1, N=512, d_model=512, d_hidden=2048, chunk=256, eta=1e-3),
])
def test_small_cases(lib, kw):
    from oracle import inplace as IP
    p = InplaceProblem(**kw)
    announce(f"inplace {p}")
    x = make_inplace_inputs(p, 500 + p.N)
    O, W = _gpu(lib, p, x)
    ref = IP.inplace_forward(x["Hs"], x["W_gate"], x["W_up"], x["W_down"], x["Vbar"], float(x["eta"]),
                             chunk=p.chunk)
    eo, ew = max_abs_rel(host(O), ref["O"]), max_abs_rel(host(W), ref["W_down"])
    print(f"inplace O={eo:.2e} W={ew:.2e}")
    assert eo <= BF16_TOL and ew <= BF16_TOL
    # the writes are visible in the outputs
    assert max_abs_rel(ref["W_down"][0], x["W_down"]) > 1e-3


def test_config4_full_size_sampled(lib):
    from oracle import inplace as IP
    p = CONFIGS[4]
    announce("inplace config4 full size (sampled)")
    x = make_inplace_inputs(p, 4)
    O, W = _gpu(lib, p, x)
    cols = [0, 777, 8191, 14335]
    # rows of the first two chunks, a middle chunk (16) and the last chunk (31): the late rows
    # see the writes of every earlier chunk
    rows = [0, 511, 1023, 1024, 1500, 2047, 16 * 1024 + 3, 16 * 1024 + 700, 31 * 1024, 31 * 1024 + 555,
            32 * 1024 - 1]
    f32 = np.float32
    refW = IP.final_wdown_columns(x["Hs"][0], x["W_gate"], x["W_up"], x["W_down"], x["Vbar"][0],
                                  float(x["eta"]), cols, dtype=f32)
    refO = IP.output_rows(x["Hs"][0], x["W_gate"], x["W_up"], x["W_down"], x["Vbar"][0], float(x["eta"]),
                          chunk=p.chunk, rows=rows, dtype=f32)
    ew = max_abs_rel(host(W[0][:, cols]), refW)
    eo = max_abs_rel(host(O[0][rows]), refO)
    print(f"config4 sampled: W cols {ew:.2e}, O rows {eo:.2e}")
    assert ew <= BF16_TOL and eo <= BF16_TOL


# ---- the LM-aligned target built on the device (section 3.2, Eq. 3) ----

def _gpu_target(lib, p, x, taps, W_target=None):
    import torch
    return lib.inplace_down_forward(dev(x["Hs"], torch.bfloat16), dev(x["W_gate"], torch.bfloat16),
                                    dev(x["W_up"], torch.bfloat16), dev(x["W_down"], torch.float32), None,
                                    chunk=p.chunk, eta=float(x["eta"]), X0=dev(x["X0"], torch.bfloat16),
                                    conv_taps=dev(taps, torch.float32),
                                    W_target=None if W_target is None else dev(W_target, torch.bfloat16))


def test_next_token_target_is_bitwise_the_given_shift(lib):
    """Taps (0, 1) and no projection: the device builds exactly the next-token shift, so the call
    equals the one that is handed the shifted embeddings, bit for bit."""
    import torch
    p = InplaceProblem(B=2, N=512, d_model=256, d_hidden=512, chunk=128, eta=1e-2)
    announce(f"inplace next-token target on the device {p}")
    x = make_inplace_inputs(p, 610)
    taps = np.stack([np.zeros(p.d_model, np.float32), np.ones(p.d_model, np.float32)])
    O1, W1 = _gpu(lib, p, x)
    O2, W2 = _gpu_target(lib, p, x, taps)
    assert torch.equal(O1, O2) and torch.equal(W1, W2)


@pytest.mark.parametrize("kw,k,proj", [
    (dict(B=2, N=512, d_model=256, d_hidden=512, chunk=128, eta=5e-2), 3, False),
    (dict(B=1, N=1024, d_model=512, d_hidden=768, chunk=256, eta=5e-2), 4, True),
    # projection product 1024 x 2048 over K = 1024: the large-tile kernel
    (dict(B=1, N=2048, d_model=1024, d_hidden=2048, chunk=256, eta=2e-2), 2, True),
])
def test_general_target(lib, kw, k, proj):
    """General taps and a projection, against the oracle's target and recurrence. The step size is
    raised so that the writes carry weight in the outputs."""
    from oracle import inplace as IP
    from workloads import bf16_round
    p = InplaceProblem(**kw)
    announce(f"inplace LM-aligned target k={k} projection={proj} {p}")
    x = make_inplace_inputs(p, 620 + k)
    rng = np.random.default_rng(k)
    taps = rng.uniform(-1.0, 1.0, (k, p.d_model)).astype(np.float32)
    W_target = bf16_round((rng.standard_normal((p.d_model, p.d_model)) / np.sqrt(p.d_model)).astype(np.float32)) \
        if proj else None
    O, W = _gpu_target(lib, p, x, taps, W_target)
    Vbar = np.stack([IP.lm_aligned_target(x["X0"][b], taps, W_target) for b in range(p.B)])
    ref = IP.inplace_forward(x["Hs"], x["W_gate"], x["W_up"], x["W_down"], Vbar, float(x["eta"]), chunk=p.chunk)
    eo, ew = max_abs_rel(host(O), ref["O"]), max_abs_rel(host(W), ref["W_down"])
    print(f"inplace target O={eo:.2e} W={ew:.2e}", flush=True)
    assert eo <= BF16_TOL and ew <= BF16_TOL
    assert max_abs_rel(ref["W_down"][0], x["W_down"]) > 1e-2  # the writes are visible
