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
