"""GPU parity of ssm_causal_conv1d_fwd (causal depthwise conv1d + SiLU, carried state)
against the fp64 numpy oracle.  fp32 outputs are held to 1e-5 (K <= 4 products and SiLU in
fp32); bf16 outputs to one rounding of the exact value (2^-8 relative) plus 1e-5 of the
largest value."""
import numpy as np
import pytest

import oracle
import synth
from helpers import lib, report

pytestmark = pytest.mark.gpu


def _gpu(inp, device, silu, **kw):
    import torch
    t = inp.torch(device)
    y, so = lib().ssm_causal_conv1d_fwd(t["x"], t["w"], t["bias"], t["state"], silu=silu, return_state=True, **kw)
    torch.cuda.synchronize()
    return y.float().cpu().numpy(), None if so is None else so.cpu().numpy()


def _check(name, inp, y, yo, dtype):
    scale = float(np.abs(yo).max())
    if dtype == "f32":
        e = synth.max_rel_err(y, yo)
        report(name, y=e)
        assert e <= 1e-5
    else:
        ex = float((np.abs(y - yo) - 2.0 ** -8 * np.abs(yo)).max() / scale)
        report(name, excess_over_rounding=ex)
        assert ex <= 1e-5


CASES = [  # batch, L, channels, K, dtype, silu, state
    (2, 100, 64, 4, "bf16", True, True),       # 8 channels per lane
    (1, 37, 24, 3, "bf16", False, True),
    (2, 70, 36, 4, "f32", True, True),         # 4 channels per lane
    (1, 65, 7, 4, "f32", True, False),         # one channel per lane
    (1, 129, 13, 2, "bf16", True, True),       # one channel per lane, bf16
    (3, 2, 16, 4, "f32", False, True),         # shorter than the conv: state tail carried
    (1, 50, 40, 1, "bf16", True, False),       # K = 1: no state
    (2, 300, 1792, 4, "bf16", True, True),     # Mamba-2 x, B, C channels
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b{}L{}C{}K{}{}s{}st{}".format(*[int(v) if isinstance(v, bool) else v for v in c]))
def test_conv_shapes(cuda_device, case):
    batch, L, Cc, K, dtype, silu, st = case
    inp = synth.conv_inputs(batch, L, Cc, K, seed=(L, Cc), dtype=dtype, state=st)
    y, so = _gpu(inp, cuda_device, silu)
    a = inp.arrays
    yo, soo = oracle.causal_conv1d(a["x"], a["w"], a["bias"], a["state"], silu=silu)
    _check(f"conv {case}", inp, y, yo, dtype)
    if K > 1:
        assert np.array_equal(so, soo.astype(np.float32))


def test_conv_state_in_place_carry(cuda_device):
    """Two calls carrying the state in place equal one call, bit for bit."""
    import torch
    inp = synth.conv_inputs(2, 200, 64, 4, seed=(71,), dtype="bf16")
    t = inp.torch(cuda_device)
    m = lib()
    y_all, s_all = m.ssm_causal_conv1d_fwd(t["x"], t["w"], t["bias"], t["state"], silu=True, return_state=True)
    st = t["state"].clone()
    y1 = m.ssm_causal_conv1d_fwd(t["x"][:, :77].clone(), t["w"], t["bias"], st, silu=True, state_out=st)[0]
    y2 = m.ssm_causal_conv1d_fwd(t["x"][:, 77:].clone(), t["w"], t["bias"], st, silu=True, state_out=st)[0]
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([y1, y2], dim=1), y_all) and torch.equal(st, s_all)


def test_conv_mamba2_workload(cuda_device):
    """Full Mamba-2 conv (8 x 4096 x 1792 channels, K 4, bf16, SiLU), every element."""
    inp = synth.workload_inputs("conv_mamba2")
    y, so = _gpu(inp, cuda_device, True)
    a = inp.arrays
    yo, soo = oracle.causal_conv1d(a["x"], a["w"], a["bias"], a["state"], silu=True)
    _check("conv_mamba2", inp, y, yo, "bf16")
    assert np.array_equal(so, soo.astype(np.float32))
