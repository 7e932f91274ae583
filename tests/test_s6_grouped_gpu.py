"""GPU parity of ssm_s6_scan_grouped_fwd (the S6 scan with B, C per group of channels, up to
per channel) against the fp64 grouped S6 oracle."""
import numpy as np
import pytest

import oracle
import synth
from helpers import TOL_BF16, TOL_F32, lib, report, sample_units

pytestmark = pytest.mark.gpu

ZOH, DT, ONE = oracle.BBAR_ZOH, oracle.BBAR_DT, oracle.BBAR_ONE


def _gpu(inp, device, flags):
    import torch
    t = inp.torch(device)
    y, hf = lib().ssm_s6_scan_grouped_fwd(t["u"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"], t["D"],
                                          t["h0"], flags=flags, return_final=True)
    torch.cuda.synchronize()
    return y.cpu().numpy(), hf.cpu().numpy()


CASES = [  # batch, L, d_inner, N, ngroups, dtype, flags, h0, a_log
    (2, 100, 48, 16, 48, "f32", ZOH, True, "index"),       # per channel
    (1, 37, 20, 16, 20, "f32", DT, False, "index"),        # ragged tile and channel block
    (2, 5, 33, 32, 11, "f32", ZOH, True, "uniform"),       # two states per lane, groups of 3
    (1, 1, 16, 4, 16, "f32", ONE, True, "index"),          # one step, 4 of 16 lanes hold a state
    (3, 17, 24, 20, 6, "bf16", ZOH, True, "uniform"),      # bf16, 20 states, groups of 4
    (1, 300, 40, 8, 40, "f32", ZOH, True, -3.0),           # |A| < 1/8: the series path
    (2, 64, 64, 16, 2, "f32", ZOH, True, "index"),         # groups of 32
    (1, 513, 16, 16, 16, "bf16", DT, True, "index"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b{}L{}D{}N{}G{}{}f{}h{}".format(*[int(v) if isinstance(v, bool) else v for v in c[:8]]))
def test_grouped_shapes(cuda_device, case):
    batch, L, Dm, N, G, dtype, flags, h0, a_log = case
    inp = synth.s6_inputs(batch, L, Dm, N, seed=(600 + L, G), dtype=dtype, h0=h0, a_log=a_log, ngroups=G)
    y, hf = _gpu(inp, cuda_device, flags)
    yo, ho = oracle.s6_grouped_fwd(**inp.arrays, flags=flags)
    ey, eh = synth.max_rel_err(y, yo), synth.max_rel_err(hf, ho)
    report(f"s6 grouped {case}", y=ey, h_final=eh)
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    assert np.isfinite(y).all() and np.isfinite(hf).all()
    assert ey <= tol and eh <= tol


def test_one_group_is_the_shared_kernel(cuda_device):
    """ngroups = 1 runs the shared-B kernel: equal bits to ssm_s6_scan_fwd."""
    import torch
    inp = synth.s6_inputs(2, 300, 96, 16, seed=(61,), h0=True, ngroups=1)
    t = inp.torch(cuda_device)
    m = lib()
    y1, h1 = m.ssm_s6_scan_grouped_fwd(t["u"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"], t["D"], t["h0"],
                                       return_final=True)
    y2, h2 = m.ssm_s6_scan_fwd(t["u"], t["dt"], t["dt_bias"], t["A_log"], t["B"][:, :, 0].contiguous(),
                               t["C"][:, :, 0].contiguous(), t["D"], t["h0"], return_final=True)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(h1, h2)


def test_decode_steps_in_place(cuda_device):
    """T single-step calls carrying h in place equal the oracle over T steps."""
    import torch
    T = 12
    inp = synth.s6_inputs(2, T, 32, 16, seed=(62,), h0=True, ngroups=32)
    yo, ho = oracle.s6_grouped_fwd(**inp.arrays)
    t = inp.torch(cuda_device)
    h = t["h0"].clone()
    m = lib()
    ys = []
    for s in range(T):
        sl = {n: t[n][:, s:s + 1].clone() for n in ("u", "dt", "B", "C")}
        ys.append(m.ssm_s6_scan_grouped_fwd(sl["u"], sl["dt"], t["dt_bias"], t["A_log"], sl["B"], sl["C"], t["D"],
                                            h, h_final=h)[0])
    torch.cuda.synchronize()
    ey = synth.max_rel_err(torch.cat(ys, 1).cpu().numpy(), yo)
    eh = synth.max_rel_err(h.cpu().numpy(), ho)
    report("s6 grouped decode", y=ey, h_final=eh)
    assert ey <= TOL_F32 and eh <= TOL_F32


def test_per_channel_workload_sampled(cuda_device):
    """Full per-channel shape (8 x 2048 x 1536, N 16, fp32) against the oracle on 48 sampled
    (b, d) channels over the whole sequence."""
    w = synth.WORKLOADS["s6_pc_mamba1"]
    inp = synth.workload_inputs("s6_pc_mamba1")
    y, hf = _gpu(inp, cuda_device, ZOH)
    units = sample_units(np.random.default_rng(8), w["batch"], w["d_inner"], 48)
    yo, ho = oracle.s6_grouped_fwd(**inp.arrays, units=units)
    yg = np.stack([y[b, :, d] for b, d in units])
    hg = np.stack([hf[b, d] for b, d in units])
    ey, eh = synth.max_rel_err(yg, yo), synth.max_rel_err(hg, ho)
    report("s6_pc_mamba1 sampled", y=ey, h_final=eh)
    assert ey <= TOL_F32 and eh <= TOL_F32
