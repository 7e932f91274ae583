"""GPU parity of ssd_cplx_mimo_chunk_scan_fwd (fp32, rank R inputs and outputs per head
and step) against the fp64 MIMO oracle, and rank 1 against the complex SSD entry point."""
import numpy as np
import pytest

import oracle
import synth
from helpers import TOL_F32, lib, report, sample_units

pytestmark = pytest.mark.gpu

ZOH, DT, ONE, CONJ = oracle.BBAR_ZOH, oracle.BBAR_DT, oracle.BBAR_ONE, oracle.CPLX_CONJ_C


def _gpu(inp, device, flags, Q=64):
    import torch
    t = inp.torch(device)
    y, hf = lib().ssd_cplx_mimo_chunk_scan_fwd(t["x"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"],
                                               t["D"], t["h0"], chunk_len=Q, flags=flags, return_final=True)
    torch.cuda.synchronize()
    return y.cpu().numpy(), hf.cpu().numpy()


CASES = [  # batch, L, rank, H, P, Nc, G, flags, h0
    (2, 50, 2, 4, 64, 32, 1, ZOH, True),
    (1, 37, 4, 4, 32, 16, 2, ZOH, False),            # ragged: 148 rows
    (2, 300, 4, 2, 64, 32, 1, ZOH, True),            # several segments
    (1, 130, 8, 2, 128, 64, 1, DT, True),
    (1, 90, 2, 2, 64, 24, 1, ZOH | CONJ, True),
    (1, 70, 16, 2, 32, 8, 1, ONE, True),             # a step fills a 16-row tile
    (1, 1, 16, 2, 64, 32, 1, ZOH, True),             # one step
    (1, 3, 4, 3, 32, 8, 3, ZOH, True),
    (1, 700, 2, 2, 64, 32, 2, ZOH, False),
    (1, 45, 4, 12, 32, 16, 1, ZOH, True),           # 12 heads per group: two prep blocks
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b{}L{}R{}H{}P{}N{}G{}f{}h{}".format(*[int(v) if isinstance(v, bool) else v for v in c]))
def test_mimo_shapes(cuda_device, case):
    batch, L, R, H, P, Nc, G, flags, h0 = case
    inp = synth.mimo_inputs(batch, L, R, H, P, Nc, G, seed=(400 + L, R), h0=h0)
    y, hf = _gpu(inp, cuda_device, flags)
    yo, ho = oracle.cssd_mimo_fwd(**inp.arrays, ngroups=G, flags=flags)
    ey, eh = synth.max_rel_err(y, yo), synth.max_rel_err(hf, ho)
    report(f"cssd mimo {case}", y=ey, h_final=eh)
    assert np.isfinite(y).all() and np.isfinite(hf).all()
    assert ey <= TOL_F32 and eh <= TOL_F32


def test_rank_one_is_the_complex_ssd_entry_point(cuda_device):
    """With rank 1 the two entry points run the same kernels on the same rows: equal bits."""
    import torch
    inp = synth.mimo_inputs(2, 600, 1, 2, 64, 32, 1, seed=(41,), h0=True)
    t = inp.torch(cuda_device)
    m = lib()
    y1, h1 = m.ssd_cplx_mimo_chunk_scan_fwd(t["x"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"], t["D"],
                                            t["h0"], return_final=True)
    y2, h2 = m.ssd_cplx_chunk_scan_fwd(t["x"][:, :, 0].contiguous(), t["dt"], t["dt_bias"], t["A_log"],
                                       t["B"][:, :, 0].contiguous(), t["C"][:, :, 0].contiguous(), t["D"],
                                       t["h0"], return_final=True)
    torch.cuda.synchronize()
    assert torch.equal(y1[:, :, 0], y2) and torch.equal(h1, h2)


def test_two_calls_carry_the_state(cuda_device):
    import torch
    inp = synth.mimo_inputs(1, 400, 4, 2, 64, 32, 1, seed=(42,), h0=True)
    yo, ho = oracle.cssd_mimo_fwd(**inp.arrays)
    t = inp.torch(cuda_device)
    m = lib()
    c = 150
    part = {n: (t[n][:, :c].clone(), t[n][:, c:].clone()) for n in ("x", "dt", "B", "C")}
    ya, ha = m.ssd_cplx_mimo_chunk_scan_fwd(part["x"][0], part["dt"][0], t["dt_bias"], t["A_log"], part["B"][0],
                                            part["C"][0], t["D"], t["h0"], return_final=True)
    yb, hb = m.ssd_cplx_mimo_chunk_scan_fwd(part["x"][1], part["dt"][1], t["dt_bias"], t["A_log"], part["B"][1],
                                            part["C"][1], t["D"], ha, return_final=True)
    torch.cuda.synchronize()
    ey = synth.max_rel_err(torch.cat([ya, yb], 1).cpu().numpy(), yo)
    eh = synth.max_rel_err(hb.cpu().numpy(), ho)
    report("cssd mimo two calls", y=ey, h_final=eh)
    assert ey <= TOL_F32 and eh <= TOL_F32


def test_mimo_workload_sampled(cuda_device):
    """Full rank-4 shape (4 x 4096 steps, 32 heads x 64, 32 complex states) against the
    oracle on 4 sampled (b, head) units over the whole sequence."""
    w = synth.WORKLOADS["cssd_mimo_mamba3"]
    inp = synth.workload_inputs("cssd_mimo_mamba3")
    y, hf = _gpu(inp, cuda_device, ZOH, w["chunk_len"])
    units = sample_units(np.random.default_rng(3), w["batch"], w["nheads"], 4)
    yo, ho = oracle.cssd_mimo_fwd(**inp.arrays, ngroups=w["ngroups"], units=units)
    yg = np.stack([y[b, :, :, h, :] for b, h in units])
    hg = np.stack([hf[b, h] for b, h in units])
    ey, eh = synth.max_rel_err(yg, yo), synth.max_rel_err(hg, ho)
    report("cssd_mimo_mamba3 sampled", y=ey, h_final=eh)
    assert ey <= TOL_F32 and eh <= TOL_F32
