"""GPU parity of the SSD and trapezoidal decode steps: L = 1 calls of ssd_chunk_scan_fwd and
ssd_trap_chunk_scan_fwd carrying the state in place (and, for the trapezoidal form, the
previous x and k) over T steps, against the fp64 sequential oracles over the T steps.

The step kernel forms every product in fp32 from the exact bf16 input values (no bf16
rounding of intermediates), so it is held to the fp32 bar."""
import numpy as np
import pytest

import oracle
import synth
from helpers import TOL_F32, lib, report

pytestmark = pytest.mark.gpu

ZOH, DT, ONE = oracle.BBAR_ZOH, oracle.BBAR_DT, oracle.BBAR_ONE


@pytest.mark.parametrize("case", [  # batch, H, P, N, G, flags
    (3, 4, 64, 128, 2, DT), (2, 2, 32, 96, 1, ZOH), (1, 3, 128, 256, 3, ONE), (2, 2, 64, 32, 1, DT)],
    ids=lambda c: "b{}H{}P{}N{}G{}f{}".format(*c))
def test_ssd_decode_chain(cuda_device, case):
    import torch
    batch, H, P, N, G, flags = case
    T = 20
    inp = synth.ssd_inputs(batch, T, H, P, N, G, seed=(61, N), h0=True, D="normal")
    yo, ho = oracle.ssd_fwd(**inp.arrays, ngroups=G, flags=flags)
    t = inp.torch(cuda_device)
    h = t["h0"].clone()
    m = lib()
    ys = []
    for s in range(T):
        sl = {n: t[n][:, s:s + 1].clone() for n in ("x", "dt", "B", "C")}
        ys.append(m.ssd_chunk_scan_fwd(sl["x"], sl["dt"], t["dt_bias"], t["A_log"], sl["B"], sl["C"], t["D"], h,
                                       flags=flags, h_final=h)[0])
    torch.cuda.synchronize()
    ey = synth.max_rel_err(torch.cat(ys, dim=1).cpu().numpy(), yo)
    eh = synth.max_rel_err(h.cpu().numpy(), ho)
    report(f"ssd decode {case}", y=ey, h_final=eh)
    assert ey <= TOL_F32 and eh <= TOL_F32


@pytest.mark.parametrize("case", [(2, 3, 64, 128), (1, 2, 32, 64), (2, 2, 128, 256)],
                         ids=lambda c: "b{}H{}P{}N{}".format(*c))
def test_trap_decode_chain(cuda_device, case):
    """Each step passes the previous step's x and k (the carried input) and the state in
    place; the first step takes the initial carried pair."""
    import torch
    batch, H, P, N = case
    T = 20
    inp = synth.trap_inputs(batch, T, H, P, N, seed=(62, N), h0=True, prev=True)
    yo, ho = oracle.trap_fwd(**inp.arrays)
    t = inp.torch(cuda_device)
    h = t["h0"].clone()
    kp, xp = t["k_prev"], t["x_prev"]
    m = lib()
    ys = []
    for s in range(T):
        sl = {n: t[n][:, s:s + 1].clone() for n in ("x", "k", "q", "dt", "a", "trap")}
        ys.append(m.ssd_trap_chunk_scan_fwd(sl["x"], sl["k"], sl["q"], sl["dt"], sl["a"], sl["trap"], t["D"], h,
                                            kp, xp, h_final=h)[0])
        kp, xp = sl["k"][:, 0].clone(), sl["x"][:, 0].clone()
    torch.cuda.synchronize()
    ey = synth.max_rel_err(torch.cat(ys, dim=1).cpu().numpy(), yo)
    eh = synth.max_rel_err(h.cpu().numpy(), ho)
    report(f"trap decode {case}", y=ey, h_final=eh)
    assert ey <= TOL_F32 and eh <= TOL_F32
