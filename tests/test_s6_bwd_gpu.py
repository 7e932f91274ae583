"""GPU parity of ssm_s6_scan_bwd against the fp64 backward oracle (every
output, element by element)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import TOL_BWD, lib, report

pytestmark = pytest.mark.gpu

ZOH, DT, ONE = oracle.BBAR_ZOH, oracle.BBAR_DT, oracle.BBAR_ONE
GRADS = ("du", "ddt", "dB", "dC", "dA_log", "dD", "ddt_bias", "dh0")


def gpu_s6_bwd(inp, dy, dhf, device, flags):
    t = inp.torch(device)
    g = lib().ssm_s6_scan_bwd(t["u"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"], t["D"],
                              t["h0"], torch.from_numpy(dy).to(device),
                              None if dhf is None else torch.from_numpy(dhf).to(device),
                              flags=flags)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in g.items()}


def _errs(g, o):
    return {k: synth.max_rel_err(g[k], o[k]) for k in GRADS}


def _check(name, inp, device, flags, tol, dh_final=True, seed=(0,)):
    d = inp.dims
    dy, dhf = synth.s6_cotangents(d["batch"], d["L"], d["d_inner"], d["d_state"], seed=seed,
                                  dh_final=dh_final)
    g = gpu_s6_bwd(inp, dy, dhf, device, flags)
    o = oracle.s6_bwd(**inp.arrays, dy=dy, dh_final=dhf, flags=flags)
    e = _errs(g, o)
    report(name, **e)
    for k in GRADS:
        assert np.isfinite(g[k]).all(), k
    bad = {k: v for k, v in e.items() if not v <= tol}
    assert not bad, bad


def test_s6_bwd_tiny_workload(cuda_device):
    _check("s6_bwd tiny", synth.workload_inputs("s6_tiny"), cuda_device, ZOH, TOL_BWD)


CASES = [  # batch, L, d_inner, d_state, flags, dtype, h0, dh_final, a_log
    (2, 37, 40, 16, ZOH, "f32", True, True, "index"),
    (1, 200, 33, 4, ZOH, "f32", False, False, "index"),
    (3, 17, 16, 1, DT, "f32", True, True, "uniform"),
    (1, 50, 20, 5, ONE, "f32", True, True, "uniform"),
    (2, 64, 48, 16, ZOH, "f32", True, True, "uniform"),
    (1, 1, 3, 16, ZOH, "f32", True, True, "index"),
    (1, 16, 16, 16, DT, "f32", False, True, "index"),
    (2, 300, 70, 16, ZOH, "f32", True, True, "index"),
    (2, 70, 300, 16, ZOH, "bf16", True, True, "index"),
    (1, 64, 48, 8, DT, "bf16", False, False, "uniform"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"b{c[0]}L{c[1]}D{c[2]}N{c[3]}f{c[4]}{c[5]}"
                         f"{'h0' if c[6] else ''}{'dhf' if c[7] else ''}")
def test_s6_bwd_shapes(cuda_device, case):
    batch, L, Dm, N, flags, dtype, h0, dhf, a_log = case
    inp = synth.s6_inputs(batch, L, Dm, N, seed=(200 + L,), dtype=dtype, h0=h0, a_log=a_log)
    _check(f"s6_bwd {case}", inp, cuda_device, flags, TOL_BWD, dh_final=dhf, seed=(L,))


@pytest.mark.parametrize("a_log", [-30.0, -3.0, 4.0])
def test_s6_bwd_degenerate_A(cuda_device, a_log):
    # A -> 0 (series branches everywhere), slow decay, very fast decay
    inp = synth.s6_inputs(2, 45, 20, 16, seed=(17,), a_log=a_log, h0=True)
    _check(f"s6_bwd A_log={a_log}", inp, cuda_device, ZOH, TOL_BWD)


def test_s6_bwd_optional_outputs_and_inputs(cuda_device):
    """NULL dt_bias, D, h0, dh_final; NULL dD, ddt_bias, dh0 outputs are not written."""
    inp = synth.s6_inputs(1, 40, 20, 16, seed=(18,), dt_bias=None, D=None)
    dy, _ = synth.s6_cotangents(1, 40, 20, 16, seed=(18,), dh_final=False)
    t = inp.torch(cuda_device)
    dy_d = torch.from_numpy(dy).to(cuda_device)     # held for the whole call
    s = lib()
    ws = torch.empty(s.ssm_s6_scan_bwd_workspace_size(1, 40, 20, 16), dtype=torch.uint8,
                     device=cuda_device)
    out = {k: torch.full(sh, 7.0, device=cuda_device) for k, sh in
           dict(du=(1, 40, 20), ddt=(1, 40, 20), dB=(1, 40, 16), dC=(1, 40, 16), dA_log=(20, 16)).items()}
    r = s._lib.ssm_s6_scan_bwd(
        s._ptr(t["u"]), s._ptr(t["dt"]), None, s._ptr(t["A_log"]), s._ptr(t["B"]), s._ptr(t["C"]),
        None, None, s._ptr(dy_d), None,
        s._ptr(out["du"]), s._ptr(out["ddt"]), s._ptr(out["dB"]), s._ptr(out["dC"]),
        s._ptr(out["dA_log"]), None, None, None, 1, 40, 20, 16, s.SSM_F32, ZOH,
        s._ptr(ws), ws.numel(), s._stream(cuda_device))
    assert r == 0, s.ssm_last_error()
    torch.cuda.synchronize()
    o = oracle.s6_bwd(**inp.arrays, dy=dy)
    e = {k: synth.max_rel_err(out[k].cpu().numpy(), o[k]) for k in out}
    report("s6_bwd optional", **e)
    assert max(e.values()) <= TOL_BWD, e


def test_s6_bwd_bitwise_deterministic(cuda_device):
    inp = synth.s6_inputs(2, 300, 100, 16, seed=(19,), h0=True)
    dy, dhf = synth.s6_cotangents(2, 300, 100, 16, seed=(19,))
    a = gpu_s6_bwd(inp, dy, dhf, cuda_device, ZOH)
    b = gpu_s6_bwd(inp, dy, dhf, cuda_device, ZOH)
    for k in GRADS:
        assert np.array_equal(a[k], b[k]), k


def test_s6_bwd_mamba1_workload(cuda_device):
    """Full Mamba-1 layer shape (8 x 2048 x 1536, N = 16) in the benchmark's
    launch configuration; every output checked against the oracle."""
    inp = synth.workload_inputs("s6_mamba1")
    d = inp.dims
    dy, dhf = synth.s6_cotangents(d["batch"], d["L"], d["d_inner"], d["d_state"], seed=(1,))
    g = gpu_s6_bwd(inp, dy, dhf, cuda_device, ZOH)
    o = oracle.s6_bwd(**inp.arrays, dy=dy, dh_final=dhf, flags=ZOH)
    e = _errs(g, o)
    report("s6_bwd mamba1", **e)
    bad = {k: v for k, v in e.items() if not v <= TOL_BWD}
    assert not bad, bad


@pytest.mark.parametrize("flags", [ZOH, DT, ONE])
def test_s6_bwd_extreme_dt(cuda_device, flags):
    """Raw dt of -25 (delta ~ 1e-11) next to +25 (delta ~ 25, decays of e^{-25 |A|} and
    below).  Where a step all but erases the state, the derivatives of Abar are of that
    step's size: they take the exponential itself, not the 1 + A beta of the recurrence,
    whose absolute rounding (~1e-7) would otherwise dominate ddt and dA_log."""
    inp = synth.s6_inputs(2, 300, 64, 16, seed=(37,), h0=True)
    dt = inp.arrays["dt"]
    dt[:, ::3] = -25.0
    dt[:, 1::7] = 25.0
    _check(f"s6_bwd extreme dt flags={flags}", inp, cuda_device, flags, TOL_BWD, seed=(37,))
