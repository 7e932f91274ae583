"""GPU parity of ssm_s6_scan_grouped_bwd (gradients of the S6 scan with B, C per group of
channels, up to per channel) against the fp64 grouped backward oracle, element by element."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import TOL_BWD, lib, report

pytestmark = pytest.mark.gpu

ZOH, DT, ONE = oracle.BBAR_ZOH, oracle.BBAR_DT, oracle.BBAR_ONE
GRADS = ("du", "ddt", "dB", "dC", "dA_log", "dD", "ddt_bias", "dh0")


def _gpu(inp, dy, dhf, device, flags):
    t = inp.torch(device)
    g = lib().ssm_s6_scan_grouped_bwd(t["u"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"], t["D"], t["h0"],
                                      torch.from_numpy(dy).to(device),
                                      None if dhf is None else torch.from_numpy(dhf).to(device), flags=flags)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in g.items()}


CASES = [  # batch, L, d_inner, N, ngroups, dtype, flags, h0, dh_final, a_log
    (2, 100, 48, 16, 48, "f32", ZOH, True, True, "index"),       # per channel
    (2, 70, 32, 16, 8, "f32", ZOH, True, True, "uniform"),       # groups of 4 channels
    (1, 37, 20, 8, 20, "f32", DT, False, True, "index"),         # ragged tile and channel block
    (1, 1, 16, 16, 16, "f32", ZOH, True, True, "index"),         # one step
    (1, 130, 24, 12, 6, "bf16", ZOH, True, False, "uniform"),
    (1, 300, 40, 4, 40, "f32", ZOH, True, True, -3.0),           # |A| < 1/8: the series paths
    (2, 64, 16, 16, 16, "f32", ONE, False, True, "index"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b{}L{}D{}N{}G{}{}f{}h{}g{}".format(*[int(v) if isinstance(v, bool) else v for v in c[:9]]))
def test_grouped_bwd_shapes(cuda_device, case):
    batch, L, Dm, N, G, dtype, flags, h0, dhf_on, a_log = case
    inp = synth.s6_inputs(batch, L, Dm, N, seed=(900 + L, G), dtype=dtype, h0=h0, a_log=a_log, ngroups=G)
    dy, dhf = synth.s6_cotangents(batch, L, Dm, N, seed=(L, G), dh_final=dhf_on)
    g = _gpu(inp, dy, dhf, cuda_device, flags)
    o = oracle.s6_grouped_bwd(**inp.arrays, dy=dy, dh_final=dhf, flags=flags)
    errs = {k: synth.max_rel_err(g[k], o[k]) for k in GRADS}
    report(f"s6 grouped bwd {case}", **errs)
    for k in GRADS:
        assert np.isfinite(g[k]).all(), k
        assert errs[k] <= TOL_BWD, (k, errs[k])


def test_one_group_is_the_shared_backward(cuda_device):
    inp = synth.s6_inputs(2, 200, 64, 16, seed=(91,), h0=True, ngroups=1)
    dy, dhf = synth.s6_cotangents(2, 200, 64, 16, seed=(91,))
    t = inp.torch(cuda_device)
    m = lib()
    dyt, dht = torch.from_numpy(dy).to(cuda_device), torch.from_numpy(dhf).to(cuda_device)
    g1 = m.ssm_s6_scan_grouped_bwd(t["u"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"], t["D"], t["h0"],
                                   dyt, dht)
    g2 = m.ssm_s6_scan_bwd(t["u"], t["dt"], t["dt_bias"], t["A_log"], t["B"][:, :, 0].contiguous(),
                           t["C"][:, :, 0].contiguous(), t["D"], t["h0"], dyt, dht)
    torch.cuda.synchronize()
    for k in GRADS:
        a = g1[k][:, :, 0] if k in ("dB", "dC") else g1[k]
        assert torch.equal(a, g2[k]), k


def test_grouped_bwd_per_channel_workload_sampled(cuda_device):
    """Full per-channel shape (8 x 2048 x 1536, N 16): 16 channels over every batch row and
    step against the oracle (per-channel groups make their dB, dC exact on the slice)."""
    w = synth.WORKLOADS["s6_pc_mamba1"]
    inp = synth.workload_inputs("s6_pc_mamba1")
    dy, dhf = synth.s6_cotangents(w["batch"], w["L"], w["d_inner"], w["d_state"], seed=(5,))
    g = _gpu(inp, dy, dhf, cuda_device, ZOH)
    d0 = 704
    a = inp.arrays
    cs = slice(d0, d0 + 16)      # per-channel groups: 16 channels with their own groups form a problem
    sub = dict(u=a["u"][:, :, cs], dt=a["dt"][:, :, cs], dt_bias=a["dt_bias"][cs], A_log=a["A_log"][cs],
               B=a["B"][:, :, cs], C=a["C"][:, :, cs], D=a["D"][cs], h0=None if a["h0"] is None else a["h0"][:, cs])
    o = oracle.s6_grouped_bwd(**sub, dy=dy[:, :, cs], dh_final=dhf[:, cs])
    sl = {"du": g["du"][:, :, d0:d0 + 16], "ddt": g["ddt"][:, :, d0:d0 + 16],
          "dB": g["dB"][:, :, d0:d0 + 16], "dC": g["dC"][:, :, d0:d0 + 16],
          "dA_log": g["dA_log"][d0:d0 + 16], "dD": g["dD"][d0:d0 + 16], "ddt_bias": g["ddt_bias"][d0:d0 + 16],
          "dh0": g["dh0"][:, d0:d0 + 16]}
    errs = {k: synth.max_rel_err(sl[k], o[k]) for k in GRADS}
    report("s6_pc_mamba1 bwd sampled", **errs)
    for k in GRADS:
        assert errs[k] <= TOL_BWD, (k, errs[k])


@pytest.mark.parametrize("G", [64, 16])
@pytest.mark.parametrize("flags", [ZOH, DT])
def test_grouped_bwd_extreme_dt(cuda_device, flags, G):
    """Raw dt of -25 next to +25: the derivatives of Abar at steps that all but erase the
    state are of those steps' size (the exponential itself, not 1 + A beta)."""
    inp = synth.s6_inputs(2, 300, 64, 16, seed=(38, G), h0=True, ngroups=G)
    dt = inp.arrays["dt"]
    dt[:, ::3] = -25.0
    dt[:, 1::7] = 25.0
    dy, dhf = synth.s6_cotangents(2, 300, 64, 16, seed=(38,))
    g = _gpu(inp, dy, dhf, cuda_device, flags)
    o = oracle.s6_grouped_bwd(**inp.arrays, dy=dy, dh_final=dhf, flags=flags)
    errs = {k: synth.max_rel_err(g[k], o[k]) for k in GRADS}
    report(f"s6 grouped bwd extreme dt flags={flags} G={G}", **errs)
    for k in GRADS:
        assert np.isfinite(g[k]).all(), k
        assert errs[k] <= TOL_BWD, (k, errs[k])
