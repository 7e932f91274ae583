"""GPU parity of the S6 saved-state pair: ssm_s6_scan_fwd_save (the forward that also saves
the state entering each 16-step tile) and ssm_s6_scan_bwd_saved (the backward that reads
them instead of recomputing), against the forward entry point, the fp64 forward oracle (the
saved states, through the forward's own prefix runs) and the fp64 backward oracle (the
gradients)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import TOL_BWD, TOL_F32, lib, report

pytestmark = pytest.mark.gpu

ZOH, DT, ONE = oracle.BBAR_ZOH, oracle.BBAR_DT, oracle.BBAR_ONE
GRADS = ("du", "ddt", "dB", "dC", "dA_log", "dD", "ddt_bias", "dh0")

CASES = [  # batch, L, d_inner, N, dtype, flags, h0, dh_final
    (2, 100, 48, 16, "f32", ZOH, True, True),
    (1, 16, 20, 16, "f32", DT, False, True),     # exactly one tile
    (1, 1, 16, 16, "f32", ZOH, True, True),      # one step
    (2, 257, 33, 8, "f32", ONE, True, False),    # ragged tail, ragged channel block
    (1, 300, 40, 4, "bf16", ZOH, True, True),
    (2, 129, 64, 16, "f32", ZOH, False, True),
]


def _run(inp, device, flags, dy, dhf):
    t = inp.torch(device)
    m = lib()
    y, hf, ck = m.ssm_s6_scan_fwd_save(t["u"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"], t["D"],
                                       t["h0"], flags=flags)
    y0, h0f = m.ssm_s6_scan_fwd(t["u"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"], t["D"], t["h0"],
                                flags=flags, return_final=True)
    dyt = torch.from_numpy(dy).to(device)
    dht = None if dhf is None else torch.from_numpy(dhf).to(device)
    gs = m.ssm_s6_scan_bwd_saved(t["u"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"], t["D"], t["h0"],
                                 dyt, dht, ck, flags=flags)
    gr = m.ssm_s6_scan_bwd(t["u"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"], t["D"], t["h0"],
                           dyt, dht, flags=flags)
    torch.cuda.synchronize()
    # L > 1: the outputs of ssm_s6_scan_fwd, bit for bit.  L = 1: the plain entry point takes
    # the one-step kernel, so the saving forward is held to the fp32 bar against the oracle
    if t["u"].shape[1] > 1:
        same_fwd = torch.equal(y, y0) and torch.equal(hf, h0f)
    else:
        yo, ho = oracle.s6_fwd(**inp.arrays, flags=flags)
        same_fwd = (synth.max_rel_err(y.cpu().numpy(), yo) <= TOL_F32
                    and synth.max_rel_err(hf.cpu().numpy(), ho) <= TOL_F32)
    return (ck.cpu().numpy(), same_fwd, {k: v.cpu().numpy() for k, v in gs.items()},
            {k: v.cpu().numpy() for k, v in gr.items()})


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b{}L{}D{}N{}{}f{}h{}g{}".format(*[int(v) if isinstance(v, bool) else v for v in c]))
def test_saved_pair(cuda_device, case):
    batch, L, Dm, N, dtype, flags, h0, dhf_on = case
    inp = synth.s6_inputs(batch, L, Dm, N, seed=(700 + L, Dm), dtype=dtype, h0=h0)
    dy, dhf = synth.s6_cotangents(batch, L, Dm, N, seed=(L,), dh_final=dhf_on)
    ck, same_fwd, gs, gr = _run(inp, cuda_device, flags, dy, dhf)
    assert same_fwd
    # the saved states: tile 0 holds h0 (or 0); tile k is the forward's own state after step
    # 16k - 1, i.e. the h_final of ssm_s6_scan_fwd on the first 16k steps, bit for bit (that
    # state's parity with the oracle is the forward's h_final parity)
    a = inp.arrays
    h0ref = a["h0"] if a["h0"] is not None else np.zeros((batch, Dm, N), np.float32)
    assert np.array_equal(ck[:, 0], h0ref)
    t = inp.torch(cuda_device)
    nt = ck.shape[1]
    for kt in sorted(k for k in {1, nt // 2, nt - 1} if 0 < k < nt):
        pre = {k: (t[k][:, :16 * kt].clone() if k in ("u", "dt", "B", "C") else t[k]) for k in t}
        _, hk = lib().ssm_s6_scan_fwd(pre["u"], pre["dt"], pre["dt_bias"], pre["A_log"], pre["B"], pre["C"],
                                      pre["D"], pre["h0"], flags=flags, return_final=True)
        torch.cuda.synchronize()
        assert np.array_equal(ck[:, kt], hk.cpu().numpy()), kt
    # the gradients: against the oracle at the backward's bar, and next to the recomputing backward
    o = oracle.s6_bwd(**a, dy=dy, dh_final=dhf, flags=flags)
    errs = {k: synth.max_rel_err(gs[k], o[k]) for k in GRADS}
    diffs = {k: synth.max_rel_err(gs[k], gr[k]) for k in GRADS}
    report(f"s6 saved {case}", **errs)
    for k in GRADS:
        assert np.isfinite(gs[k]).all(), k
        assert errs[k] <= TOL_BWD, (k, errs[k])
        assert diffs[k] <= 1e-5, (k, diffs[k])     # the same arithmetic up to the states' rounding


def test_saved_pair_mamba1_workload(cuda_device):
    """Full Mamba-1 scan shape (8 x 2048 x 1536, N 16): the saving forward equals the plain one
    bit for bit, and the saved-state backward matches the recomputing backward."""
    w = synth.WORKLOADS["s6_mamba1"]
    inp = synth.workload_inputs("s6_mamba1")
    dy, dhf = synth.s6_cotangents(w["batch"], w["L"], w["d_inner"], w["d_state"], seed=(3,))
    ck, same_fwd, gs, gr = _run(inp, cuda_device, ZOH, dy, dhf)
    assert same_fwd
    diffs = {k: synth.max_rel_err(gs[k], gr[k]) for k in GRADS}
    report("s6_mamba1 saved vs recomputed", **diffs)
    for k in GRADS:
        assert diffs[k] <= 1e-5, (k, diffs[k])
