"""GPU parity of ssd_chunk_scan_bwd against the fp64 SSD backward oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import TOL_BWD, lib, report

pytestmark = pytest.mark.gpu

ZOH, DT, ONE = oracle.BBAR_ZOH, oracle.BBAR_DT, oracle.BBAR_ONE
GRADS = ("dx", "ddt", "dB", "dC", "dA_log", "dD", "ddt_bias", "dh0")


def _cot(batch, L, H, P, N, seed, dh_final=True):
    rng = np.random.default_rng([5, *seed])
    dy = rng.standard_normal((batch, L, H, P), dtype=np.float32)
    dhf = rng.standard_normal((batch, H, P, N), dtype=np.float32) if dh_final else None
    return dy, dhf


def gpu_ssd_bwd(inp, dy, dhf, device, flags):
    t = inp.torch(device)
    g = lib().ssd_chunk_scan_bwd(t["x"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"], t["D"],
                                 t["h0"], torch.from_numpy(dy).to(device),
                                 None if dhf is None else torch.from_numpy(dhf).to(device),
                                 flags=flags)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in g.items()}


CASES = [  # batch, L, H, P, N, G, flags, h0, dh_final
    (1, 40, 2, 32, 32, 1, DT, True, True),
    (2, 300, 4, 64, 64, 2, DT, True, True),
    (1, 777, 3, 32, 128, 3, ZOH, True, True),
    (1, 600, 2, 64, 32, 1, ONE, False, False),
    (2, 1000, 2, 128, 64, 1, DT, True, True),
    (1, 64, 2, 64, 128, 1, DT, False, True),
    (1, 1, 1, 32, 32, 1, ZOH, True, True),
    (1, 2100, 2, 32, 32, 1, DT, True, True),     # 8 segments of at most 512 steps
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"b{c[0]}L{c[1]}H{c[2]}P{c[3]}N{c[4]}G{c[5]}f{c[6]}"
                         f"{'h0' if c[7] else ''}{'dhf' if c[8] else ''}")
def test_ssd_bwd_shapes(cuda_device, case):
    batch, L, H, P, N, G, flags, h0, dhf_on = case
    inp = synth.ssd_inputs(batch, L, H, P, N, G, seed=(300 + L,), h0=h0, D="normal")
    dy, dhf = _cot(batch, L, H, P, N, (L,), dhf_on)
    g = gpu_ssd_bwd(inp, dy, dhf, cuda_device, flags)
    o = oracle.ssd_bwd(**inp.arrays, dy=dy, dh_final=dhf, ngroups=G, flags=flags)
    e = {k: synth.max_rel_err(g[k], o[k]) for k in GRADS}
    report(f"ssd_bwd {case}", **e)
    for k in GRADS:
        assert np.isfinite(g[k]).all(), k
    bad = {k: v for k, v in e.items() if not v <= TOL_BWD}
    assert not bad, bad


def test_ssd_bwd_bitwise_deterministic(cuda_device):
    inp = synth.ssd_inputs(1, 700, 3, 64, 64, 1, seed=(41,), h0=True)
    dy, dhf = _cot(1, 700, 3, 64, 64, (41,))
    a = gpu_ssd_bwd(inp, dy, dhf, cuda_device, DT)
    b = gpu_ssd_bwd(inp, dy, dhf, cuda_device, DT)
    for k in GRADS:
        assert np.array_equal(a[k], b[k]), k


def test_ssd_bwd_mamba2_workload_row(cuda_device):
    """The Mamba-2 layer shape (8 x 4096, 24 heads x 64, N = 128, one group) in the
    benchmark's launch configuration; batch row 0 checked against the oracle on all
    its heads (dx, ddt, dh0 per head, and dB, dC, which sum over the heads)."""
    inp = synth.workload_inputs("ssd_mamba2")
    d = inp.dims
    dy, dhf = _cot(d["batch"], d["L"], d["nheads"], d["headdim"], d["d_state"], (7,))
    g = gpu_ssd_bwd(inp, dy, dhf, cuda_device, DT)
    H = d["nheads"]
    units = np.stack([np.zeros(H, np.int64), np.arange(H)], 1)
    o = oracle.ssd_bwd(**inp.arrays, dy=dy, dh_final=dhf, ngroups=d["ngroups"], flags=DT, units=units)
    e = dict(dx=synth.max_rel_err(g["dx"][0].transpose(1, 0, 2), o["dx"]),
             ddt=synth.max_rel_err(g["ddt"][0].T, o["ddt"]),
             dh0=synth.max_rel_err(g["dh0"][0], o["dh0"]),
             dB=synth.max_rel_err(g["dB"][0, :, 0], o["dB"].sum(0)),
             dC=synth.max_rel_err(g["dC"][0, :, 0], o["dC"].sum(0)))
    report("ssd_bwd mamba2 row 0", **e)
    bad = {k: v for k, v in e.items() if not v <= TOL_BWD}
    assert not bad, bad


EPS32 = 2.0 ** -24


def _suffix_scale(inp, dy, dhf, flags, ou):
    """Per (head, step): the scale of the rounding that the decay gradient da_t carries.

    da_t = dL/da_t is the sum over t' >= t of the per-step scalars dL/dcs_t' (plus the
    final state's <dh_final, h_final> at the last step), each a contraction of the states
    with C_t' and x_t'.  Summed in fp32 pieces, da_t is accurate to some units of rounding
    of the absolute terms of that suffix, not of da_t itself: where a step's decay all but
    erases the state, da_t is ~0 while the suffix holds terms of size 1e2 to 1e4.  The
    absolute terms are read off the oracle's own per-head outputs: |C_t| . |dC_t| (the
    dy_t S_t contraction) and |x_t| . |dx_t - D dy_t| (sigma_t x_t . G_t B_t).
    """
    ar = inp.arrays
    H = ar["x"].shape[2]
    _, hf = oracle.ssd_fwd(**ar, ngroups=1, flags=flags)
    suf = []
    for h in range(H):
        mag = (np.abs(ar["C"][0, :, 0]).astype(np.float64) * np.abs(ou["dC"][h])).sum(1) + \
              (np.abs(ar["x"][0, :, h]).astype(np.float64) *
               np.abs(ou["dx"][h] - ar["D"][h] * dy[0, :, h])).sum(1)
        suf.append(np.cumsum(mag[::-1])[::-1] + np.abs(hf[0, h] * dhf[0, h]).sum())
    return np.stack(suf, 1)                                  # (L, H)


@pytest.mark.parametrize("flags", [DT, ZOH])
def test_ssd_bwd_extreme_dt(cuda_device, flags):
    """delta ~ 1e-11 next to delta ~ 25 (softplus' of 1e-11 and 1, decays of e^{-25 |A|}),
    over two segments.  dx, dB, dC, dD, ddt_bias and dh0 meet the usual bar.  ddt and
    dA_log go through da_t, whose fp32 suffix sum is accurate to a rounding unit of its
    absolute terms (see _suffix_scale): their bar adds EPS32 times that scale, carried
    through ddt_t = sigmoid(dt_t + bias) (da_t A + ...) and dA_log = A sum_t delta_t da_t + ...
    (one unit of rounding per absolute suffix, against the worst case of the contraction
    length times that; the GPU stays within a tenth of it on these inputs)."""
    inp = synth.ssd_inputs(1, 700, 2, 64, 64, 1, seed=(13,), h0=True, D="normal")
    ar = inp.arrays
    dt = ar["dt"]
    dt[:, ::3] = -25.0
    dt[:, 1::7] = 25.0
    dy, dhf = _cot(1, 700, 2, 64, 64, (13,))
    g = gpu_ssd_bwd(inp, dy, dhf, cuda_device, flags)
    o = oracle.ssd_bwd(**ar, dy=dy, dh_final=dhf, ngroups=1, flags=flags)
    e = {k: synth.max_rel_err(g[k], o[k]) for k in GRADS}
    report(f"ssd_bwd extreme dt flags={flags}", **e)
    for k in GRADS:
        assert np.isfinite(g[k]).all(), k
    bad = {k: v for k, v in e.items() if k not in ("ddt", "dA_log") and not v <= TOL_BWD}
    assert not bad, bad
    ou = oracle.ssd_bwd(**ar, dy=dy, dh_final=dhf, ngroups=1, flags=flags,
                        units=np.array([[0, 0], [0, 1]], np.int64))
    suf = _suffix_scale(inp, dy, dhf, flags, ou)
    A = -np.exp(ar["A_log"].astype(np.float64))
    z = dt[0].astype(np.float64) + ar["dt_bias"]
    delta = np.logaddexp(0.0, z)
    sg = 1.0 / (1.0 + np.exp(-z))
    rms = np.sqrt(np.mean(o["ddt"] ** 2))
    bar = TOL_BWD * (np.abs(o["ddt"][0]) + 0.01 * rms) + EPS32 * sg * np.abs(A) * suf
    err = np.abs(g["ddt"][0].astype(np.float64) - o["ddt"][0])
    assert (err <= bar).all(), f"ddt: worst err/bar {np.max(err / bar):.3f}"
    bar_a = TOL_BWD * np.abs(o["dA_log"]) + EPS32 * np.abs(A) * (delta * suf).sum(0)
    err_a = np.abs(g["dA_log"].astype(np.float64) - o["dA_log"])
    assert (err_a <= bar_a).all(), f"dA_log: err {err_a}, bar {bar_a}"
    report(f"ssd_bwd extreme dt flags={flags} (err/bar)", ddt=float(np.max(err / bar)),
           dA_log=float(np.max(err_a / bar_a)))
