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
