"""GPU parity of ssd_trap_chunk_scan_bwd (gradients of the Mamba-3 trapezoidal SSD: the SSD
backward of the shifted state, the chunk diagonal's gamma correction and the chain to dt, a,
trap) against the fp64 reverse-time oracle, at the backward's bar (fp32 sums, TOL_BWD)."""
import numpy as np
import pytest

import oracle
import synth
from helpers import TOL_BWD, lib, report, sample_units

pytestmark = pytest.mark.gpu

KEYS = ("dx", "dk", "dq", "ddt", "da", "dtrap", "dh0", "dx_prev", "dk_prev", "dD")


def _cot(batch, L, H, P, N, seed, dhf=True):
    rng = np.random.default_rng([9, *seed])
    dy = rng.standard_normal((batch, L, H, P), dtype=np.float32)
    dh = rng.standard_normal((batch, H, P, N), dtype=np.float32) if dhf else None
    return dy, dh


def _gpu(inp, dy, dhf, device):
    import torch
    t = inp.torch(device)
    g = lib().ssd_trap_chunk_scan_bwd(t["x"], t["k"], t["q"], t["dt"], t["a"], t["trap"], t["D"], t["h0"],
                                      t["k_prev"], t["x_prev"], torch.from_numpy(dy).to(device),
                                      None if dhf is None else torch.from_numpy(dhf).to(device))
    torch.cuda.synchronize()
    return {k: (None if v is None else v.cpu().numpy()) for k, v in g.items()}


CASES = [  # batch, L, H, P, N, h0, carried pair, dh_final
    (2, 300, 2, 64, 128, True, True, True),
    (1, 130, 3, 32, 64, False, True, False),
    (2, 100, 2, 128, 32, True, False, True),
    (1, 1100, 2, 64, 128, True, True, True),      # several segments
    (1, 2000, 1, 64, 64, False, False, True),
    (1, 1, 2, 64, 128, True, True, True),         # one step
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b{}L{}H{}P{}N{}h{}p{}f{}".format(*[int(v) if isinstance(v, bool) else v for v in c]))
def test_trap_bwd_shapes(cuda_device, case):
    batch, L, H, P, N, h0, prev, dhf = case
    inp = synth.trap_inputs(batch, L, H, P, N, seed=(500 + L,), h0=h0, prev=prev)
    dy, dh = _cot(batch, L, H, P, N, (L,), dhf)
    g = _gpu(inp, dy, dh, cuda_device)
    go = oracle.trap_bwd(**inp.arrays, dy=dy, dh_final=dh)
    errs = {}
    for k in KEYS:
        if g.get(k) is None:
            continue
        errs[k] = synth.max_rel_err(g[k], go[k])
    report(f"trap bwd {case}", **errs)
    for k, e in errs.items():
        assert np.isfinite(g[k]).all(), k
        assert e <= TOL_BWD, (k, e)


def test_trap_bwd_bitwise_deterministic(cuda_device):
    inp = synth.trap_inputs(2, 700, 2, 64, 128, seed=(77,), h0=True, prev=True)
    dy, dh = _cot(2, 700, 2, 64, 128, (77,))
    a = _gpu(inp, dy, dh, cuda_device)
    b = _gpu(inp, dy, dh, cuda_device)
    for k in KEYS:
        if a.get(k) is not None:
            assert np.array_equal(a[k], b[k]), k


def test_trap_bwd_mamba3_workload_sampled(cuda_device):
    """Full trapezoidal workload (4 x 8192, 32 heads x 64, N 128), 2 sampled (b, h) heads over
    the whole sequence against the oracle."""
    w = synth.WORKLOADS["trap_mamba3"]
    inp = synth.workload_inputs("trap_mamba3")
    dy, dh = _cot(w["batch"], w["L"], w["nheads"], w["headdim"], w["d_state"], (0,))
    g = _gpu(inp, dy, dh, cuda_device)
    units = sample_units(np.random.default_rng(11), w["batch"], w["nheads"], 2)
    go = oracle.trap_bwd(**inp.arrays, dy=dy, dh_final=dh, units=units)
    errs = {}
    for k, sl in (("dx", lambda v, b, h: v[b, :, h]), ("dk", lambda v, b, h: v[b, :, h]),
                  ("dq", lambda v, b, h: v[b, :, h]), ("ddt", lambda v, b, h: v[b, :, h]),
                  ("da", lambda v, b, h: v[b, :, h]), ("dtrap", lambda v, b, h: v[b, :, h]),
                  ("dh0", lambda v, b, h: v[b, h])):
        gg = np.stack([sl(g[k], b, h) for b, h in units])
        errs[k] = synth.max_rel_err(gg, go[k])
    report("trap_mamba3 bwd sampled", **errs)
    for k, e in errs.items():
        assert e <= TOL_BWD, (k, e)
