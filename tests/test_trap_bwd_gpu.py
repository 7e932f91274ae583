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


EPS32 = 2.0 ** -24


def test_trap_bwd_extreme_dt(cuda_device):
    """dt of 1e-11 next to 25 (decays of e^{25 a}, a in [-16, -1]) over two segments.  All
    outputs but da and ddt meet the usual bar.  da_t = dt_t s_t and ddt_t = a_t s_t + ...
    go through s_t, the gradient of the log decay at t: a suffix sum over t' >= t of
    per-step contractions, accurate in fp32 to a rounding unit of its absolute terms, not
    of s_t itself (where a step erases the state s_t is ~0 while the suffix holds terms of
    1e5 and more).  Their bar adds EPS32 times that absolute suffix, read off the oracle's
    outputs: |q_t| . |dq_t| (the dy_t h_t contraction) and |x_t| . |dx_t - D dy_t| (the
    injected input against the state's cotangent), plus |h_final dh_final|."""
    inp = synth.trap_inputs(1, 700, 2, 64, 128, seed=(36,), h0=True, prev=True)
    ar = inp.arrays
    dt = ar["dt"]
    dt[:, ::3] = 1e-11
    dt[:, 1::7] = 25.0
    dy, dh = _cot(1, 700, 2, 64, 128, (36,))
    g = _gpu(inp, dy, dh, cuda_device)
    o = oracle.trap_bwd(**ar, dy=dy, dh_final=dh)
    errs = {k: synth.max_rel_err(g[k], o[k]) for k in KEYS if g.get(k) is not None}
    report("trap bwd extreme dt", **errs)
    for k, e in errs.items():
        assert np.isfinite(g[k]).all(), k
        if k not in ("da", "ddt"):
            assert e <= TOL_BWD, (k, e)
    _, hf = oracle.trap_fwd(**ar)
    suf = []
    for h in range(ar["x"].shape[2]):
        mag = (np.abs(ar["q"][0, :, h]).astype(np.float64) * np.abs(o["dq"][0, :, h])).sum(1) + \
              (np.abs(ar["x"][0, :, h]).astype(np.float64) *
               np.abs(o["dx"][0, :, h] - ar["D"][h] * dy[0, :, h])).sum(1)
        suf.append(np.cumsum(mag[::-1])[::-1] + np.abs(hf[0, h] * dh[0, h]).sum())
    suf = np.stack(suf, 1)                                   # (L, H)
    ratios = {}
    for k, scale in (("da", dt[0].astype(np.float64)), ("ddt", np.abs(ar["a"][0].astype(np.float64)))):
        rms = np.sqrt(np.mean(o[k][0] ** 2))
        bar = TOL_BWD * (np.abs(o[k][0]) + 0.01 * rms) + EPS32 * scale * suf
        err = np.abs(g[k][0].astype(np.float64) - o[k][0])
        ratios[k] = float(np.max(err / bar))
        assert (err <= bar).all(), f"{k}: worst err/bar {ratios[k]:.3f}"
    report("trap bwd extreme dt (err/bar)", **ratios)
