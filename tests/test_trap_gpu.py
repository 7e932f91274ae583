"""GPU parity of ssd_trap_chunk_scan_fwd (Mamba-3 trapezoidal SSD; bf16 x, k, q, fp32
state) against the fp64 sequential oracle of the same recurrence."""
import numpy as np
import pytest

import oracle
import synth
from helpers import TOL_BF16, gpu_trap, lib, report, sample_units

pytestmark = pytest.mark.gpu


def _check(name, inp, device, Q=64, tol=TOL_BF16):
    y, hf = gpu_trap(inp, device, Q)
    yo, ho = oracle.trap_fwd(**inp.arrays)
    ey, eh = synth.max_rel_err(y, yo), synth.max_rel_err(hf, ho)
    report(name, y=ey, h_final=eh)
    assert np.isfinite(y).all() and np.isfinite(hf).all()
    assert ey <= tol and eh <= tol
    return y, hf


CASES = [  # batch, L, H, P, N, Q, h0, carried previous input
    (2, 300, 4, 64, 128, 64, True, True),
    (1, 1, 2, 64, 128, 64, True, True),          # one step: only gamma and the carried input
    (1, 2, 2, 32, 64, 64, False, True),
    (1, 65, 2, 32, 64, 128, False, True),
    (1, 200, 3, 128, 64, 256, True, False),
    (2, 130, 2, 64, 256, 64, False, False),
    (1, 100, 2, 64, 96, 64, True, True),          # state size not a power of two
    # long enough to be cut into segments (state kernel + pass + scan), last segment partial
    (1, 2000, 2, 64, 128, 64, True, True),
    (1, 1500, 1, 32, 64, 64, False, True),
    (1, 777, 3, 128, 128, 128, True, True),
    (1, 1100, 2, 64, 160, 64, False, False),
    (1, 900, 2, 64, 256, 64, True, True),        # the largest state size, with segments
]


@pytest.mark.parametrize("case", CASES,
                         ids=lambda c: f"b{c[0]}L{c[1]}H{c[2]}P{c[3]}N{c[4]}Q{c[5]}h{int(c[6])}p{int(c[7])}")
def test_trap_shapes(cuda_device, case):
    batch, L, H, P, N, Q, h0, prev = case
    inp = synth.trap_inputs(batch, L, H, P, N, seed=(300 + L,), h0=h0, prev=prev)
    _check(f"trap {case}", inp, cuda_device, Q)


@pytest.mark.parametrize("tr", [0.0, 1.0])
def test_trap_constant_blend(cuda_device, tr):
    """trap = 1: the plain SSD scan with input scale dt (beta = 0); trap = 0: only the
    previous step's input enters (gamma = 0, the diagonal of every chunk is empty)."""
    inp = synth.trap_inputs(2, 700, 2, 64, 128, seed=(31, int(tr)), h0=True, prev=True, trap=tr)
    _check(f"trap={tr}", inp, cuda_device)


def test_trap_carry_across_calls(cuda_device):
    """Two calls that carry (h_final, last x, last k) equal one call over the whole sequence."""
    import torch
    inp = synth.trap_inputs(1, 1200, 3, 64, 128, seed=(33,), h0=True, prev=True)
    t = inp.torch(cuda_device)
    m = lib()
    y_all, hf_all = m.ssd_trap_chunk_scan_fwd(t["x"], t["k"], t["q"], t["dt"], t["a"], t["trap"],
                                              t["D"], t["h0"], t["k_prev"], t["x_prev"],
                                              return_final=True)
    cut = 517
    s1 = {n: t[n][:, :cut].clone() for n in ("x", "k", "q", "dt", "a", "trap")}
    s2 = {n: t[n][:, cut:].clone() for n in ("x", "k", "q", "dt", "a", "trap")}
    y1, hf1 = m.ssd_trap_chunk_scan_fwd(s1["x"], s1["k"], s1["q"], s1["dt"], s1["a"], s1["trap"],
                                        t["D"], t["h0"], t["k_prev"], t["x_prev"], return_final=True)
    kp, xp = s1["k"][:, -1].clone(), s1["x"][:, -1].clone()
    y2, hf2 = m.ssd_trap_chunk_scan_fwd(s2["x"], s2["k"], s2["q"], s2["dt"], s2["a"], s2["trap"],
                                        t["D"], hf1, kp, xp, return_final=True)
    torch.cuda.synchronize()
    y_split = torch.cat([y1, y2], dim=1).cpu().numpy()
    ey = synth.max_rel_err(y_split, y_all.cpu().numpy())
    eh = synth.max_rel_err(hf2.cpu().numpy(), hf_all.cpu().numpy())
    report("trap carry", y=ey, h_final=eh)
    assert ey <= TOL_BF16 and eh <= TOL_BF16
    yo, ho = oracle.trap_fwd(**inp.arrays)
    assert synth.max_rel_err(y_split, yo) <= TOL_BF16
    assert synth.max_rel_err(hf2.cpu().numpy(), ho) <= TOL_BF16


def test_trap_chunk_len_invariance(cuda_device):
    inp = synth.trap_inputs(1, 700, 2, 64, 128, seed=(34,), h0=True, prev=True)
    ys = [gpu_trap(inp, cuda_device, Q) for Q in (64, 128, 256)]
    for y, hf in ys[1:]:
        assert np.array_equal(y, ys[0][0]) and np.array_equal(hf, ys[0][1])


def test_trap_bitwise_deterministic(cuda_device):
    inp = synth.trap_inputs(2, 1000, 4, 64, 128, seed=(35,), h0=True, prev=True)
    a = gpu_trap(inp, cuda_device)
    b = gpu_trap(inp, cuda_device)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_trap_mamba3_workload_sampled(cuda_device):
    """Full Mamba-3 workload shape (4 x 8192, 32 heads x 64, N 128); 4 sampled (b, h)
    heads checked over the whole sequence against the oracle."""
    name = "trap_mamba3"
    w = synth.WORKLOADS[name]
    inp = synth.workload_inputs(name)
    y, hf = gpu_trap(inp, cuda_device, w["chunk_len"])
    rng = np.random.default_rng(3)
    units = sample_units(rng, w["batch"], w["nheads"], 4)
    yo, ho = oracle.trap_fwd(**inp.arrays, units=units)
    yg = np.stack([y[b, :, h, :] for b, h in units])
    hg = np.stack([hf[b, h] for b, h in units])
    ey, eh = synth.max_rel_err(yg, yo), synth.max_rel_err(hg, ho)
    report(f"{name} sampled", y=ey, h_final=eh)
    assert np.isfinite(y).all()
    assert ey <= TOL_BF16 and eh <= TOL_BF16


@pytest.mark.parametrize("L", [300, 1100])
def test_trap_extreme_dt(cuda_device, L):
    """dt of 1e-11 next to dt of 25 (decays e^{-25 |a|}, inputs scaled by 25), within one
    segment and across segment boundaries."""
    inp = synth.trap_inputs(1, L, 2, 64, 128, seed=(35, L), h0=True, prev=True)
    dt = inp.arrays["dt"]
    dt[:, ::3] = 1e-11
    dt[:, 1::7] = 25.0
    _check(f"trap extreme dt L={L}", inp, cuda_device, 64)
