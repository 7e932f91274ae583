"""GPU parity of the segmented S6 scan: ssm_s6_scan_fwd with the workspace the library
asks for, on shapes whose few channel blocks would leave the chip idle, so time is cut
into segments joined by the associative carry.  Against the fp64 oracle element by element
(small shapes) or on sampled channels (long context), and against the sequential walk."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import TOL_BF16, TOL_F32, lib, report

pytestmark = pytest.mark.gpu

ZOH, DT, ONE = oracle.BBAR_ZOH, oracle.BBAR_DT, oracle.BBAR_ONE


def _run(inp, device, flags, workspace="auto"):
    t = inp.torch(device)
    y, hf = lib().ssm_s6_scan_fwd(t["u"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"], t["D"],
                                  t["h0"], flags=flags, return_final=True, workspace=workspace)
    torch.cuda.synchronize()
    return y.cpu().numpy(), hf.cpu().numpy()


CASES = [  # batch, L, d_inner, N, flags, dtype, h0, A_log, seed
    (1, 4096, 64, 16, ZOH, "f32", True, "index", (70, 4096, 64)),      # 4 blocks: 8 segments of 512
    (2, 3000, 40, 16, ZOH, "f32", True, "uniform", (70, 3000, 40)),    # ragged last segment and block
    (1, 1100, 16, 16, DT, "f32", False, "uniform", (70, 1100, 16)),    # 2 segments
    (1, 2600, 100, 4, ZOH, "f32", True, "index", (70, 2600, 100)),     # 64 channels per block
    (2, 2048, 24, 1, ONE, "f32", True, "uniform", (70, 2048, 24)),     # one state
    (1, 5000, 33, 8, ZOH, "bf16", True, "index", (70, 5000, 33)),
    # slow states (|A| = e^-1.5, e^-1): a segment's decay is 2e-2 and 4e-3, so the carried
    # state is a visible part of the next segment's outputs.  (Slower ones, with memories of
    # several hundred steps, exceed the fp32 bar even for a recurrence that rounds every
    # operation once: 1.1e-4 at |A| = e^-2.5, L = 1500.)
    (3, 1100, 20, 16, ZOH, "f32", True, -1.5, (74, 0)),
    (1, 2048, 32, 16, ZOH, "f32", True, -1.0, (74, 0)),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"b{c[0]}L{c[1]}D{c[2]}N{c[3]}f{c[4]}{c[5]}A{c[7]}")
def test_seg_shapes(cuda_device, case):
    batch, L, Dm, N, flags, dtype, h0, a_log, seed = case
    assert lib().ssm_s6_scan_fwd_workspace_size(batch, L, Dm, N) > 0      # the segmented path
    inp = synth.s6_inputs(batch, L, Dm, N, seed=seed, dtype=dtype, h0=h0, a_log=a_log)
    y, hf = _run(inp, cuda_device, flags)
    yo, ho = oracle.s6_fwd(**inp.arrays, flags=flags)
    ey, eh = synth.max_rel_err(y, yo), synth.max_rel_err(hf, ho)
    yw, hw = _run(inp, cuda_device, flags, workspace=None)     # the sequential walk
    report(f"s6 segmented {case}", y=ey, h_final=eh, vs_walk=max(synth.max_rel_err(y, yw), synth.max_rel_err(hf, hw)))
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    assert np.isfinite(y).all() and np.isfinite(hf).all()
    assert ey <= tol and eh <= tol


def test_seg_bitwise_deterministic(cuda_device):
    inp = synth.s6_inputs(1, 4096, 48, 16, seed=(71,), h0=True)
    a = _run(inp, cuda_device, ZOH)
    b = _run(inp, cuda_device, ZOH)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_seg_in_place_state(cuda_device):
    """h0 and h_final may be one buffer: the carry reads h0 before the last segment writes."""
    inp = synth.s6_inputs(1, 3000, 32, 16, seed=(72,), h0=True)
    t = inp.torch(cuda_device)
    m = lib()
    y_ref, h_ref = m.ssm_s6_scan_fwd(t["u"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"], t["D"],
                                     t["h0"], return_final=True)
    state = t["h0"].clone()
    y = m.ssm_s6_scan_fwd(t["u"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"], t["D"], state,
                          h_final=state)[0]
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref) and torch.equal(state, h_ref)


def _spread(rng, batch, d_inner, per_row):
    return np.array([(b, int(blk) * 16 + i % 16) for b in range(batch)
                     for i, blk in enumerate(rng.choice(d_inner // 16, size=per_row, replace=False))])


@pytest.mark.parametrize("batch,L", [(1, 32768), (2, 8192)])
def test_seg_long_context_sampled(cuda_device, batch, L):
    """A Mamba-1 layer's scan at long context (d_inner 1536, N 16, the Mamba-1 input recipe):
    96 channels of every batch row over the whole sequence, against the oracle."""
    Dm, N = 1536, 16
    assert lib().ssm_s6_scan_fwd_workspace_size(batch, L, Dm, N) > 0
    inp = synth.s6_inputs(batch, L, Dm, N, seed=(73, L), h0=True)
    y, hf = _run(inp, cuda_device, ZOH)
    units = _spread(np.random.default_rng(L), batch, Dm, 96)
    yo, ho = oracle.s6_fwd(**inp.arrays, units=units)
    yg = np.stack([y[b, :, d] for b, d in units])
    hg = np.stack([hf[b, d] for b, d in units])
    ey, eh = synth.max_rel_err(yg, yo), synth.max_rel_err(hg, ho)
    report(f"s6 segmented b{batch} L{L} sampled ({len(units)} channels)", y=ey, h_final=eh)
    assert np.isfinite(y).all()
    assert ey <= TOL_F32 and eh <= TOL_F32


def test_seg_extreme_dt(cuda_device):
    """delta ~ 1e-11 next to delta ~ 25 across the segments: the carried decay products
    underflow to zero within a segment, and the states cross segment boundaries intact."""
    assert lib().ssm_s6_scan_fwd_workspace_size(1, 4096, 64, 16) > 0
    inp = synth.s6_inputs(1, 4096, 64, 16, seed=(75,), h0=True)
    dt = inp.arrays["dt"]
    dt[:, ::3] = -25.0
    dt[:, 1::7] = 25.0
    y, hf = _run(inp, cuda_device, ZOH)
    yo, ho = oracle.s6_fwd(**inp.arrays, flags=ZOH)
    ey, eh = synth.max_rel_err(y, yo), synth.max_rel_err(hf, ho)
    report("s6 segmented extreme dt", y=ey, h_final=eh)
    assert np.isfinite(y).all() and np.isfinite(hf).all()
    assert ey <= TOL_F32 and eh <= TOL_F32
