"""GPU parity of ssd_chunk_scan_fwd (bf16 inputs, fp32 state) against the fp64 oracle."""
import numpy as np
import pytest

import oracle
import synth
from helpers import TOL_BF16, gpu_ssd, report, sample_units

pytestmark = pytest.mark.gpu

ZOH, DT, ONE = oracle.BBAR_ZOH, oracle.BBAR_DT, oracle.BBAR_ONE


def _check(name, inp, device, flags, Q, tol=TOL_BF16):
    y, hf = gpu_ssd(inp, device, flags, Q)
    yo, ho = oracle.ssd_fwd(**inp.arrays, ngroups=inp.dims["ngroups"], flags=flags)
    ey, eh = synth.max_rel_err(y, yo), synth.max_rel_err(hf, ho)
    report(name, y=ey, h_final=eh)
    assert np.isfinite(y).all() and np.isfinite(hf).all()
    assert ey <= tol and eh <= tol
    return y


CASES = [  # batch, L, H, P, N, G, Q, flags, h0
    (2, 300, 4, 64, 64, 2, 64, DT, True),
    (2, 300, 4, 64, 128, 2, 128, DT, True),
    (1, 600, 2, 64, 128, 1, 256, DT, True),
    (1, 300, 3, 64, 128, 3, 256, ZOH, False),
    (1, 200, 2, 32, 32, 1, 64, ONE, True),
    (1, 130, 2, 128, 64, 2, 128, DT, True),
    (1, 100, 2, 64, 256, 1, 64, DT, True),
    (1, 1, 2, 64, 128, 1, 256, DT, True),
    (3, 5, 2, 64, 128, 1, 64, DT, True),          # batch rows shorter than a chunk, back to back
    (1, 65, 2, 64, 128, 1, 64, ZOH, True),
    (2, 513, 4, 64, 128, 1, 256, DT, False),
    # long enough to be cut into segments (state kernel + pass + scan), last segment partial
    (1, 2000, 2, 64, 128, 1, 256, DT, True),
    (1, 1500, 1, 32, 64, 1, 64, ZOH, True),
    (1, 777, 3, 128, 128, 3, 128, DT, True),
    (1, 1100, 2, 64, 96, 2, 64, ONE, False),
    (1, 1100, 2, 64, 256, 1, 256, DT, True),      # the largest state size, with segments
    (1, 900, 4, 32, 64, 2, 64, DT, True),         # segment states of head pairs, 2 waves per head
    (1, 700, 4, 64, 96, 2, 128, ZOH, True),       # head pairs with a state narrower than its tile
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"b{c[0]}L{c[1]}H{c[2]}P{c[3]}N{c[4]}G{c[5]}Q{c[6]}f{c[7]}")
def test_ssd_shapes(cuda_device, case):
    batch, L, H, P, N, G, Q, flags, h0 = case
    inp = synth.ssd_inputs(batch, L, H, P, N, G, seed=(200 + L,), h0=h0, D="normal")
    _check(f"ssd {case}", inp, cuda_device, flags, Q)


def test_ssd_chunk_len_invariance(cuda_device):
    inp = synth.ssd_inputs(1, 700, 2, 64, 128, 1, seed=(5,), h0=True)
    ys = [gpu_ssd(inp, cuda_device, DT, Q) for Q in (64, 128, 256)]
    for y, hf in ys[1:]:
        assert synth.max_rel_err(y, ys[0][0]) < TOL_BF16
        assert synth.max_rel_err(hf, ys[0][1]) < TOL_BF16


def test_ssd_bitwise_deterministic(cuda_device):
    inp = synth.ssd_inputs(2, 1000, 4, 64, 128, 2, seed=(6,), h0=True)
    a = gpu_ssd(inp, cuda_device, DT, 256)
    b = gpu_ssd(inp, cuda_device, DT, 256)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def _group_units(rng, batch, nheads, ngroups, per_group):
    """per_group heads of every group of every batch row (drawn at random in the group)."""
    hpg = nheads // ngroups
    return np.array([(b, g * hpg + int(h)) for b in range(batch) for g in range(ngroups)
                     for h in rng.choice(hpg, size=per_group, replace=False)], dtype=np.int64)


@pytest.mark.parametrize("name,per_group", [("ssd_mamba2", 3), ("ssd_long", 1)])
def test_ssd_workloads_sampled(cuda_device, name, per_group):
    """Full workload shape; sampled (b, h) heads checked over the whole sequence: the
    Mamba-2 shape 24 heads (3 of every batch row), the long shape 16 (one per group and
    batch row, so every group's B and C)."""
    inp = synth.workload_inputs(name)
    w = synth.WORKLOADS[name]
    y, hf = gpu_ssd(inp, cuda_device, DT, w["chunk_len"])
    a = inp.arrays
    units = _group_units(np.random.default_rng(1), w["batch"], w["nheads"], w["ngroups"], per_group)
    yo, ho = oracle.ssd_fwd(**a, ngroups=w["ngroups"], units=units)
    yg = np.stack([y[b, :, h, :] for b, h in units])
    hg = np.stack([hf[b, h] for b, h in units])
    ey, eh = synth.max_rel_err(yg, yo), synth.max_rel_err(hg, ho)
    report(f"{name} sampled ({len(units)} heads)", y=ey, h_final=eh, margin=TOL_BF16 / max(ey, eh))
    assert np.isfinite(y).all()
    assert ey <= TOL_BF16 and eh <= TOL_BF16


@pytest.mark.parametrize("shape", [(2, 4096, 80, 64, 128, 8, DT), (4, 4096, 64, 32, 64, 4, ZOH),
                                   (2, 4096, 80, 64, 96, 8, ZOH)],
                         ids=["b2L4096H80P64N128G8", "b4L4096H64P32N64G4", "b2L4096H80P64N96G8"])
def test_ssd_head_pairs_sampled(cuda_device, shape):
    """Shapes whose plan runs several rounds of segments, where the segment states are
    formed for two heads of a group per work group: two heads of every group and batch
    row (an even and an odd one, so both halves of a pair) over the whole sequence."""
    batch, L, H, P, N, G, flags = shape
    inp = synth.ssd_inputs(batch, L, H, P, N, G, seed=(31, L), h0=True, D="normal")
    y, hf = gpu_ssd(inp, cuda_device, flags, 256)
    hpg = H // G
    rng = np.random.default_rng(3)
    units = np.array([(b, g * hpg + int(2 * rng.integers(hpg // 2)) + o)
                      for b in range(batch) for g in range(G) for o in (0, 1)], dtype=np.int64)
    yo, ho = oracle.ssd_fwd(**inp.arrays, ngroups=G, flags=flags, units=units)
    ey = synth.max_rel_err(np.stack([y[b, :, h, :] for b, h in units]), yo)
    eh = synth.max_rel_err(np.stack([hf[b, h] for b, h in units]), ho)
    report(f"ssd head pairs {shape} ({len(units)} heads)", y=ey, h_final=eh)
    assert np.isfinite(y).all() and np.isfinite(hf).all()
    assert ey <= TOL_BF16 and eh <= TOL_BF16


def test_ssd_in_place_state(cuda_device):
    """h0 and h_final may be the same buffer (the carried state is updated in place)."""
    import torch
    from helpers import lib
    inp = synth.ssd_inputs(1, 1800, 2, 64, 128, 1, seed=(7,), h0=True)
    t = inp.torch(cuda_device)
    ref = lib().ssd_chunk_scan_fwd(t["x"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"], t["D"],
                                   t["h0"], return_final=True)
    state = t["h0"].clone()
    y = lib().ssd_chunk_scan_fwd(t["x"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"], t["D"],
                                 state, h_final=state)[0]
    torch.cuda.synchronize()
    assert torch.equal(y, ref[0]) and torch.equal(state, ref[1])


def test_ssd_carry_composition(cuda_device):
    """Scanning [0, L1) then [L1, L) from the carried state matches one scan of [0, L)."""
    import torch
    from helpers import lib
    inp = synth.ssd_inputs(1, 1600, 2, 64, 128, 1, seed=(8,), h0=True)
    t = inp.torch(cuda_device)
    whole = lib().ssd_chunk_scan_fwd(t["x"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"], t["D"],
                                     t["h0"], return_final=True)
    L1 = 700
    part = lambda a, lo, hi: a[:, lo:hi].contiguous()
    first = lib().ssd_chunk_scan_fwd(part(t["x"], 0, L1), part(t["dt"], 0, L1), t["dt_bias"], t["A_log"],
                                     part(t["B"], 0, L1), part(t["C"], 0, L1), t["D"], t["h0"],
                                     return_final=True)
    second = lib().ssd_chunk_scan_fwd(part(t["x"], L1, None), part(t["dt"], L1, None), t["dt_bias"],
                                      t["A_log"], part(t["B"], L1, None), part(t["C"], L1, None), t["D"],
                                      first[1], return_final=True)
    torch.cuda.synchronize()
    y = torch.cat([first[0], second[0]], 1).cpu().numpy()
    assert synth.max_rel_err(y, whole[0].cpu().numpy()) <= TOL_BF16
    assert synth.max_rel_err(second[1].cpu().numpy(), whole[1].cpu().numpy()) <= TOL_BF16


@pytest.mark.parametrize("flags", [DT, ZOH])
@pytest.mark.parametrize("L", [300, 1100])
def test_ssd_extreme_dt(cuda_device, flags, L):
    """Steps with delta ~ 1e-11 (no decay, no input) next to steps with delta ~ 25 (the state
    all but erased, inputs scaled by 25): cumulative decays of hundreds inside a chunk, within
    one segment (L = 300) and across segment boundaries (L = 1100)."""
    inp = synth.ssd_inputs(1, L, 3, 64, 128, 1, seed=(11, L), h0=True, D="normal")
    dt = inp.arrays["dt"]
    dt[:, ::3] = -25.0
    dt[:, 1::7] = 25.0
    _check(f"ssd extreme dt L={L} flags={flags}", inp, cuda_device, flags, 256)


@pytest.mark.parametrize("a_log", [-30.0, -3.0, 4.0])
def test_ssd_degenerate_A(cuda_device, a_log):
    """A -> 0 (no decay: the scan is a running sum), slow decay, and fast decay (|A| = e^4)."""
    inp = synth.ssd_inputs(1, 900, 2, 64, 128, 1, seed=(12,), h0=True, D="normal")
    inp.arrays["A_log"][:] = a_log
    _check(f"ssd A_log={a_log}", inp, cuda_device, ZOH, 256)
