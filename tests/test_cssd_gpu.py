"""GPU parity of ssd_cplx_chunk_scan_fwd (fp32) against the fp64 oracle."""
import numpy as np
import pytest

import oracle
import synth
from helpers import TOL_F32, gpu_cssd, report

pytestmark = pytest.mark.gpu

STABLE, DOC, CODE, CONJ = oracle.CPLX_STABLE, oracle.CPLX_DOC, oracle.CPLX_CODE, oracle.CPLX_CONJ_C
ZOH, DT, ONE = oracle.BBAR_ZOH, oracle.BBAR_DT, oracle.BBAR_ONE

CASES = [  # batch, L, H, P, Nc, G, Q, flags, h0
    (2, 150, 4, 32, 8, 2, 32, STABLE | ZOH, True),
    (1, 200, 2, 64, 32, 1, 64, STABLE | ZOH, True),
    (1, 260, 2, 64, 16, 2, 128, STABLE | DT, False),
    (1, 100, 2, 32, 8, 1, 64, STABLE | ONE, True),
    (1, 120, 2, 32, 8, 1, 64, DOC | ZOH, True),
    (1, 120, 2, 32, 8, 1, 64, CODE, True),
    (1, 90, 2, 64, 32, 1, 64, STABLE | ZOH | CONJ, True),
    (1, 1, 2, 32, 8, 1, 64, STABLE | ZOH, True),
    (3, 7, 2, 32, 8, 1, 64, STABLE | ZOH, True),  # batch rows shorter than a chunk, back to back
    (1, 64, 2, 128, 8, 1, 64, STABLE | ZOH, False),
    # long enough to be cut into segments (state kernel + pass + scan), last segment partial
    (1, 1000, 2, 64, 24, 1, 64, STABLE | ZOH, True),
    (1, 800, 2, 64, 32, 1, 64, STABLE | ZOH | CONJ, True),
    (2, 700, 3, 128, 64, 3, 128, STABLE | DT, False),
    (1, 513, 1, 32, 40, 1, 32, STABLE | ONE, True),
    # heads per group beyond one prep block of 8: a full and a half block (12), one wave
    # with a single valid half (5 per group, 2 groups)
    (1, 300, 12, 32, 8, 1, 32, STABLE | ZOH, True),
    (2, 333, 10, 32, 16, 2, 64, STABLE | ZOH | CONJ, False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"b{c[0]}L{c[1]}H{c[2]}P{c[3]}N{c[4]}G{c[5]}Q{c[6]}f{c[7]}")
def test_cssd_shapes(cuda_device, case):
    batch, L, H, P, Nc, G, Q, flags, h0 = case
    inp = synth.cssd_inputs(batch, L, H, P, Nc, G, seed=(300 + L,), h0=h0)
    y, hf = gpu_cssd(inp, cuda_device, flags, Q)
    yo, ho = oracle.cssd_fwd(**inp.arrays, ngroups=G, flags=flags)
    ey, eh = synth.max_rel_err(y, yo), synth.max_rel_err(hf, ho)
    report(f"cssd {case}", y=ey, h_final=eh)
    assert np.isfinite(y).all() and np.isfinite(hf).all()
    assert ey <= TOL_F32 and eh <= TOL_F32


def test_cssd_workload_all_heads(cuda_device):
    """Full complex workload (4 x 8192, 32 heads x 64, 32 complex states): every one of
    the 128 (b, h) heads checked against the oracle over the whole sequence."""
    inp = synth.workload_inputs("cssd_mamba3")
    w = synth.WORKLOADS["cssd_mamba3"]
    y, hf = gpu_cssd(inp, cuda_device, STABLE | ZOH, w["chunk_len"])
    yo, ho = oracle.cssd_fwd(**inp.arrays, ngroups=w["ngroups"])
    ey, eh = synth.max_rel_err(y, yo), synth.max_rel_err(hf, ho)
    # worst head, for the record
    per_head = [max(synth.max_rel_err(y[b, :, h], yo[b, :, h]), synth.max_rel_err(hf[b, h], ho[b, h]))
                for b in range(w["batch"]) for h in range(w["nheads"])]
    report("cssd_mamba3 all heads", y=ey, h_final=eh, worst_head=max(per_head), margin=TOL_F32 / max(ey, eh))
    assert ey <= TOL_F32 and eh <= TOL_F32


def _one_head(inp, h, G, H):
    """The inputs of head h alone: one head in one group (the group's B and C)."""
    import copy
    g = h * G // H
    a = dict(inp.arrays)
    for k in ("x", "dt"):
        a[k] = np.ascontiguousarray(a[k][:, :, h:h + 1])
    for k in ("A_log", "dt_bias", "D"):
        a[k] = np.ascontiguousarray(a[k][h:h + 1])
    for k in ("B", "C"):
        a[k] = np.ascontiguousarray(a[k][:, :, g:g + 1])
    if a["h0"] is not None:
        a["h0"] = np.ascontiguousarray(a["h0"][:, h:h + 1])
    one = copy.copy(inp)
    one.arrays = a
    return one


@pytest.mark.parametrize("case", [(1, 1100, 9, 64, 32, 1, 64, True), (2, 333, 10, 32, 16, 2, 64, False)],
                         ids=lambda c: f"b{c[0]}L{c[1]}H{c[2]}P{c[3]}N{c[4]}G{c[5]}")
def test_head_grouping_changes_no_value(cuda_device, case):
    """The prep pass shares C.B^T among up to 8 heads of a group and forms two heads' scalars per
    wave: every head's outputs and final state must be bitwise those of the head run alone
    (9 heads: a ninth head alone in its block, with segments; 10 heads in 2 groups: a wave with
    one valid half)."""
    batch, L, H, P, Nc, G, Q, h0 = case
    inp = synth.cssd_inputs(batch, L, H, P, Nc, G, seed=(310 + L,), h0=h0)
    y, hf = gpu_cssd(inp, cuda_device, STABLE | ZOH, Q)
    for h in range(H):
        y1, h1 = gpu_cssd(_one_head(inp, h, G, H), cuda_device, STABLE | ZOH, Q)
        assert np.array_equal(y1[:, :, 0], y[:, :, h]), f"head {h}: y differs from the head alone"
        assert np.array_equal(h1[:, 0], hf[:, h]), f"head {h}: h_final differs from the head alone"


@pytest.mark.parametrize("L", [300, 1100])
def test_cssd_extreme_dt(cuda_device, L):
    """Steps with delta ~ 1e-11 next to steps with delta ~ 25: per-step decays down to
    e^{-68} and rotations of tens of radians, within one segment and across segments."""
    inp = synth.cssd_inputs(1, L, 2, 64, 32, 1, seed=(37, L), h0=True)
    dt = inp.arrays["dt"]
    dt[:, ::3] = -25.0
    dt[:, 1::7] = 25.0
    y, hf = gpu_cssd(inp, cuda_device, STABLE | ZOH, 64)
    yo, ho = oracle.cssd_fwd(**inp.arrays, ngroups=1, flags=STABLE | ZOH)
    ey, eh = synth.max_rel_err(y, yo), synth.max_rel_err(hf, ho)
    report(f"cssd extreme dt L={L}", y=ey, h_final=eh)
    assert np.isfinite(y).all() and np.isfinite(hf).all()
    assert ey <= TOL_F32 and eh <= TOL_F32
