"""GPU parity of ssd_trap_rotate_qk (Mamba-3 angle accumulation + rotation of k and q)
against the fp64 oracle, alone and followed by the trapezoidal scan."""
import numpy as np
import pytest

import oracle
import synth
from helpers import TOL_BF16, gpu_trap, lib, report, sample_units

pytestmark = pytest.mark.gpu

# one rounding of an fp32 result to bf16 moves it by at most 2^-8 of its size
# (half an ulp of 8 significant bits); fp32 angle and product errors add ~1e-6
# of the pair's norm, covered by the absolute term
RTOL_BF16_ROUND = 2.0 ** -8


def _rotate(inp, ang, st, device, **kw):
    import torch
    t = inp.torch(device)
    ta = torch.from_numpy(ang).to(device)
    ts = None if st is None else torch.from_numpy(st).to(device)
    k, q, so = lib().ssd_trap_rotate_qk(t["k"], t["q"], ta, t["dt"], ts, return_state=True, **kw)
    torch.cuda.synchronize()
    return k.float().cpu().numpy(), q.float().cpu().numpy(), so.cpu().numpy()


def _check_rot(name, g, o, scale):
    err = np.abs(g - o) - RTOL_BF16_ROUND * np.abs(o)
    worst = float(err.max() / scale)
    report(name, excess_over_rounding=worst)
    assert worst <= 2e-5, worst


CASES = [  # batch, L, H, N, n_angles, angle state
    (2, 300, 4, 128, 64, True),
    (1, 1, 2, 64, 32, True),
    (1, 777, 3, 64, 20, False),        # the tail past 2 n_angles is copied
    (2, 130, 2, 256, 128, True),
    (3, 100, 5, 96, 48, True),
    (1, 1200, 3, 128, 64, True),
    (1, 65, 1, 32, 16, False),
    # scalar path (d_state % 8 != 0 or n_angles % 4 != 0): one pair per lane
    (1, 300, 3, 10, 5, True),
    (2, 150, 2, 64, 30, True),
    (1, 90, 3, 12, 3, False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"b{c[0]}L{c[1]}H{c[2]}N{c[3]}A{c[4]}s{int(c[5])}")
def test_rotate_shapes(cuda_device, case):
    batch, L, H, N, NA, has_st = case
    inp = synth.trap_inputs(batch, L, H, 32, N, seed=(400 + L,))
    ang, st = synth.rotation_inputs(batch, L, H, NA, seed=(L,), angle_state=has_st)
    a = inp.arrays
    k, q, so = _rotate(inp, ang, st, cuda_device)
    ko, qo, sto = oracle.trap_rotate(a["k"], a["q"], ang, a["dt"], st)
    scale = float(np.abs(ko).max())
    _check_rot(f"rotate k {case}", k, ko, scale)
    _check_rot(f"rotate q {case}", q, qo, scale)
    # the pairs past 2 n_angles are the inputs bit for bit
    assert np.array_equal(k[..., 2 * NA:], a["k"][..., 2 * NA:])
    assert np.array_equal(q[..., 2 * NA:], a["q"][..., 2 * NA:])
    np.testing.assert_allclose(so, sto, rtol=1e-4, atol=1e-4)


def test_rotate_zero_angles_copy(cuda_device):
    inp = synth.trap_inputs(1, 200, 2, 32, 64, seed=(41,))
    ang = np.zeros((1, 200, 0), np.float32)
    import torch
    t = inp.torch(cuda_device)
    k, q = lib().ssd_trap_rotate_qk(t["k"], t["q"], torch.from_numpy(ang).to(cuda_device), t["dt"])
    torch.cuda.synchronize()
    assert torch.equal(k, t["k"]) and torch.equal(q, t["q"])


def test_rotate_in_place_and_state_carry(cuda_device):
    """k, q and the angle state updated in place over two calls equal one call."""
    import torch
    L, cut = 900, 333
    inp = synth.trap_inputs(2, L, 3, 32, 128, seed=(42,))
    ang, st = synth.rotation_inputs(2, L, 3, 64, seed=(42,))
    t = inp.torch(cuda_device)
    m = lib()
    ta, ts = torch.from_numpy(ang).to(cuda_device), torch.from_numpy(st).to(cuda_device)
    k1, q1, s1 = m.ssd_trap_rotate_qk(t["k"], t["q"], ta, t["dt"], ts, return_state=True)
    kk, qq, aa, dd = (t["k"].clone(), t["q"].clone(), ta.clone(), t["dt"].clone())
    state = ts.clone()
    for lo, hi in ((0, cut), (cut, L)):
        kp, qp = kk[:, lo:hi].clone(), qq[:, lo:hi].clone()
        m.ssd_trap_rotate_qk(kp, qp, aa[:, lo:hi].clone(), dd[:, lo:hi].clone(), state, k=kp, q=qp,
                             angle_state_out=state)
        kk[:, lo:hi], qq[:, lo:hi] = kp, qp
    torch.cuda.synchronize()
    kd = (kk.float() - k1.float()).abs().max().item()
    qd = (qq.float() - q1.float()).abs().max().item()
    sd = (state - s1).abs().max().item()
    report("rotate carry", k=kd, q=qd, state=sd)
    # the carried angle is rounded once more at the cut: a few bf16 roundings may flip
    assert kd <= 2 * RTOL_BF16_ROUND * kk.float().abs().max().item() and sd <= 1e-4


def test_rotate_then_trap_scan_workload(cuda_device):
    """The rotation workload (4 x 8192, 32 heads, N 128, 64 angles) and the trapezoidal
    scan fed by it, in three checks:
      1. the rotation, every element against the fp64 oracle within one bf16 rounding;
      2. the scan on the oracle's rotated k, q rounded to bf16 (identical inputs on both
         sides) against the fp64 scan oracle on 3 sampled heads, to the usual bf16 bar;
      3. rotation then scan on the GPU against 2.  Here the two rotations round a few
         values to bf16 differently: at |theta| ~ 20 rad the fp32 angle carries ~1e-5 rad
         of rounding, which moves ~0.3 % of the rotated values by one bf16 ulp, and these
         flips move y by ~0.2 % of its rms.  Bound: L2 error 2e-3 of y, no element off by
         more than 1 % of y's rms."""
    import torch
    w = synth.WORKLOADS["trap_rot_mamba3"]
    inp = synth.workload_inputs("trap_rot_mamba3")
    ang, st = synth.rotation_inputs(w["batch"], w["L"], w["nheads"], w["n_angles"])
    t = inp.torch(cuda_device)
    m = lib()
    k, q, so = m.ssd_trap_rotate_qk(t["k"], t["q"], torch.from_numpy(ang).to(cuda_device), t["dt"],
                                    torch.from_numpy(st).to(cuda_device), return_state=True)
    y, hf = m.ssd_trap_chunk_scan_fwd(t["x"], k, q, t["dt"], t["a"], t["trap"], t["D"], None,
                                      return_final=True)
    torch.cuda.synchronize()
    a = inp.arrays
    ko, qo, sto = oracle.trap_rotate(a["k"], a["q"], ang, a["dt"], st)
    # 1. the rotation
    scale = float(np.abs(ko).max())
    _check_rot("trap_rot_mamba3 rotate k", k.float().cpu().numpy(), ko, scale)
    _check_rot("trap_rot_mamba3 rotate q", q.float().cpu().numpy(), qo, scale)
    np.testing.assert_allclose(so.cpu().numpy(), sto, rtol=1e-4, atol=1e-4)
    del k, q
    # 2. the scan on the oracle's rotated values
    kr, qr = synth.round_bf16(ko.astype(np.float32)), synth.round_bf16(qo.astype(np.float32))
    del ko, qo
    kt = torch.from_numpy(kr).to(torch.bfloat16).to(cuda_device)
    qt = torch.from_numpy(qr).to(torch.bfloat16).to(cuda_device)
    y2, hf2 = m.ssd_trap_chunk_scan_fwd(t["x"], kt, qt, t["dt"], t["a"], t["trap"], t["D"], None,
                                        return_final=True)
    torch.cuda.synchronize()
    units = sample_units(np.random.default_rng(5), w["batch"], w["nheads"], 3)
    yo, ho = oracle.trap_fwd(a["x"], kr, qr, a["dt"], a["a"], a["trap"], a["D"], units=units)
    yg = np.stack([y2[b, :, h, :].cpu().numpy() for b, h in units])
    hg = np.stack([hf2[b, h].cpu().numpy() for b, h in units])
    ey, eh = synth.max_rel_err(yg, yo), synth.max_rel_err(hg, ho)
    report("trap_rot_mamba3 scan of rotated k, q sampled", y=ey, h_final=eh)
    assert ey <= TOL_BF16 and eh <= TOL_BF16
    # 3. the chained GPU path
    d = (y - y2).float()
    rms = float(y2.float().pow(2).mean().sqrt())
    l2 = float(d.pow(2).mean().sqrt()) / rms
    mx = float(d.abs().max()) / rms
    report("trap_rot_mamba3 rotate then scan", l2_rel=l2, max_over_rms=mx)
    assert l2 <= 2e-3 and mx <= 1e-2
