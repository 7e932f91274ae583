"""GPU parity of ssm_s6_fused_fwd (causal conv1d + SiLU, the S6 scan, SiLU(z) gating, the
carried conv state) against the fp64 layer oracle, including the decode step (L = 1 with
the state and the conv state carried in place)."""
import numpy as np
import pytest

from scipy.special import expit

import oracle
import synth
from helpers import TOL_BF16, TOL_F32, lib, report, sample_units

pytestmark = pytest.mark.gpu

ZOH, DT, ONE = oracle.BBAR_ZOH, oracle.BBAR_DT, oracle.BBAR_ONE


def _gpu(inp, device, flags, **kw):
    import torch
    t = inp.torch(device)
    u = torch.empty(t["x"].shape, dtype=torch.float32, device=device)
    y, hf, cs = lib().ssm_s6_fused_fwd(t["x"], t["conv_w"], t["conv_b"], t["dt"], t["dt_bias"], t["A_log"],
                                       t["B"], t["C"], t["D"], t["h0"], t["conv_state"], t["z"], flags=flags,
                                       return_final=True, u_out=u, **kw)
    torch.cuda.synchronize()
    return y.cpu().numpy(), hf.cpu().numpy(), u.cpu().numpy(), None if cs is None else cs.cpu().numpy()


def _ungate(y, z):
    """y / SiLU(z), the gate formed in fp64 from the inputs: a printed diagnostic of the
    scan's own error apart from the gate (the parity bar applies to the gated y)."""
    if z is None:
        return y
    z = z.astype(np.float64)
    return y / (z * expit(z))


def _oracle(inp, flags, units=None):
    a = inp.arrays
    return oracle.s6_layer_fwd(a["x"], a["conv_w"], a["conv_b"], a["dt"], a["dt_bias"], a["A_log"], a["B"],
                               a["C"], a["D"], a["h0"], a["conv_state"], a["z"], flags=flags, units=units)


CASES = [  # batch, L, d_inner, N, K, dtype, flags, conv state, gate, h0
    (2, 100, 48, 16, 4, "f32", ZOH, True, True, True),
    (1, 37, 20, 16, 4, "f32", ZOH, False, True, False),
    (2, 64, 32, 16, 3, "f32", DT, True, False, True),
    (1, 5, 16, 16, 4, "f32", ZOH, True, True, True),       # shorter than two tiles
    (1, 2, 16, 4, 4, "f32", ONE, True, True, False),       # shorter than the conv: state tail carried
    (1, 300, 40, 8, 2, "f32", ZOH, True, True, True),
    (1, 129, 24, 64, 4, "f32", ZOH, True, True, True),
    (2, 70, 64, 16, 1, "f32", DT, False, True, False),     # K = 1: no conv state
    (2, 200, 96, 16, 4, "bf16", ZOH, True, True, True),
    (1, 33, 33, 32, 4, "bf16", DT, True, True, False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b{}L{}D{}N{}K{}{}f{}s{}z{}h{}".format(*[int(v) if isinstance(v, bool) else v for v in c]))
def test_fused_shapes(cuda_device, case):
    batch, L, Dm, N, K, dtype, flags, st, gate, h0 = case
    inp = synth.layer_inputs(batch, L, Dm, N, K, seed=(L, Dm), dtype=dtype, conv_state=st, gate=gate, h0=h0)
    y, hf, u, cs = _gpu(inp, cuda_device, flags)
    yo, ho, uo, cso = _oracle(inp, flags)
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    z = inp.arrays["z"]
    ey = synth.max_rel_err(y, yo)
    eh, eu = synth.max_rel_err(hf, ho), synth.max_rel_err(u, uo)
    report(f"s6 fused {case}", y=ey, h_final=eh, u=eu, y_ungated=synth.max_rel_err(_ungate(y, z), _ungate(yo, z)))
    assert np.isfinite(y).all()
    assert ey <= tol and eh <= tol and eu <= TOL_F32
    if K > 1:
        # the carried state is a copy of inputs: exact
        assert np.array_equal(cs, cso.astype(np.float32))


def test_fused_decode_steps_in_place(cuda_device):
    """T decode calls (L = 1) carrying h and the conv state in place equal one call over T
    steps; the oracle runs the T steps as one sequence."""
    import torch
    T = 24
    inp = synth.layer_inputs(4, T, 64, 16, 4, seed=(51,), h0=True)
    yo, ho, _, cso = _oracle(inp, ZOH)
    t = inp.torch(cuda_device)
    h = t["h0"].clone()
    st = t["conv_state"].clone()
    m = lib()
    ys = []
    for s in range(T):
        sl = {n: t[n][:, s:s + 1].contiguous() for n in ("x", "dt", "B", "C", "z")}
        y = m.ssm_s6_fused_fwd(sl["x"], t["conv_w"], t["conv_b"], sl["dt"], t["dt_bias"], t["A_log"], sl["B"],
                               sl["C"], t["D"], h, st, sl["z"], h_final=h, conv_state_out=st)
        ys.append(y)
    torch.cuda.synchronize()
    yg = torch.cat(ys, dim=1).cpu().numpy()
    ey, eh = synth.max_rel_err(yg, yo), synth.max_rel_err(h.cpu().numpy(), ho)
    report("s6 decode in place", y=ey, h_final=eh)
    assert ey <= TOL_F32 and eh <= TOL_F32
    assert np.array_equal(st.cpu().numpy(), cso.astype(np.float32))


def test_fused_equals_plain_scan_of_its_u(cuda_device):
    """The fused kernel's scan is the plain kernel's: scanning the fused call's u with
    ssm_s6_scan_fwd and gating gives the fused y (both fp32 on the GPU)."""
    import torch
    inp = synth.layer_inputs(2, 150, 48, 16, 4, seed=(52,), h0=True)
    t = inp.torch(cuda_device)
    m = lib()
    u = torch.empty(t["x"].shape, dtype=torch.float32, device=cuda_device)
    y, hf, _ = m.ssm_s6_fused_fwd(t["x"], t["conv_w"], t["conv_b"], t["dt"], t["dt_bias"], t["A_log"], t["B"],
                                  t["C"], t["D"], t["h0"], t["conv_state"], t["z"], return_final=True, u_out=u)
    y2, hf2 = m.ssm_s6_scan_fwd(u, t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"], t["D"], t["h0"],
                                return_final=True)
    z = t["z"]
    g = y2 * (z / (1 + torch.exp(-z)))
    torch.cuda.synchronize()
    assert torch.equal(hf, hf2)
    e = synth.max_rel_err(y.cpu().numpy(), g.cpu().numpy())
    report("fused vs plain scan of u", y=e)
    assert e <= 1e-5


def test_fused_bitwise_deterministic(cuda_device):
    inp = synth.layer_inputs(2, 500, 96, 16, 4, seed=(53,))
    a = _gpu(inp, cuda_device, ZOH)
    b = _gpu(inp, cuda_device, ZOH)
    assert all(np.array_equal(p, q) for p, q in zip(a, b))


def test_fused_mamba1_workload_sampled(cuda_device):
    """Full Mamba-1 layer shape (8 x 2048 x 1536, N 16, K 4, fp32) against the oracle on
    256 sampled (b, d) channels over the whole sequence."""
    w = synth.WORKLOADS["s6_layer_mamba1"]
    inp = synth.workload_inputs("s6_layer_mamba1")
    y, hf, u, cs = _gpu(inp, cuda_device, ZOH)
    units = sample_units(np.random.default_rng(7), w["batch"], w["d_inner"], 256)
    yo, ho, uo, cso = _oracle(inp, ZOH, units=units)
    yg = np.stack([y[b, :, d] for b, d in units])
    hg = np.stack([hf[b, d] for b, d in units])
    ug = np.stack([u[b, :, d] for b, d in units])
    zs = np.stack([inp.arrays["z"][b, :, d] for b, d in units])
    ey = synth.max_rel_err(yg, yo)
    eh, eu = synth.max_rel_err(hg, ho), synth.max_rel_err(ug, uo)
    report("s6_layer_mamba1 sampled", y=ey, h_final=eh, u=eu, y_ungated=synth.max_rel_err(_ungate(yg, zs), _ungate(yo, zs)))
    assert ey <= TOL_F32 and eh <= TOL_F32 and eu <= TOL_F32
    assert np.array_equal(np.stack([cs[b, d] for b, d in units]), cso.astype(np.float32))


def test_plain_decode_steps_in_place(cuda_device):
    """ssm_s6_scan_fwd with L = 1 (the one-thread-per-channel step kernel), h carried in
    place over T calls, against the fp64 S6 oracle over the T steps; bf16 and fp32, all three
    input scales, a state size that is not a multiple of 4."""
    import torch
    T = 20
    m = lib()
    for dtype, N, flags in (("f32", 16, ZOH), ("bf16", 16, DT), ("f32", 6, ONE), ("f32", 64, ZOH)):
        inp = synth.s6_inputs(3, T, 40, N, seed=(54, N), dtype=dtype, h0=True)
        yo, ho = oracle.s6_fwd(**inp.arrays, flags=flags)
        t = inp.torch(cuda_device)
        h = t["h0"].clone()
        ys = []
        for s in range(T):
            sl = {n: t[n][:, s:s + 1].contiguous() for n in ("u", "dt", "B", "C")}
            ys.append(m.ssm_s6_scan_fwd(sl["u"], sl["dt"], t["dt_bias"], t["A_log"], sl["B"], sl["C"], t["D"],
                                        h, flags=flags, h_final=h)[0])
        torch.cuda.synchronize()
        ey = synth.max_rel_err(torch.cat(ys, dim=1).cpu().numpy(), yo)
        eh = synth.max_rel_err(h.cpu().numpy(), ho)
        report(f"s6 plain decode {dtype} N={N} flags={flags}", y=ey, h_final=eh)
        tol = TOL_F32 if dtype == "f32" else TOL_BF16
        assert ey <= tol and eh <= tol
