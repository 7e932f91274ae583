"""CPU pins of the fp64 Mamba-3 trapezoidal backward oracle (trap_bwd), by things it does
not compute itself:

  * the loss <dy, y> + <dh_final, h_final> is affine in q, D, h0, x, k, x_prev and k_prev
    (each with the others fixed), so its change under a finite perturbation, evaluated
    with the forward oracle on binary-exact values, equals <gradient, perturbation>;
  * dt, a and trap by central finite differences along random +-1 directions, on values
    and steps exact in fp32;
  * trap = 1 (beta = 0, gamma = dt) is the SSD recurrence: the separately written SSD
    backward oracle gives the same dx, dB, dC, dh0 and (through softplus) ddt.
"""
import numpy as np

import oracle
import synth

F = np.float32


def _grid(rng, shape, lo, hi, q=2.0 ** -8):
    return (np.round(rng.uniform(lo, hi, shape) / q) * q).astype(F)


def _inputs(seed, batch=2, L=13, H=2, P=3, N=4):
    rng = np.random.default_rng(1300 + seed)
    d = dict(x=_grid(rng, (batch, L, H, P), -2, 2), k=_grid(rng, (batch, L, H, N), -2, 2),
             q=_grid(rng, (batch, L, H, N), -2, 2),
             dt=_grid(rng, (batch, L, H), 0.05, 0.4, 2.0 ** -10), a=_grid(rng, (batch, L, H), -3, -0.2, 2.0 ** -10),
             trap=_grid(rng, (batch, L, H), 0.0, 1.0, 2.0 ** -10), D=_grid(rng, (H,), 0.5, 1.5),
             h0=_grid(rng, (batch, H, P, N), -1, 1), k_prev=_grid(rng, (batch, H, N), -2, 2),
             x_prev=_grid(rng, (batch, H, P), -2, 2))
    cot = dict(dy=_grid(rng, (batch, L, H, P), -1, 1), dh_final=_grid(rng, (batch, H, P, N), -1, 1))
    return d, cot


def _loss(d, cot):
    y, hf = oracle.trap_fwd(**d)
    return float((y * cot["dy"]).sum() + (hf * cot["dh_final"]).sum())


def test_affine_inputs_exactly():
    d, cot = _inputs(1)
    g = oracle.trap_bwd(**d, **cot)
    rng = np.random.default_rng(5)
    base = _loss(d, cot)
    for name, gname in (("q", "dq"), ("D", "dD"), ("h0", "dh0"), ("x", "dx"), ("k", "dk"),
                        ("x_prev", "dx_prev"), ("k_prev", "dk_prev")):
        delta = _grid(rng, d[name].shape, -1, 1)
        e = dict(d)
        e[name] = (d[name] + delta).astype(F)                     # exact: both on the 2^-8 grid
        assert np.array_equal(e[name].astype(np.float64), d[name].astype(np.float64) + delta)
        lhs = _loss(e, cot) - base
        rhs = float((g[gname] * delta).sum())
        assert abs(lhs - rhs) <= 1e-9 * (abs(rhs) + 1.0), (name, lhs, rhs)


def test_scalars_by_finite_differences():
    d, cot = _inputs(2)
    g = oracle.trap_bwd(**d, **cot)
    rng = np.random.default_rng(6)
    h = 2.0 ** -14                                  # on the 2^-10 grid, v +- h is exact in fp32
    for name, gname in (("dt", "ddt"), ("a", "da"), ("trap", "dtrap")):
        for _ in range(3):
            sgn = rng.choice([-1.0, 1.0], size=d[name].shape)
            ep, em = dict(d), dict(d)
            ep[name] = (d[name] + h * sgn).astype(F)
            em[name] = (d[name] - h * sgn).astype(F)
            assert np.array_equal(ep[name].astype(np.float64), d[name] + h * sgn)
            fd = (_loss(ep, cot) - _loss(em, cot)) / (2 * h)
            an = float((g[gname] * sgn).sum())
            assert abs(fd - an) <= 1e-6 * (abs(an) + 1.0), (name, fd, an)


def test_trap_one_is_the_ssd_backward():
    inp = synth.ssd_inputs(2, 17, 3, 4, 5, 3, seed=(73,), dtype="f32", h0=True, D="normal")
    a = inp.arrays
    rng = np.random.default_rng(7)
    dy = rng.standard_normal((2, 17, 3, 4)).astype(F)
    dhf = rng.standard_normal((2, 3, 4, 5)).astype(F)
    gs = oracle.ssd_bwd(**a, dy=dy, dh_final=dhf, ngroups=3, flags=oracle.BBAR_DT)
    raw = a["dt"].astype(np.float64) + a["dt_bias"].astype(np.float64)
    delta = np.vectorize(oracle.softplus)(raw).astype(F)
    A = -np.exp(a["A_log"].astype(np.float64))
    av = np.broadcast_to(A, delta.shape).astype(F)
    gt = oracle.trap_bwd(a["x"], a["B"], a["C"], delta, av, np.ones_like(delta), a["D"], a["h0"], None, None,
                         dy, dhf)
    for ks, kt in (("dx", "dx"), ("dB", "dk"), ("dC", "dq"), ("dh0", "dh0")):
        np.testing.assert_allclose(gt[kt], gs[ks], rtol=2e-5, atol=2e-5 * np.abs(gs[ks]).max())
    # the SSD backward's ddt is through softplus: ddt_raw = ddt_delta * sigmoid(raw)
    sig = 1.0 / (1.0 + np.exp(-raw))
    np.testing.assert_allclose(gt["ddt"] * sig, gs["ddt"], rtol=2e-5, atol=2e-5 * np.abs(gs["ddt"]).max())
    np.testing.assert_allclose(gt["dD"], gs["dD"], rtol=1e-9)


def test_long_sequence_crosses_checkpoints():
    """600 steps (three recompute segments): the affine pin on x and a finite difference on
    dt still hold."""
    d, cot = _inputs(3, batch=1, L=600, H=1, P=2, N=3)
    g = oracle.trap_bwd(**d, **cot)
    rng = np.random.default_rng(8)
    base = _loss(d, cot)
    delta = _grid(rng, d["x"].shape, -1, 1)
    e = dict(d)
    e["x"] = (d["x"] + delta).astype(F)
    lhs, rhs = _loss(e, cot) - base, float((g["dx"] * delta).sum())
    assert abs(lhs - rhs) <= 1e-9 * (abs(rhs) + 1.0)
    h = 2.0 ** -14
    sgn = rng.choice([-1.0, 1.0], size=d["dt"].shape)
    ep, em = dict(d), dict(d)
    ep["dt"] = (d["dt"] + h * sgn).astype(F)
    em["dt"] = (d["dt"] - h * sgn).astype(F)
    fd = (_loss(ep, cot) - _loss(em, cot)) / (2 * h)
    an = float((g["ddt"] * sgn).sum())
    assert abs(fd - an) <= 1e-6 * (abs(an) + 1.0)
