"""CPU pins of the fp64 S6 backward oracle (no GPU).

The gradient oracle is checked against things it does not compute itself:
  * inputs the outputs are affine in (u, B, C, D, h0): the change of the loss
    <dy, y> + <dh_final, h_final>, evaluated with the forward oracle, equals
    <gradient, perturbation> exactly (up to fp64 rounding);
  * inputs the outputs are not affine in (dt, dt_bias, A_log): central finite
    differences of the forward oracle, on inputs and steps chosen so that every
    perturbed value is exact in fp32;
  * phi1' against a numerical derivative of phi1, and its series branch.
A planted mistake anywhere in the adjoint (a dropped term, a wrong sign, a
missing sum over channels) changes one of these.
"""
import numpy as np
import pytest

import oracle
import synth

MODES = [oracle.BBAR_ZOH, oracle.BBAR_DT, oracle.BBAR_ONE]


def _q(a, step):
    """Round to a multiple of `step` (so that +-small steps stay exact in fp32)."""
    return (np.round(np.asarray(a, np.float64) / step) * step).astype(np.float32)


def _case(seed, a_log="uniform", h0=True, batch=2, L=9, Dm=3, N=5):
    inp = synth.s6_inputs(batch, L, Dm, N, seed=(700 + seed,), dt_bias="uniform", D="normal", h0=h0,
                          a_log=a_log)
    a = dict(inp.arrays)
    a["dt"] = _q(a["dt"], 2.0 ** -10)
    a["dt_bias"] = _q(a["dt_bias"], 2.0 ** -10)
    a["A_log"] = _q(a["A_log"], 2.0 ** -10)
    rng = np.random.default_rng(900 + seed)
    dy = rng.standard_normal((batch, L, Dm)).astype(np.float32)
    dhf = rng.standard_normal((batch, Dm, N)).astype(np.float32)
    return a, dy, dhf


def _loss(a, dy, dhf, mode):
    y, hf = oracle.s6_fwd(**a, flags=mode, nthreads=1)
    return float(np.sum(y * dy.astype(np.float64)) + np.sum(hf * dhf.astype(np.float64)))


def _grads(a, dy, dhf, mode):
    return oracle.s6_bwd(**a, dy=dy, dh_final=dhf, flags=mode, nthreads=2)


GRAD_OF = {"u": "du", "B": "dB", "C": "dC", "D": "dD", "h0": "dh0", "dt": "ddt",
           "dt_bias": "ddt_bias", "A_log": "dA_log"}


def _as_input_shape(name, g, a):
    """Oracle gradient arrays come in the input's shape except du/ddt/dh0 (already)."""
    return np.asarray(g).reshape(np.asarray(a[name]).shape)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("name", ["u", "B", "C", "D", "h0"])
def test_s6_bwd_affine_inputs_exact(name, mode):
    a, dy, dhf = _case(1)
    g = _as_input_shape(name, _grads(a, dy, dhf, mode)[GRAD_OF[name]], a)
    rng = np.random.default_rng(11)
    base = np.asarray(a[name], np.float32)
    pert = (base + rng.standard_normal(base.shape).astype(np.float32)).astype(np.float32)
    delta = pert.astype(np.float64) - base.astype(np.float64)     # realised perturbation
    b2 = dict(a)
    b2[name] = pert
    lhs = _loss(b2, dy, dhf, mode) - _loss(a, dy, dhf, mode)
    rhs = float(np.sum(g * delta))
    assert abs(lhs - rhs) <= 1e-9 * (abs(lhs) + abs(rhs) + 1.0), (lhs, rhs)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("name", ["dt", "dt_bias", "A_log"])
@pytest.mark.parametrize("a_log", ["uniform", -8.0])   # -8: |delta A| ~ 1e-5, the phi1' series branch
def test_s6_bwd_nonlinear_inputs_finite_differences(name, mode, a_log):
    a, dy, dhf = _case(2, a_log=a_log)
    if a_log == -8.0:
        a["A_log"] = _q(a["A_log"], 2.0 ** -10)
    g = _as_input_shape(name, _grads(a, dy, dhf, mode)[GRAD_OF[name]], a)
    rng = np.random.default_rng(12)
    base = np.asarray(a[name], np.float32)
    step = (rng.integers(1, 4, base.shape) * rng.choice([-1.0, 1.0], base.shape) * 2.0 ** -16)
    plus, minus = dict(a), dict(a)
    plus[name] = (base.astype(np.float64) + step).astype(np.float32)
    minus[name] = (base.astype(np.float64) - step).astype(np.float32)
    # the steps are exact in fp32 (inputs are multiples of 2^-10, |values| < 8)
    assert np.array_equal(plus[name].astype(np.float64) - base, step)
    assert np.array_equal(base - minus[name].astype(np.float64), step)
    fd = (_loss(plus, dy, dhf, mode) - _loss(minus, dy, dhf, mode)) / 2.0
    an = float(np.sum(g * step))
    assert abs(fd - an) <= 1e-6 * (abs(fd) + abs(an)) + 1e-12, (fd, an)


def test_s6_bwd_no_h0_and_no_dh_final():
    a, dy, _ = _case(3, h0=False)
    g = oracle.s6_bwd(**a, dy=dy, dh_final=None, flags=oracle.BBAR_ZOH, nthreads=1)
    rng = np.random.default_rng(5)
    base = a["u"]
    pert = (base + rng.standard_normal(base.shape).astype(np.float32)).astype(np.float32)
    delta = pert.astype(np.float64) - base
    y0, _ = oracle.s6_fwd(**a, flags=oracle.BBAR_ZOH, nthreads=1)
    a2 = dict(a)
    a2["u"] = pert
    y1, _ = oracle.s6_fwd(**a2, flags=oracle.BBAR_ZOH, nthreads=1)
    lhs = float(np.sum((y1 - y0) * dy))
    assert abs(lhs - float(np.sum(g["du"] * delta))) <= 1e-9 * (abs(lhs) + 1.0)


def test_s6_bwd_ranges_sum_to_full():
    a, dy, dhf = _case(4, Dm=4, batch=3)
    full = oracle.s6_bwd(**a, dy=dy, dh_final=dhf, nthreads=3)
    lo = oracle.s6_bwd(**a, dy=dy, dh_final=dhf, d_range=(0, 2), nthreads=1)
    hi = oracle.s6_bwd(**a, dy=dy, dh_final=dhf, d_range=(2, 4), nthreads=2)
    np.testing.assert_allclose(lo["dB"] + hi["dB"], full["dB"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lo["dC"] + hi["dC"], full["dC"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(np.concatenate([lo["du"], hi["du"]], 2), full["du"], rtol=1e-14)
    b1 = oracle.s6_bwd(**a, dy=dy, dh_final=dhf, b_range=(1, 2), nthreads=1)
    np.testing.assert_allclose(b1["dB"][0], full["dB"][1], rtol=1e-12, atol=1e-12)


def test_dphi1_against_numerical_derivative():
    for z in (-7.0, -1.5, -0.2, -2e-3, -1e-3, -9.9e-4, -1e-6, 0.0, 1e-4, 0.5):
        h = 1e-5
        num = (oracle.phi1(z + h) - oracle.phi1(z - h)) / (2 * h) if abs(z) > 2e-3 else None
        d = oracle.dphi1(z)
        if num is not None:
            assert abs(d - num) <= 1e-8 * max(1.0, abs(num))
    assert oracle.dphi1(0.0) == 0.5
    # the series and the closed form agree across the switch
    assert abs(oracle.dphi1(-1e-3 + 1e-12) - oracle.dphi1(-1e-3 - 1e-12)) < 1e-12
