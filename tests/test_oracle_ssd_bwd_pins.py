"""CPU pins of the fp64 SSD backward oracle (no GPU).

As for the S6 backward, the gradient oracle is checked against things it does
not compute itself:
  * inputs the outputs are affine in (x, B, C, D, h0): the change of the loss
    <dy, y> + <dh_final, h_final>, evaluated with the forward oracle, equals
    <gradient, perturbation> to fp64 rounding -- including the sums over the
    heads that share a group's B and C;
  * dt, dt_bias, A_log: central finite differences of the forward oracle on
    inputs and steps that are exact in fp32;
  * an SSD with headdim 1, one group and d_inner heads is an S6 scan whose A
    does not depend on the state index: its gradients equal the (separately
    written) S6 backward oracle's, with dA_log summed over the states.
"""
import numpy as np
import pytest

import oracle
import synth

MODES = [oracle.BBAR_DT, oracle.BBAR_ZOH, oracle.BBAR_ONE]


def _q(a, step):
    return (np.round(np.asarray(a, np.float64) / step) * step).astype(np.float32)


def _case(seed, h0=True, batch=2, L=11, H=4, P=3, N=5, G=2):
    inp = synth.ssd_inputs(batch, L, H, P, N, G, seed=(800 + seed,), dtype="f32", h0=h0, D="normal")
    a = dict(inp.arrays)
    a["dt"] = _q(a["dt"], 2.0 ** -10)
    a["dt_bias"] = _q(a["dt_bias"], 2.0 ** -10)
    a["A_log"] = _q(a["A_log"], 2.0 ** -10)
    rng = np.random.default_rng(950 + seed)
    dy = rng.standard_normal((batch, L, H, P)).astype(np.float32)
    dhf = rng.standard_normal((batch, H, P, N)).astype(np.float32)
    return a, dy, dhf, G


def _loss(a, dy, dhf, G, mode):
    y, hf = oracle.ssd_fwd(**a, ngroups=G, flags=mode, nthreads=1)
    return float(np.sum(y * dy.astype(np.float64)) + np.sum(hf * dhf.astype(np.float64)))


GRAD_OF = {"x": "dx", "B": "dB", "C": "dC", "D": "dD", "h0": "dh0", "dt": "ddt",
           "dt_bias": "ddt_bias", "A_log": "dA_log"}


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("name", ["x", "B", "C", "D", "h0"])
def test_ssd_bwd_affine_inputs_exact(name, mode):
    a, dy, dhf, G = _case(1)
    g = oracle.ssd_bwd(**a, dy=dy, dh_final=dhf, ngroups=G, flags=mode, nthreads=2)[GRAD_OF[name]]
    rng = np.random.default_rng(21)
    base = np.asarray(a[name], np.float32)
    pert = (base + rng.standard_normal(base.shape).astype(np.float32)).astype(np.float32)
    delta = pert.astype(np.float64) - base.astype(np.float64)
    b2 = dict(a)
    b2[name] = pert
    lhs = _loss(b2, dy, dhf, G, mode) - _loss(a, dy, dhf, G, mode)
    rhs = float(np.sum(np.asarray(g).reshape(base.shape) * delta))
    assert abs(lhs - rhs) <= 1e-9 * (abs(lhs) + abs(rhs) + 1.0), (lhs, rhs)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("name", ["dt", "dt_bias", "A_log"])
def test_ssd_bwd_nonlinear_inputs_finite_differences(name, mode):
    a, dy, dhf, G = _case(2)
    g = oracle.ssd_bwd(**a, dy=dy, dh_final=dhf, ngroups=G, flags=mode, nthreads=2)[GRAD_OF[name]]
    rng = np.random.default_rng(22)
    base = np.asarray(a[name], np.float32)
    step = rng.integers(1, 4, base.shape) * rng.choice([-1.0, 1.0], base.shape) * 2.0 ** -16
    plus, minus = dict(a), dict(a)
    plus[name] = (base.astype(np.float64) + step).astype(np.float32)
    minus[name] = (base.astype(np.float64) - step).astype(np.float32)
    assert np.array_equal(plus[name].astype(np.float64) - base, step)
    assert np.array_equal(base - minus[name].astype(np.float64), step)
    fd = (_loss(plus, dy, dhf, G, mode) - _loss(minus, dy, dhf, G, mode)) / 2.0
    an = float(np.sum(np.asarray(g).reshape(base.shape) * step))
    assert abs(fd - an) <= 1e-6 * (abs(fd) + abs(an)) + 1e-12, (fd, an)


def test_ssd_bwd_long_sequence_checkpoints():
    """L spans several of the oracle's 256-step recompute segments."""
    a, dy, dhf, G = _case(3, L=600, H=2, P=2, N=3, G=1, batch=1)
    g = oracle.ssd_bwd(**a, dy=dy, dh_final=dhf, ngroups=G, flags=oracle.BBAR_DT, nthreads=2)
    rng = np.random.default_rng(23)
    base = a["x"]
    pert = (base + rng.standard_normal(base.shape).astype(np.float32)).astype(np.float32)
    delta = pert.astype(np.float64) - base
    b2 = dict(a)
    b2["x"] = pert
    lhs = _loss(b2, dy, dhf, G, oracle.BBAR_DT) - _loss(a, dy, dhf, G, oracle.BBAR_DT)
    assert abs(lhs - float(np.sum(g["dx"] * delta))) <= 1e-9 * (abs(lhs) + 1.0)


@pytest.mark.parametrize("mode", MODES)
def test_ssd_bwd_equals_s6_bwd_on_an_s6_scan(mode):
    batch, L, Dm, N = 2, 9, 3, 4
    s6 = synth.s6_inputs(batch, L, Dm, N, seed=(31,), dt_bias="uniform", D="normal", h0=True,
                         a_log="uniform")
    a6 = dict(s6.arrays)
    A_head = a6["A_log"][:, 0].copy()
    a6["A_log"] = np.repeat(A_head[:, None], N, 1).astype(np.float32)     # A shared over states
    rng = np.random.default_rng(32)
    dy = rng.standard_normal((batch, L, Dm)).astype(np.float32)
    dhf = rng.standard_normal((batch, Dm, N)).astype(np.float32)
    g6 = oracle.s6_bwd(**a6, dy=dy, dh_final=dhf, flags=mode, nthreads=1)
    # the same scan as an SSD: heads = channels, headdim 1, one group
    gs = oracle.ssd_bwd(a6["u"][..., None], a6["dt"], a6["dt_bias"], A_head, a6["B"][:, :, None, :],
                        a6["C"][:, :, None, :], a6["D"], a6["h0"][:, :, None, :], dy[..., None],
                        dhf[:, :, None, :], ngroups=1, flags=mode, nthreads=1)
    np.testing.assert_allclose(gs["dx"][..., 0], g6["du"], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(gs["ddt"], g6["ddt"], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(gs["dB"][:, :, 0, :], g6["dB"], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(gs["dC"][:, :, 0, :], g6["dC"], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(gs["dA_log"], g6["dA_log"].sum(1), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(gs["dD"], g6["dD"], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(gs["ddt_bias"], g6["ddt_bias"], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(gs["dh0"][:, :, 0, :], g6["dh0"], rtol=1e-11, atol=1e-12)


def test_ssd_bwd_units_match_full():
    a, dy, dhf, G = _case(4)
    full = oracle.ssd_bwd(**a, dy=dy, dh_final=dhf, ngroups=G, nthreads=2)
    units = np.array([[1, 3], [0, 0]])
    part = oracle.ssd_bwd(**a, dy=dy, dh_final=dhf, ngroups=G, units=units, nthreads=1)
    np.testing.assert_array_equal(part["dx"][0], full["dx"][1, :, 3])
    np.testing.assert_array_equal(part["ddt"][1], full["ddt"][0, :, 0])
    np.testing.assert_array_equal(part["dh0"][0], full["dh0"][1, 3])
