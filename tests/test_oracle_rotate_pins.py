"""CPU pins of the fp64 Mamba-3 rotation oracle (angle * dt accumulation + RoPE on k, q).

  * the real scan of rotated k, q with trap = 1 is the complex-diagonal SSD with
    lambda = -exp(l) + i phi (checked against the separately written complex oracle,
    whose state is complex and whose phase enters through exp(delta lambda));
  * zero angles leave k, q unchanged; a rotation keeps every pair's norm and the
    inner product of k and q taken at the same step;
  * components past 2 n_angles are copied;
  * two calls carrying the angle state equal one call.
"""
import numpy as np

import oracle
import synth


def _delta(dt, bias):
    raw = dt.astype(np.float64) + bias.astype(np.float64)[None, None, :]
    return np.vectorize(oracle.softplus)(raw).astype(np.float32)


def test_rotated_trap_one_is_the_complex_ssd():
    """y of Re(sum conj(C) h), h_t = e^{delta lambda} h + delta B x (complex), equals the real
    trapezoidal scan (trap = 1) of k = B e^{-i Theta_t}, q = C e^{-i Theta_t} with
    Theta_t = phi sum_{r<=t} delta_r: the rotation carries the phase of every step."""
    batch, L, H, P, Nc = 2, 23, 2, 3, 4
    inp = synth.cssd_inputs(batch, L, H, P, Nc, 1, seed=(81,), phase=True)
    a = inp.arrays
    A_log = a["A_log"].copy()
    A_log[:, 1] = A_log[0, 1]                    # one phase for all heads (angles are shared)
    phi = float(A_log[0, 1])
    flags = oracle.BBAR_DT | oracle.CPLX_CONJ_C
    y_c, _ = oracle.cssd_fwd(a["x"], a["dt"], a["dt_bias"], A_log, a["B"], a["C"], a["D"], None,
                             ngroups=1, flags=flags)
    delta = _delta(a["dt"], a["dt_bias"])
    # complex pairs (re, im) of the single group, the same for every head
    Bk = np.broadcast_to(a["B"].reshape(batch, L, 1, 2 * Nc), (batch, L, H, 2 * Nc)).copy()
    Cq = np.broadcast_to(a["C"].reshape(batch, L, 1, 2 * Nc), (batch, L, H, 2 * Nc)).copy()
    angles = np.full((batch, L, Nc), -phi, np.float32)
    k, q, _ = oracle.trap_rotate(Bk, Cq, angles, delta)
    av = np.broadcast_to((-np.exp(A_log[:, 0].astype(np.float64))).astype(np.float32)[None, None, :],
                         delta.shape).copy()
    y_r, _ = oracle.trap_fwd(a["x"], k.astype(np.float32), q.astype(np.float32), delta, av,
                             np.ones_like(delta), a["D"])
    np.testing.assert_allclose(y_r, y_c, rtol=2e-5, atol=2e-5 * np.abs(y_c).max())


def test_rotation_sign_is_pinned():
    """The opposite angle (or a missing conjugate) breaks the complex equivalence."""
    batch, L, H, P, Nc = 1, 17, 1, 2, 3
    inp = synth.cssd_inputs(batch, L, H, P, Nc, 1, seed=(82,), phase=True)
    a = inp.arrays
    phi = float(a["A_log"][0, 1])
    y_c, _ = oracle.cssd_fwd(a["x"], a["dt"], a["dt_bias"], a["A_log"], a["B"], a["C"], a["D"], None,
                             ngroups=1, flags=oracle.BBAR_DT | oracle.CPLX_CONJ_C)
    delta = _delta(a["dt"], a["dt_bias"])
    Bk = a["B"].reshape(batch, L, 1, 2 * Nc)
    Cq = a["C"].reshape(batch, L, 1, 2 * Nc)
    av = np.full(delta.shape, -np.exp(np.float64(a["A_log"][0, 0])), np.float32)
    k, q, _ = oracle.trap_rotate(Bk, Cq, np.full((batch, L, Nc), +phi, np.float32), delta)
    y_r, _ = oracle.trap_fwd(a["x"], k.astype(np.float32), q.astype(np.float32), delta, av,
                             np.ones_like(delta), a["D"])
    assert np.max(np.abs(y_r - y_c)) > 1e-2 * np.abs(y_c).max()


def _rand(seed, batch=2, L=9, H=3, N=8, NA=3):
    rng = np.random.default_rng(900 + seed)
    f = np.float32
    return (rng.standard_normal((batch, L, H, N)).astype(f), rng.standard_normal((batch, L, H, N)).astype(f),
            rng.uniform(-3, 3, (batch, L, NA)).astype(f), rng.uniform(0.01, 0.5, (batch, L, H)).astype(f),
            rng.uniform(-4, 4, (batch, H, NA)).astype(f))


def test_zero_angles_are_the_identity():
    k, q, ang, dt, st = _rand(1)
    ko, qo, so = oracle.trap_rotate(k, q, np.zeros_like(ang), dt)
    assert np.array_equal(ko, k.astype(np.float64)) and np.array_equal(qo, q.astype(np.float64))
    assert np.array_equal(so, np.zeros_like(so))
    _, _, so = oracle.trap_rotate(k, q, np.zeros_like(ang), dt, st)
    assert np.array_equal(so, st.astype(np.float64))


def test_pair_norms_and_same_step_products_are_kept():
    k, q, ang, dt, st = _rand(2)
    NA = ang.shape[2]
    ko, qo, _ = oracle.trap_rotate(k, q, ang, dt, st)
    k64, q64 = k.astype(np.float64), q.astype(np.float64)
    for j in range(NA):
        sl = slice(2 * j, 2 * j + 2)
        np.testing.assert_allclose((ko[..., sl] ** 2).sum(-1), (k64[..., sl] ** 2).sum(-1), rtol=1e-12)
        np.testing.assert_allclose((ko[..., sl] * qo[..., sl]).sum(-1), (k64[..., sl] * q64[..., sl]).sum(-1),
                                   rtol=1e-10, atol=1e-12)
    # the tail past 2 n_angles is copied
    assert np.array_equal(ko[..., 2 * NA:], k64[..., 2 * NA:])
    assert np.array_equal(qo[..., 2 * NA:], q64[..., 2 * NA:])
    # and the rotated pairs did move
    assert np.abs(ko[..., :2 * NA] - k64[..., :2 * NA]).max() > 0.1


def test_angle_state_carries_across_calls():
    k, q, ang, dt, st = _rand(3, L=12)
    ko, qo, so = oracle.trap_rotate(k, q, ang, dt, st)
    c = 5
    k1, q1, s1 = oracle.trap_rotate(k[:, :c], q[:, :c], ang[:, :c], dt[:, :c], st)
    k2, q2, s2 = oracle.trap_rotate(k[:, c:], q[:, c:], ang[:, c:], dt[:, c:], s1.astype(np.float32))
    # the carried state is rounded to fp32 between the calls
    np.testing.assert_allclose(np.concatenate([k1, k2], 1), ko, rtol=0, atol=1e-5)
    np.testing.assert_allclose(np.concatenate([q1, q2], 1), qo, rtol=0, atol=1e-5)
    np.testing.assert_allclose(s2, so, rtol=1e-6)
