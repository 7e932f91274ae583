"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Each test computes its expectation independently of the oracle's code path
(exact fractions, closed forms, a brute-force materialised matrix, or an
identity between two different oracle functions) so that a dropped term, a
wrong sign or index or a transposed operand in the oracle fails one of them.
CPU only.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------ elementary ---

def test_softplus_closed_forms():
    assert oracle.softplus(0.0) == pytest.approx(math.log(2.0), rel=1e-15)
    for x in (-30.0, -3.5, -1e-3, 0.25, 2.0, 40.0):
        # softplus(x) - softplus(-x) = x  (log((1+e^x)/(1+e^-x)) = x)
        assert oracle.softplus(x) - oracle.softplus(-x) == pytest.approx(x, rel=1e-13, abs=1e-15)
    assert oracle.softplus(1000.0) == 1000.0          # no overflow
    assert oracle.softplus(-50.0) == pytest.approx(math.exp(-50.0), rel=1e-12)


def test_phi1_closed_forms():
    assert oracle.phi1(0.0) == 1.0
    assert oracle.phi1(-1.0) == pytest.approx(1.0 - math.exp(-1.0), rel=1e-15)
    for z in (-1e-9, -1e-5, -0.01):
        series = 1 + z / 2 + z * z / 6 + z ** 3 / 24 + z ** 4 / 120 + z ** 5 / 720
        assert oracle.phi1(z) == pytest.approx(series, rel=1e-14)


# -------------------------------------------------------------------- S6 ---

def _hand_rows():
    rows = []
    with open(os.path.join(GOLDEN, "s6_hand_cases.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, L, u, D, h0, t, val = [c.strip() for c in line.split("|")]
            rows.append((name, int(L), [float(v) for v in u.split(",")], float(D), float(h0),
                         int(t), Fraction(val)))
    return rows


@pytest.mark.parametrize("row", _hand_rows(), ids=lambda r: r[0])
def test_s6_hand_cases(row):
    name, L, u, D, h0, t, expect = row
    N = 4
    uu = np.array(u, np.float32).reshape(1, L, 1)
    dt = np.zeros((1, L, 1), np.float32)
    A_log = np.log(np.arange(1, N + 1, dtype=np.float64)).astype(np.float32).reshape(1, N)
    B = np.ones((1, L, N), np.float32)
    C = np.ones((1, L, N), np.float32)
    h0a = np.full((1, 1, N), h0, np.float32)
    y, _ = oracle.s6_fwd(uu, dt, None, A_log, B, C, np.array([D], np.float32), h0=h0a)
    # A_log is float32-rounded, so A_n is (n+1)(1 + O(6e-8)): agree to ~1e-7
    assert y[0, t, 0] == pytest.approx(float(expect), rel=3e-7)


def test_s6_exact_case_unit_A():
    # A_log = 0 is exact in fp32: A = -1, delta = ln 2, Abar = 1/2, beta = 1/2.
    L, N = 3, 2
    u = np.array([1.0, 2.0, -1.0], np.float32).reshape(1, L, 1)
    B = np.array([[1, 2], [3, 4], [5, 6]], np.float32).reshape(1, L, N)
    C = np.array([[1, -1], [2, 0], [0, 3]], np.float32).reshape(1, L, N)
    y, hf = oracle.s6_fwd(u, np.zeros((1, L, 1), np.float32), None, np.zeros((1, N), np.float32),
                          B, C, np.array([0.5], np.float32))
    h = np.zeros(N)
    ys = []
    for t in range(L):
        h = 0.5 * h + 0.5 * B[0, t] * u[0, t, 0]
        ys.append(C[0, t] @ h + 0.5 * u[0, t, 0])
    np.testing.assert_allclose(y[0, :, 0], ys, rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(hf[0, 0], h, rtol=1e-15)


def _s6_closed_form(i, mode):
    """Independent brute force: h_t = sum_s exp(A(Lam_t - Lam_s)) beta_s B_s u_s + exp(A Lam_t) h0,
    Lam the inclusive running sum of delta."""
    a = {k: (None if v is None else v.astype(np.float64)) for k, v in i.arrays.items()}
    batch, L, Dm = a["u"].shape
    N = a["A_log"].shape[1]
    bias = a["dt_bias"] if a["dt_bias"] is not None else np.zeros(Dm)
    xb = a["dt"] + bias
    delta = np.logaddexp(0.0, xb)                       # softplus
    Lam = np.cumsum(delta, axis=1)                       # (b, L, d)
    A = -np.exp(a["A_log"])                              # (d, n)
    z = delta[..., None] * A                             # (b, L, d, n)
    if mode == oracle.BBAR_ZOH:
        beta = (np.exp(z) - 1.0) / A                     # exact formula of the page helper
    elif mode == oracle.BBAR_DT:
        beta = np.broadcast_to(delta[..., None], z.shape)
    else:
        beta = np.ones_like(z)
    drive = beta * a["B"][:, :, None, :] * a["u"][..., None]     # (b, s, d, n)
    dl = Lam[:, :, None, :] - Lam[:, None, :, :]                 # (b, t, s, d) = Lam_t - Lam_s
    W = np.exp(dl[..., None] * A)                                # (b, t, s, d, n)
    tri = np.tril(np.ones((L, L)))[None, :, :, None, None]
    H = np.einsum("btsdn,bsdn->btdn", W * tri, drive)
    if a["h0"] is not None:
        H = H + np.exp(Lam[..., None] * A) * a["h0"][:, None]
    Dv = a["D"] if a["D"] is not None else np.zeros(Dm)
    y = np.einsum("btn,btdn->btd", a["C"], H) + Dv * a["u"]
    return y, H[:, -1]


@pytest.mark.parametrize("mode", [oracle.BBAR_ZOH, oracle.BBAR_DT, oracle.BBAR_ONE])
def test_s6_matches_closed_form(mode):
    i = synth.s6_inputs(2, 19, 5, 6, seed=(11,), a_log="uniform", h0=True)
    y, hf = oracle.s6_fwd(**i.arrays, flags=mode)
    ye, he = _s6_closed_form(i, mode)
    np.testing.assert_allclose(y, ye, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(hf, he, rtol=1e-11, atol=1e-12)


def test_s6_zoh_tends_to_weighted_cumsum_as_A_to_0():
    # A_log -> -inf: A -> 0-, Abar -> 1, beta -> delta, so y_t = C_t . sum_{s<=t} delta_s B_s u_s + D u_t
    i = synth.s6_inputs(1, 30, 3, 4, seed=(3,), a_log=-40.0)
    y, _ = oracle.s6_fwd(**i.arrays, flags=oracle.BBAR_ZOH)
    a = i.arrays
    delta = np.logaddexp(0.0, a["dt"].astype(np.float64) + a["dt_bias"])
    acc = np.cumsum(delta[..., None] * a["B"][:, :, None, :] * a["u"][..., None], axis=1)
    ye = (np.einsum("btn,btdn->btd", a["C"].astype(np.float64), acc)
          + a["D"].astype(np.float64) * a["u"].astype(np.float64))
    np.testing.assert_allclose(y, ye, rtol=1e-12, atol=1e-13)


def test_s6_zoh_over_dt_is_phi1_single_step():
    # one step from h0 = 0 and N = 1: y_ZOH / y_DT = beta/delta = phi1(delta*A)
    i = synth.s6_inputs(1, 1, 7, 1, seed=(5,), a_log="uniform", D=None)
    yz, _ = oracle.s6_fwd(**i.arrays, flags=oracle.BBAR_ZOH)
    yd, _ = oracle.s6_fwd(**i.arrays, flags=oracle.BBAR_DT)
    a = i.arrays
    delta = np.logaddexp(0.0, a["dt"].astype(np.float64) + a["dt_bias"])[0, 0]
    z = delta * -np.exp(a["A_log"][:, 0].astype(np.float64))
    np.testing.assert_allclose(yz[0, 0] / yd[0, 0], np.expm1(z) / z, rtol=1e-13)


def test_s6_carry_composition():
    i = synth.s6_inputs(2, 40, 4, 8, seed=(7,), h0=True)
    a = i.arrays
    y, hf = oracle.s6_fwd(**a)
    L1 = 17
    first = {k: v for k, v in a.items()}
    second = {k: v for k, v in a.items()}
    for k in ("u", "dt", "B", "C"):
        first[k] = a[k][:, :L1].copy()
        second[k] = a[k][:, L1:].copy()
    y1, h1 = oracle.s6_fwd(**first)
    second["h0"] = h1.astype(np.float32)
    # the carried state is rounded to float32 on the way, so compare loosely
    y2, h2 = oracle.s6_fwd(**second)
    np.testing.assert_allclose(y[:, :L1], y1, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(y[:, L1:], y2, rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(hf, h2, rtol=1e-6, atol=1e-6)


def test_s6_linearity_in_u_and_batch_independence():
    i = synth.s6_inputs(3, 25, 4, 5, seed=(8,))
    a = dict(i.arrays)
    u2 = synth.s6_inputs(3, 25, 4, 5, seed=(9,)).arrays["u"]
    y1, _ = oracle.s6_fwd(**a)
    b = dict(a); b["u"] = u2
    y2, _ = oracle.s6_fwd(**b)
    c = dict(a); c["u"] = (a["u"].astype(np.float64) + 2 * u2.astype(np.float64)).astype(np.float32)
    y3, _ = oracle.s6_fwd(**c)
    # the combined u is rounded to float32; compare against the same rounding
    np.testing.assert_allclose(y3, y1 + 2 * y2, rtol=1e-5, atol=1e-5)
    perm = [2, 0, 1]
    d = dict(a)
    for k in ("u", "dt", "B", "C"):
        d[k] = a[k][perm].copy()
    y4, _ = oracle.s6_fwd(**d)
    np.testing.assert_allclose(y4, y1[perm], rtol=0, atol=0)


def test_s6_units_subset_matches_full():
    i = synth.s6_inputs(2, 12, 6, 3, seed=(4,), h0=True)
    y, hf = oracle.s6_fwd(**i.arrays)
    units = [(1, 5), (0, 0), (1, 2)]
    yu, hu = oracle.s6_fwd(**i.arrays, units=units)
    for k, (b, d) in enumerate(units):
        np.testing.assert_array_equal(yu[k], y[b, :, d])
        np.testing.assert_array_equal(hu[k], hf[b, d])


# ------------------------------------------------------------------- SSD ---

def _ssd_brute(i, mode):
    """Materialised semiseparable matrix (fp64): y = M x + exp(cs_t) C_t.h0 + D x."""
    a = {k: (None if v is None else v.astype(np.float64)) for k, v in i.arrays.items()}
    batch, L, H, P = a["x"].shape
    G, N = a["B"].shape[2:]
    bias = a["dt_bias"] if a["dt_bias"] is not None else np.zeros(H)
    delta = np.logaddexp(0.0, a["dt"] + bias)                 # (b, L, H)
    A = -np.exp(a["A_log"])                                  # (H,)
    aa = delta * A
    if mode == oracle.BBAR_DT:
        sig = delta
    elif mode == oracle.BBAR_ZOH:
        sig = np.expm1(aa) / A
    else:
        sig = np.ones_like(delta)
    cs = np.cumsum(aa, axis=1)                                # inclusive
    y = np.zeros((batch, L, H, P))
    hf = np.zeros((batch, H, P, N))
    for h in range(H):
        g = (h * G) // H
        for b in range(batch):
            CB = a["C"][b, :, g, :] @ a["B"][b, :, g, :].T    # (t, s)
            dec = np.exp(cs[b, :, h][:, None] - cs[b, :, h][None, :])
            M = np.tril(CB * dec * sig[b, :, h][None, :])
            yy = M @ a["x"][b, :, h, :]
            w_end = np.exp(cs[b, -1, h] - cs[b, :, h]) * sig[b, :, h]
            S = (a["x"][b, :, h, :] * w_end[:, None]).T @ a["B"][b, :, g, :]
            if a["h0"] is not None:
                yy += np.exp(cs[b, :, h])[:, None] * (a["C"][b, :, g, :] @ a["h0"][b, h].T)
                S += np.exp(cs[b, -1, h]) * a["h0"][b, h]
            Dv = a["D"][h] if a["D"] is not None else 0.0
            y[b, :, h, :] = yy + Dv * a["x"][b, :, h, :]
            hf[b, h] = S
    return y, hf


@pytest.mark.parametrize("mode", [oracle.BBAR_DT, oracle.BBAR_ZOH, oracle.BBAR_ONE])
def test_ssd_matches_semiseparable_brute_force(mode):
    i = synth.ssd_inputs(2, 37, 4, 3, 5, 2, seed=(21,), dtype="f32", h0=True, D="normal")
    y, hf = oracle.ssd_fwd(**i.arrays, ngroups=2, flags=mode)
    ye, he = _ssd_brute(i, mode)
    np.testing.assert_allclose(y, ye, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(hf, he, rtol=1e-10, atol=1e-11)


def _ssd_chunked_fp64(i, Q, mode=oracle.BBAR_DT):
    """The chunked decomposition the GPU uses (per-chunk cumsum, chunk-local states,
    inter-chunk pass, intra-chunk masked product, state-to-output), in fp64."""
    a = {k: (None if v is None else v.astype(np.float64)) for k, v in i.arrays.items()}
    batch, L, H, P = a["x"].shape
    G, N = a["B"].shape[2:]
    bias = a["dt_bias"] if a["dt_bias"] is not None else np.zeros(H)
    delta = np.logaddexp(0.0, a["dt"] + bias)
    A = -np.exp(a["A_log"])
    aa = delta * A
    sig = delta if mode == oracle.BBAR_DT else (np.expm1(aa) / A if mode == oracle.BBAR_ZOH
                                               else np.ones_like(delta))
    y = np.zeros((batch, L, H, P))
    hf = np.zeros((batch, H, P, N))
    for b in range(batch):
        for h in range(H):
            g = (h * G) // H
            S = a["h0"][b, h].copy() if a["h0"] is not None else np.zeros((P, N))
            for c0 in range(0, L, Q):
                sl = slice(c0, min(c0 + Q, L))
                cs = np.cumsum(aa[b, sl, h])
                X, Bc, Cc = a["x"][b, sl, h, :], a["B"][b, sl, g, :], a["C"][b, sl, g, :]
                s = sig[b, sl, h]
                Lm = np.tril(np.exp(cs[:, None] - cs[None, :]) * s[None, :])
                yc = ((Cc @ Bc.T) * Lm) @ X + np.exp(cs)[:, None] * (Cc @ S.T)
                y[b, sl, h, :] = yc + a["D"][h] * X
                Shat = (X * (np.exp(cs[-1] - cs) * s)[:, None]).T @ Bc
                S = np.exp(cs[-1]) * S + Shat
            hf[b, h] = S
    return y, hf


@pytest.mark.parametrize("Q", [1, 3, 16, 64])
def test_ssd_chunked_decomposition_equals_sequential(Q):
    i = synth.ssd_inputs(2, 45, 4, 3, 4, 2, seed=(22,), dtype="f32", h0=True)
    y, hf = oracle.ssd_fwd(**i.arrays, ngroups=2)
    yc, hc = _ssd_chunked_fp64(i, Q)
    np.testing.assert_allclose(yc, y, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(hc, hf, rtol=1e-10, atol=1e-11)


@pytest.mark.parametrize("mode", [oracle.BBAR_DT, oracle.BBAR_ZOH, oracle.BBAR_ONE])
def test_ssd_reduces_to_s6(mode):
    # S6 with A constant over n per head, delta/dt_bias/D broadcast over a head's
    # channels and shared B, C is the SSD recurrence.
    batch, L, H, P, N = 2, 23, 3, 4, 5
    i = synth.ssd_inputs(batch, L, H, P, N, 1, seed=(23,), dtype="f32", h0=True, D="normal")
    a = i.arrays
    ys, hs = oracle.ssd_fwd(**a, ngroups=1, flags=mode)
    u = a["x"].reshape(batch, L, H * P)
    dt = np.repeat(a["dt"], P, axis=2)
    bias = np.repeat(a["dt_bias"], P)
    A_log = np.repeat(a["A_log"], P)[:, None] * np.ones((1, N), np.float32)
    Dv = np.repeat(a["D"], P)
    h0 = a["h0"].reshape(batch, H * P, N)
    y6, h6 = oracle.s6_fwd(u, dt, bias, A_log.astype(np.float32), a["B"][:, :, 0], a["C"][:, :, 0],
                           Dv, h0=h0, flags=mode)
    np.testing.assert_allclose(y6.reshape(ys.shape), ys, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(h6.reshape(hs.shape), hs, rtol=1e-12, atol=1e-13)


def test_ssd_group_replication():
    i = synth.ssd_inputs(1, 20, 4, 3, 6, 1, seed=(24,), dtype="f32")
    a = dict(i.arrays)
    y1, h1 = oracle.ssd_fwd(**a, ngroups=1)
    a["B"] = np.repeat(a["B"], 4, axis=2)
    a["C"] = np.repeat(a["C"], 4, axis=2)
    y4, h4 = oracle.ssd_fwd(**a, ngroups=4)
    np.testing.assert_array_equal(y1, y4)
    np.testing.assert_array_equal(h1, h4)


def test_ssd_one_step_hand_case():
    # L = 1, h0 = 0: y = sigma * x * (C . B) + D x, with sigma = delta = softplus(dt + bias)
    x = np.array([1.0, -2.0], np.float32).reshape(1, 1, 1, 2)
    B = np.array([1.0, 2.0, 3.0], np.float32).reshape(1, 1, 1, 3)
    C = np.array([0.5, -1.0, 2.0], np.float32).reshape(1, 1, 1, 3)
    dt = np.zeros((1, 1, 1), np.float32)
    y, hf = oracle.ssd_fwd(x, dt, None, np.zeros(1, np.float32), B, C, np.array([3.0], np.float32))
    cb = 0.5 * 1 - 1.0 * 2 + 2.0 * 3
    xd = x[0, 0, 0].astype(np.float64)
    np.testing.assert_allclose(y[0, 0, 0], math.log(2) * cb * xd + 3.0 * xd, rtol=1e-15)
    np.testing.assert_allclose(hf[0, 0], math.log(2) * np.outer(xd, B[0, 0, 0].astype(np.float64)),
                               rtol=1e-15)


# --------------------------------------------------------------- complex ---

def _cssd_brute(i, flags):
    a = {k: (None if v is None else v.astype(np.float64)) for k, v in i.arrays.items()}
    batch, L, H, P = a["x"].shape
    G, Nc = a["B"].shape[2:4]
    Bc = a["B"][..., 0] + 1j * a["B"][..., 1]
    Cc = a["C"][..., 0] + 1j * a["C"][..., 1]
    if flags & oracle.CPLX_CONJ_C:
        Cc = np.conj(Cc)
    delta = np.logaddexp(0.0, a["dt"] + a["dt_bias"])
    Lam = np.cumsum(delta, axis=1)
    ell, phi = a["A_log"][:, 0], a["A_log"][:, 1]
    am = flags & 0xC
    y = np.zeros((batch, L, H, P))
    hf = np.zeros((batch, H, P, Nc), complex)
    for h in range(H):
        g = (h * G) // H
        if am == oracle.CPLX_CODE:
            mu = ell[h] + 1j * phi[h]
            beta = np.expm1(delta[:, :, h] * mu) * np.exp(-mu)
        else:
            mu = (np.exp(ell[h]) * np.exp(1j * phi[h])) if am == oracle.CPLX_DOC else (-np.exp(ell[h]) + 1j * phi[h])
            bm = flags & 0x3
            beta = (np.expm1(delta[:, :, h] * mu) / mu if bm == oracle.BBAR_ZOH
                    else (delta[:, :, h] + 0j if bm == oracle.BBAR_DT else np.ones_like(delta[:, :, h]) + 0j))
        for b in range(batch):
            dl = Lam[b, :, h][:, None] - Lam[b, :, h][None, :]
            E = np.tril(np.exp(mu * dl))                                  # (t, s)
            G_ts = Cc[b, :, g, :] @ Bc[b, :, g, :].T                       # (t, s), no conjugation
            M = (G_ts * E * beta[b][None, :]).real
            yy = M @ a["x"][b, :, h, :]
            Send = ((np.exp(mu * (Lam[b, -1, h] - Lam[b, :, h])) * beta[b])[:, None, None]
                    * a["x"][b, :, h, :][:, :, None] * Bc[b, :, g, :][:, None, :]).sum(0)
            if a["h0"] is not None:
                h0c = a["h0"][b, h, :, :, 0] + 1j * a["h0"][b, h, :, :, 1]
                yy += ((np.exp(mu * Lam[b, :, h])[:, None] * Cc[b, :, g, :]) @ h0c.T).real
                Send += np.exp(mu * Lam[b, -1, h]) * h0c
            y[b, :, h, :] = yy + a["D"][h] * a["x"][b, :, h, :]
            hf[b, h] = Send
    return y, np.stack([hf.real, hf.imag], -1)


@pytest.mark.parametrize("flags", [oracle.CPLX_STABLE | oracle.BBAR_ZOH, oracle.CPLX_STABLE | oracle.BBAR_DT,
                                   oracle.CPLX_DOC | oracle.BBAR_ZOH, oracle.CPLX_CODE,
                                   oracle.CPLX_STABLE | oracle.CPLX_CONJ_C])
def test_cssd_matches_brute_force(flags):
    i = synth.cssd_inputs(2, 21, 4, 3, 4, 2, seed=(31,), h0=True)
    y, hf = oracle.cssd_fwd(**i.arrays, ngroups=2, flags=flags)
    ye, he = _cssd_brute(i, flags)
    np.testing.assert_allclose(y, ye, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(hf, he, rtol=1e-10, atol=1e-10)


def test_cssd_zero_phase_real_inputs_reduce_to_real_ssd():
    i = synth.cssd_inputs(2, 30, 3, 4, 5, 1, seed=(32,), h0=True, phase=False)
    a = dict(i.arrays)
    a["B"] = a["B"].copy(); a["B"][..., 1] = 0.0
    a["C"] = a["C"].copy(); a["C"][..., 1] = 0.0
    a["h0"] = a["h0"].copy(); a["h0"][..., 1] = 0.0
    yc, hc = oracle.cssd_fwd(**a, flags=oracle.CPLX_STABLE | oracle.BBAR_ZOH)
    yr, hr = oracle.ssd_fwd(a["x"], a["dt"], a["dt_bias"], a["A_log"][:, 0].copy(), a["B"][..., 0].copy(),
                            a["C"][..., 0].copy(), a["D"], h0=a["h0"][..., 0].copy(), flags=oracle.BBAR_ZOH)
    np.testing.assert_allclose(yc, yr, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(hc[..., 0], hr, rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(hc[..., 1], 0.0)


def test_cssd_one_step_closed_form():
    i = synth.cssd_inputs(1, 1, 2, 3, 4, 1, seed=(33,))
    a = i.arrays
    y, _ = oracle.cssd_fwd(**a)
    delta = np.logaddexp(0.0, a["dt"][0, 0].astype(np.float64) + a["dt_bias"])
    lam = -np.exp(a["A_log"][:, 0].astype(np.float64)) + 1j * a["A_log"][:, 1]
    beta = np.expm1(delta * lam) / lam
    Bc = a["B"][0, 0, 0, :, 0] + 1j * a["B"][0, 0, 0, :, 1]
    Cc = a["C"][0, 0, 0, :, 0] + 1j * a["C"][0, 0, 0, :, 1]
    for h in range(2):
        expect = (np.sum(Cc * beta[h] * Bc)).real * a["x"][0, 0, h] + a["D"][h] * a["x"][0, 0, h]
        np.testing.assert_allclose(y[0, 0, h], expect, rtol=1e-13)


def test_cssd_conj_flag_equals_negated_imag_c():
    i = synth.cssd_inputs(1, 15, 2, 3, 4, 1, seed=(34,))
    a = dict(i.arrays)
    y1, _ = oracle.cssd_fwd(**a, flags=oracle.CPLX_STABLE | oracle.CPLX_CONJ_C)
    a["C"] = a["C"].copy(); a["C"][..., 1] *= -1
    y2, _ = oracle.cssd_fwd(**a, flags=oracle.CPLX_STABLE)
    np.testing.assert_array_equal(y1, y2)
