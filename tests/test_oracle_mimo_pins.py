"""CPU pins of the fp64 multi-input multi-output complex SSD oracle (cssd_mimo_fwd), by
things it does not compute itself:

  * rank 1 is the complex SSD oracle (cssd_fwd, pinned on its own), for every input
    scale and both C conventions;
  * superposition: rank-R outputs are sums of single-input complex SSD runs, one per
    (input rank r, output rank r') pair with (x^r, B^r, C^r'), plus the entering
    state's run through C^r' and the skip term D x^r';
  * a numpy brute force in complex128 with causality at whole-step granularity (every
    input of step t reaches every output of step t);
  * relabelling the ranks relabels the outputs; two calls carrying the state equal one.
"""
import numpy as np

import oracle
import synth


def _inp(seed, batch=2, L=17, R=3, H=2, P=4, Nc=3, G=1, h0=True):
    return dict(synth.mimo_inputs(batch, L, R, H, P, Nc, G, seed=(seed,), h0=h0).arrays)


def _rank1(a, r_in, r_out):
    """Single-input arrays taking input rank r_in and output rank r_out."""
    return dict(a, x=a["x"][:, :, r_in], B=a["B"][:, :, r_in], C=a["C"][:, :, r_out])


def test_rank_one_is_the_complex_ssd():
    for flags in (oracle.BBAR_ZOH, oracle.BBAR_DT, oracle.BBAR_ONE, oracle.BBAR_ZOH | oracle.CPLX_CONJ_C):
        a = _inp(1, R=1, G=2, H=4)
        y, hf = oracle.cssd_mimo_fwd(**a, ngroups=2, flags=flags)
        ys, hs = oracle.cssd_fwd(**_rank1(a, 0, 0), ngroups=2, flags=flags)
        np.testing.assert_allclose(y[:, :, 0], ys, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(hf, hs, rtol=1e-13, atol=1e-13)


def test_superposition_of_single_input_runs():
    a = _inp(2, R=3)
    y, hf = oracle.cssd_mimo_fwd(**a)
    R = a["x"].shape[2]
    zero = np.zeros_like(a["x"][:, :, 0])
    scale = np.abs(y).max()
    for ro in range(R):
        ref = np.zeros_like(y[:, :, ro])
        for ri in range(R):
            s = _rank1(a, ri, ro)
            s["h0"], s["D"] = None, None
            ref += oracle.cssd_fwd(**s)[0]
        s = _rank1(a, 0, ro)                       # the entering state alone
        s["x"], s["D"] = zero, None
        ref += oracle.cssd_fwd(**s)[0]
        ref += a["D"][None, None, :, None].astype(np.float64) * a["x"][:, :, ro].astype(np.float64)
        np.testing.assert_allclose(y[:, :, ro], ref, rtol=1e-11, atol=1e-12 * scale)
    # the final state: the sum of the per-rank states plus the decayed entering state
    hsum = np.zeros_like(hf)
    for ri in range(R):
        s = _rank1(a, ri, 0)
        s["h0"] = None
        hsum += oracle.cssd_fwd(**s)[1]
    s = _rank1(a, 0, 0)
    s["x"] = zero
    hsum += oracle.cssd_fwd(**s)[1]
    np.testing.assert_allclose(hf, hsum, rtol=1e-11, atol=1e-12 * np.abs(hf).max())


def _brute(a):
    """y from the materialised step-causal operator, complex128."""
    x, dt, bias, A_log, B, C, D, h0 = (a[k] for k in ("x", "dt", "dt_bias", "A_log", "B", "C", "D", "h0"))
    batch, L, R, H, P = x.shape
    G, Nc = B.shape[3], B.shape[4]
    Bc = B[..., 0].astype(np.float64) + 1j * B[..., 1]
    Cc = C[..., 0].astype(np.float64) + 1j * C[..., 1]
    y = np.zeros((batch, L, R, H, P))
    for b in range(batch):
        for h in range(H):
            g = h * G // H
            lam = -np.exp(np.float64(A_log[h, 0])) + 1j * np.float64(A_log[h, 1])
            raw = dt[b, :, h].astype(np.float64) + np.float64(bias[h])
            delta = np.logaddexp(0.0, raw)                     # softplus
            w = delta * lam
            beta = np.expm1(w) / lam                           # delta * phi1(delta lam)
            cum = np.cumsum(delta)
            T = np.arange(L)
            dec = np.exp(lam * (cum[:, None] - cum[None, :])) * (T[None, :] <= T[:, None])
            M = dec * beta[None, :]                            # (t, s)
            u = np.einsum("srn,srp->snp", Bc[b, :, :, g], x[b, :, :, h].astype(np.float64))
            S = np.einsum("ts,snp->tnp", M, u)
            if h0 is not None:
                h0c = h0[b, h, :, :, 0].astype(np.float64) + 1j * h0[b, h, :, :, 1]
                S += np.exp(lam * cum)[:, None, None] * h0c.T[None]
            out = np.einsum("trn,tnp->trp", Cc[b, :, :, g], S).real
            y[b, :, :, h] = out + np.float64(D[h]) * x[b, :, :, h]
    return y


def test_brute_force_step_causal_operator():
    for seed, kw in ((3, {}), (4, dict(R=4, H=3, G=3, L=9)), (5, dict(R=2, h0=False, L=25))):
        a = _inp(seed, **kw)
        y, _ = oracle.cssd_mimo_fwd(**a, ngroups=a["B"].shape[3])
        np.testing.assert_allclose(y, _brute(a), rtol=1e-9, atol=1e-10 * np.abs(y).max())


def test_rank_relabelling():
    a = _inp(6, R=4)
    y, hf = oracle.cssd_mimo_fwd(**a)
    perm = np.array([2, 0, 3, 1])
    b = dict(a, x=a["x"][:, :, perm], B=a["B"][:, :, perm], C=a["C"][:, :, perm])
    y2, hf2 = oracle.cssd_mimo_fwd(**b)
    np.testing.assert_allclose(y2, y[:, :, perm], rtol=1e-12, atol=1e-13 * np.abs(y).max())
    np.testing.assert_allclose(hf2, hf, rtol=1e-12, atol=1e-13 * np.abs(hf).max())


def test_two_calls_carry_the_state():
    a = _inp(7, L=30)
    y, hf = oracle.cssd_mimo_fwd(**a)
    c = 11
    seq = ("x", "dt", "B", "C")
    a1 = {k: (v[:, :c] if k in seq else v) for k, v in a.items()}
    y1, h1 = oracle.cssd_mimo_fwd(**a1)
    a2 = {k: (v[:, c:] if k in seq else v) for k, v in a.items()}
    a2["h0"] = h1.astype(np.float32)                 # rounded to fp32 between the calls
    y2, h2 = oracle.cssd_mimo_fwd(**a2)
    np.testing.assert_allclose(np.concatenate([y1, y2], 1), y, rtol=1e-5, atol=1e-6 * np.abs(y).max())
    np.testing.assert_allclose(h2, hf, rtol=1e-5, atol=1e-6 * np.abs(hf).max())
