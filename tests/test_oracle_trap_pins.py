"""CPU pins of the fp64 Mamba-3 trapezoidal recurrence oracle (no GPU).

  * trap = 1 makes beta = 0 and gamma = dt: the SSD recurrence with input scale
    delta (checked against the separately written ssd_fwd, with ngroups = nheads);
  * a brute force from the closed form of the unrolled recurrence: y_t is the
    sum over s <= t of (q_t . k_s) x_s w_ts with
        w_ts = e^{cs_t - cs_s} gamma_s + [s < t] e^{cs_t - cs_{s+1}} beta_{s+1},
    plus the decayed h0 and the carried previous input;
  * an exact hand case (L = 1, numbers exact in binary);
  * two calls carrying (h, k_prev, x_prev) equal one call.
"""
import numpy as np

import oracle
import synth


def _inputs(seed, batch=2, L=13, H=3, P=4, N=5, prev=True, h0=True):
    rng = np.random.default_rng(1000 + seed)
    f = np.float32
    x = rng.standard_normal((batch, L, H, P)).astype(f)
    k = rng.standard_normal((batch, L, H, N)).astype(f)
    q = rng.standard_normal((batch, L, H, N)).astype(f)
    dt = rng.uniform(0.01, 0.3, (batch, L, H)).astype(f)
    a = -rng.uniform(0.2, 3.0, (batch, L, H)).astype(f)
    trap = rng.uniform(0.0, 1.0, (batch, L, H)).astype(f)
    D = rng.normal(1.0, 0.1, (H,)).astype(f)
    return dict(x=x, k=k, q=q, dt=dt, a=a, trap=trap, D=D,
                h0=rng.standard_normal((batch, H, P, N)).astype(f) if h0 else None,
                k_prev=rng.standard_normal((batch, H, N)).astype(f) if prev else None,
                x_prev=rng.standard_normal((batch, H, P)).astype(f) if prev else None)


def test_trap_one_is_the_ssd_recurrence():
    inp = synth.ssd_inputs(2, 17, 3, 4, 5, 3, seed=(71,), dtype="f32", h0=True, D="normal")
    a = inp.arrays
    y_ssd, hf_ssd = oracle.ssd_fwd(**a, ngroups=3, flags=oracle.BBAR_DT)
    # delta = softplus(dt + dt_bias), rounded to fp32 for the trapezoidal oracle's dt input
    raw = a["dt"].astype(np.float64) + a["dt_bias"].astype(np.float64)
    delta = np.array([[[oracle.softplus(v) for v in r] for r in bt] for bt in raw]).astype(np.float32)
    A = -np.exp(a["A_log"].astype(np.float64))
    aa = np.broadcast_to(A, delta.shape).astype(np.float32)
    y, hf = oracle.trap_fwd(a["x"], a["B"], a["C"], delta, aa, np.ones_like(delta), a["D"], a["h0"])
    np.testing.assert_allclose(y, y_ssd, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(hf, hf_ssd, rtol=1e-5, atol=1e-6)


def test_trap_brute_force_semiseparable():
    d = _inputs(1)
    y, hf = oracle.trap_fwd(**d)
    x, k, q = (d[n].astype(np.float64) for n in ("x", "k", "q"))
    dt, aa, tr = (d[n].astype(np.float64) for n in ("dt", "a", "trap"))
    batch, L, H, P = x.shape
    yb = np.empty_like(y)
    for b in range(batch):
        for h in range(H):
            la = aa[b, :, h] * dt[b, :, h]
            cs = np.cumsum(la)
            gam = tr[b, :, h] * dt[b, :, h]
            bet = np.exp(la) * dt[b, :, h] * (1.0 - tr[b, :, h])
            for t in range(L):
                acc = d["D"][h] * x[b, t, h]
                for s in range(t + 1):
                    w = np.exp(cs[t] - cs[s]) * gam[s]
                    if s < t:
                        w += np.exp(cs[t] - cs[s + 1]) * bet[s + 1]
                    acc = acc + (q[b, t, h] @ k[b, s, h]) * w * x[b, s, h]
                # h0 and the carried previous input enter before step 0
                acc = acc + np.exp(cs[t]) * (d["h0"][b, h].astype(np.float64) @ q[b, t, h])
                acc = acc + np.exp(cs[t] - cs[0]) * bet[0] * (q[b, t, h] @ d["k_prev"][b, h]) * \
                    d["x_prev"][b, h].astype(np.float64)
                yb[b, t, h] = acc
    np.testing.assert_allclose(y, yb, rtol=1e-11, atol=1e-12)


def test_trap_hand_case():
    f = np.float32
    one = lambda v: np.full((1, 1, 1), v, f)   # noqa: E731
    # dt = 1, a = 0: alpha = 1, beta = 1 - trap = 0.75, gamma = trap = 0.25
    y, hf = oracle.trap_fwd(x=np.full((1, 1, 1, 1), 4.0, f), k=np.full((1, 1, 1, 1), 1.0, f),
                            q=np.full((1, 1, 1, 1), 0.5, f), dt=one(1.0), a=one(0.0), trap=one(0.25),
                            D=np.full((1,), 0.5, f), h0=np.full((1, 1, 1, 1), 2.0, f),
                            k_prev=np.full((1, 1, 1), 3.0, f), x_prev=np.full((1, 1, 1), 1.0, f))
    # h = 2 + 0.75*3*1 + 0.25*1*4 = 5.25; y = 0.5*5.25 + 0.5*4 = 4.625
    assert hf[0, 0, 0, 0] == 5.25 and y[0, 0, 0, 0] == 4.625


def test_trap_carry_composition():
    d = _inputs(2, L=20)
    y, hf = oracle.trap_fwd(**d)
    m = 9
    first = {n: (v[:, :m] if n in ("x", "k", "q", "dt", "a", "trap") else v) for n, v in d.items()}
    y1, h1 = oracle.trap_fwd(**first)
    second = {n: (v[:, m:] if n in ("x", "k", "q", "dt", "a", "trap") else v) for n, v in d.items()}
    second.update(h0=h1.astype(np.float32), k_prev=d["k"][:, m - 1], x_prev=d["x"][:, m - 1])
    y2, h2 = oracle.trap_fwd(**second)
    # the carried state is rounded to fp32 between the calls
    np.testing.assert_allclose(np.concatenate([y1, y2], 1), y, rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(h2, hf, rtol=1e-6, atol=1e-6)
