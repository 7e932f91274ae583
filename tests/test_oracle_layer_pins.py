"""CPU pins of the fp64 Mamba-1 layer oracle around the scan: causal depthwise conv1d +
SiLU before it, SiLU(z) gating after it, the carried conv state, and the decode step.

  * u against numpy's convolve and scipy's expit (with and without a carried state);
  * K = 1, w = 1, no bias: the plain S6 oracle on SiLU(x);
  * the gated output over the ungated one is SiLU(z) (scipy's expit);
  * two calls carrying (h, conv state) equal one call; the carried conv state is the
    last K-1 inputs (or the old state's tail when the call is shorter);
  * L single-step calls (decode) equal one call over L steps.
"""
import numpy as np
from scipy.special import expit

import oracle
import synth


def _layer_inputs(seed, batch=2, L=19, Dm=5, N=4, K=4, state=True):
    rng = np.random.default_rng(700 + seed)
    f = np.float32
    inp = synth.s6_inputs(batch, L, Dm, N, seed=(seed,), dtype="f32", dt_bias="uniform", D="normal")
    a = dict(inp.arrays)
    x = a.pop("u")
    return dict(x=x, conv_w=rng.normal(0, 0.5, (Dm, K)).astype(f), conv_b=rng.normal(0, 0.2, (Dm,)).astype(f),
                conv_state=rng.standard_normal((batch, Dm, K - 1)).astype(f) if state else None,
                z=rng.standard_normal((batch, L, Dm)).astype(f), **a)


def _u_ref(d):
    x, w, cb, st = d["x"].astype(np.float64), d["conv_w"].astype(np.float64), d["conv_b"], d["conv_state"]
    batch, L, Dm = x.shape
    K = w.shape[1]
    u = np.empty_like(x)
    for b in range(batch):
        for c in range(Dm):
            prev = st[b, c].astype(np.float64) if st is not None else np.zeros(K - 1)
            xe = np.concatenate([prev, x[b, :, c]])
            pre = np.convolve(xe, w[c])[K - 1:K - 1 + L] + float(cb[c])
            u[b, :, c] = pre * expit(pre)
    return u


def test_conv_silu_against_numpy_convolve():
    for state in (False, True):
        d = _layer_inputs(1, state=state)
        _, _, u, _ = oracle.s6_layer_fwd(**d)
        np.testing.assert_allclose(u, _u_ref(d), rtol=1e-12, atol=1e-14)


def test_kernel_one_is_the_scan_of_silu_x():
    d = _layer_inputs(2, K=1, state=False)
    d["conv_w"] = np.ones_like(d["conv_w"])
    d["conv_b"] = None
    z = d.pop("z")
    y, hf, u, _ = oracle.s6_layer_fwd(**d)
    x64 = d["x"].astype(np.float64)
    silu_x = (x64 * expit(x64)).astype(np.float32)
    yo, ho = oracle.s6_fwd(silu_x, d["dt"], d["dt_bias"], d["A_log"], d["B"], d["C"], d["D"], d["h0"])
    np.testing.assert_allclose(y, yo, rtol=2e-6, atol=1e-6 * np.abs(yo).max())
    np.testing.assert_allclose(hf, ho, rtol=2e-6, atol=1e-6 * np.abs(ho).max())
    assert z is not None


def test_gating_is_silu_of_z():
    d = _layer_inputs(3)
    y_g, hf_g, u_g, _ = oracle.s6_layer_fwd(**d)
    z = d.pop("z").astype(np.float64)
    y, hf, u, _ = oracle.s6_layer_fwd(**d)
    np.testing.assert_allclose(y_g, y * (z * expit(z)), rtol=1e-12, atol=1e-14)
    assert np.array_equal(hf_g, hf) and np.array_equal(u_g, u)


def test_two_calls_carry_state():
    d = _layer_inputs(4, L=23)
    y, hf, u, cs = oracle.s6_layer_fwd(**d)
    K = d["conv_w"].shape[1]
    np.testing.assert_array_equal(cs, np.transpose(d["x"][:, -(K - 1):, :], (0, 2, 1)))
    c = 9
    part = lambda a, s: None if a is None else a[:, s]
    seq = ("x", "dt", "B", "C", "z")
    d1 = {k: (part(v, slice(0, c)) if k in seq else v) for k, v in d.items()}
    y1, hf1, _, cs1 = oracle.s6_layer_fwd(**d1)
    d2 = {k: (part(v, slice(c, None)) if k in seq else v) for k, v in d.items()}
    d2["h0"], d2["conv_state"] = hf1.astype(np.float32), cs1.astype(np.float32)
    y2, hf2, _, cs2 = oracle.s6_layer_fwd(**d2)
    # h is rounded to fp32 between the calls
    np.testing.assert_allclose(np.concatenate([y1, y2], 1), y, rtol=1e-6, atol=1e-6 * np.abs(y).max())
    np.testing.assert_allclose(hf2, hf, rtol=1e-6, atol=1e-6 * np.abs(hf).max())
    np.testing.assert_array_equal(cs2, cs)


def test_short_call_keeps_the_old_state_tail():
    d = _layer_inputs(5, L=2, K=4)
    _, _, _, cs = oracle.s6_layer_fwd(**d)
    st, x = d["conv_state"], d["x"]
    ref = np.concatenate([st[:, :, 2:], np.transpose(x, (0, 2, 1))], axis=2)
    np.testing.assert_array_equal(cs, ref)


def test_decode_steps_equal_one_call():
    d = _layer_inputs(6, L=11)
    y, hf, _, cs = oracle.s6_layer_fwd(**d)
    h, st, ys = d["h0"], d["conv_state"], []
    seq = ("x", "dt", "B", "C", "z")
    for t in range(d["x"].shape[1]):
        dt_ = {k: (v[:, t:t + 1] if k in seq else v) for k, v in d.items()}
        dt_["h0"], dt_["conv_state"] = h, st
        yt, h, _, st = oracle.s6_layer_fwd(**dt_)
        h, st = h.astype(np.float32), st.astype(np.float32)
        ys.append(yt)
    np.testing.assert_allclose(np.concatenate(ys, 1), y, rtol=1e-6, atol=1e-6 * np.abs(y).max())
    np.testing.assert_allclose(h, hf, rtol=1e-6, atol=1e-6 * np.abs(hf).max())
    np.testing.assert_array_equal(st, cs)
