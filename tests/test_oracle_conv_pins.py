"""CPU pins of the fp64 causal depthwise conv1d oracle (numpy, no shared code with the C
layer oracle):

  * every channel against numpy's convolve (a library routine), with and without a state;
  * with SiLU, against the separately written C layer oracle's scan input u;
  * two calls carrying the state equal one call, and a call shorter than K - 1 keeps the
    old state's tail;
  * a hand case with small integers (exact).
"""
import numpy as np
from scipy.special import expit

import oracle
import synth


def _inp(seed, batch=2, L=17, Dc=6, K=4):
    rng = np.random.default_rng(800 + seed)
    f = np.float32
    return (rng.standard_normal((batch, L, Dc)).astype(f), rng.normal(0, 0.5, (Dc, K)).astype(f),
            rng.normal(0, 0.2, (Dc,)).astype(f), rng.standard_normal((batch, Dc, K - 1)).astype(f))


def test_against_numpy_convolve():
    x, w, b, st = _inp(1)
    for state in (None, st):
        y, so = oracle.causal_conv1d(x, w, b, state)
        K, L = w.shape[1], x.shape[1]
        for bb in range(x.shape[0]):
            for c in range(x.shape[2]):
                prev = state[bb, c].astype(np.float64) if state is not None else np.zeros(K - 1)
                full = np.convolve(np.concatenate([prev, x[bb, :, c]]), w[c].astype(np.float64))
                np.testing.assert_allclose(y[bb, :, c], full[K - 1:K - 1 + L] + b[c], rtol=1e-13, atol=1e-14)
        np.testing.assert_array_equal(so, np.transpose(x[:, -(K - 1):, :], (0, 2, 1)))


def test_silu_against_the_c_layer_oracle():
    inp = synth.layer_inputs(2, 21, 5, 4, 4, seed=(9,))
    a = inp.arrays
    _, _, u, cs = oracle.s6_layer_fwd(a["x"], a["conv_w"], a["conv_b"], a["dt"], a["dt_bias"], a["A_log"],
                                      a["B"], a["C"], a["D"], None, a["conv_state"], None)
    y, so = oracle.causal_conv1d(a["x"], a["conv_w"], a["conv_b"], a["conv_state"], silu=True)
    np.testing.assert_allclose(y, u, rtol=1e-13, atol=1e-15)
    np.testing.assert_array_equal(so, cs)
    pre, _ = oracle.causal_conv1d(a["x"], a["conv_w"], a["conv_b"], a["conv_state"])
    np.testing.assert_allclose(y, pre * expit(pre), rtol=1e-13, atol=1e-15)


def test_state_carry_and_short_calls():
    x, w, b, st = _inp(2, L=15)
    y, so = oracle.causal_conv1d(x, w, b, st)
    y1, s1 = oracle.causal_conv1d(x[:, :6], w, b, st)
    y2, s2 = oracle.causal_conv1d(x[:, 6:], w, b, s1.astype(np.float32))
    np.testing.assert_array_equal(np.concatenate([y1, y2], 1), y)
    np.testing.assert_array_equal(s2, so)
    _, s_short = oracle.causal_conv1d(x[:, :2], w, b, st)       # L = 2 < K - 1 = 3
    np.testing.assert_array_equal(s_short, np.concatenate([st[:, :, 2:], np.transpose(x[:, :2], (0, 2, 1))], 2))


def test_hand_case():
    x = np.array([[[1.0], [2.0], [3.0]]], np.float32)          # (1, 3, 1)
    w = np.array([[10.0, 100.0, 1000.0]], np.float32)          # tap k multiplies x[t-k]
    st = np.array([[[4.0, 5.0]]], np.float32)                  # x[-2] = 4, x[-1] = 5
    y, so = oracle.causal_conv1d(x, w, np.array([0.5], np.float32), st)
    # t=0: 10*1 + 100*5 + 1000*4;  t=1: 10*2 + 100*1 + 1000*5;  t=2: 10*3 + 100*2 + 1000*1
    np.testing.assert_array_equal(y[0, :, 0], [4510.5, 5120.5, 1230.5])
    np.testing.assert_array_equal(so[0, 0], [2.0, 3.0])
