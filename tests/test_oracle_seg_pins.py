"""Pins of the oracle's segmented S6 scan (the associative carry of the recurrence,
builderforce-memory-engine selective_scan.js forward_scan, with the composition order
of reading R6): it must equal the plain sequential recurrence for every segment length,
its segment decay must be the closed form exp(A * sum of delta), and the page's printed
combine must not equal the recurrence."""
import numpy as np
import pytest

import oracle
import synth

ZOH, DT, ONE = oracle.BBAR_ZOH, oracle.BBAR_DT, oracle.BBAR_ONE


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / np.max(np.abs(b)))


@pytest.mark.parametrize("flags", [ZOH, DT, ONE])
@pytest.mark.parametrize("seg_len", [1, 7, 64, 150, 400])
def test_segmented_equals_sequential(flags, seg_len):
    inp = synth.s6_inputs(2, 150, 6, 5, seed=(61, seg_len), h0=True, a_log="uniform")
    ys, hs = oracle.s6_fwd(**inp.arrays, flags=flags)
    yg, hg = oracle.s6_segmented_fwd(**inp.arrays, flags=flags, seg_len=seg_len)
    assert _rel(yg, ys) < 1e-12 and _rel(hg, hs) < 1e-12


def test_segment_decay_is_the_closed_form():
    # the product of a segment's Abar equals exp(A * sum of its deltas)
    inp = synth.s6_inputs(1, 40, 3, 4, seed=(62,), a_log="uniform")
    a = inp.arrays
    Abar, _ = oracle._s6_coeffs_np(a["u"], a["dt"], a["dt_bias"], a["A_log"], a["B"], ZOH)
    x = a["dt"].astype(np.float64) + a["dt_bias"].astype(np.float64)
    delta = np.array([[[oracle.softplus(v) for v in row] for row in b] for b in x])
    A = -np.exp(a["A_log"].astype(np.float64))
    prod = np.prod(Abar[0, 5:29], axis=0)
    closed = np.exp(delta[0, 5:29].sum(0)[:, None] * A)
    assert np.max(np.abs(prod / closed - 1)) < 1e-13


def test_page_combine_is_not_the_recurrence():
    # the printed combine (P1 P2, P1 c2 + c1) applies the earlier decay to the later input:
    # with three or more segments of different decays it departs from the recurrence
    inp = synth.s6_inputs(1, 96, 4, 4, seed=(63,), h0=True, a_log="uniform")
    ys, hs = oracle.s6_fwd(**inp.arrays)
    yp, hp = oracle.s6_segmented_fwd(**inp.arrays, seg_len=16, order="page")
    assert _rel(hp, hs) > 1e-3 and _rel(yp, ys) > 1e-3
