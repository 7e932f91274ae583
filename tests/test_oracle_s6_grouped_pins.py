"""CPU pins of the fp64 S6 oracle with B, C per group of channels (s6_grouped_fwd), by the
shared-B oracle (s6_fwd, pinned on its own):

  * one group is the shared-B oracle;
  * every channel's output and final state equal the shared-B oracle run on that channel
    alone with its group's B, C rows, for per-channel and for coarser groups;
  * per-channel rows that are all equal give the shared-B result.
"""
import numpy as np

import oracle
import synth


def _one_channel(a, d, g):
    """Arrays of channel d alone, with B, C of group g."""
    sl = slice(d, d + 1)
    return dict(u=a["u"][:, :, sl], dt=a["dt"][:, :, sl], dt_bias=a["dt_bias"][sl], A_log=a["A_log"][sl],
                B=a["B"][:, :, g], C=a["C"][:, :, g], D=a["D"][sl],
                h0=None if a["h0"] is None else a["h0"][:, sl])


def test_one_group_is_the_shared_oracle():
    for flags in (oracle.BBAR_ZOH, oracle.BBAR_DT, oracle.BBAR_ONE):
        a = synth.s6_inputs(2, 23, 6, 5, seed=(1,), h0=True, ngroups=1, a_log="uniform").arrays
        y, hf = oracle.s6_grouped_fwd(**a, flags=flags)
        ys, hs = oracle.s6_fwd(**dict(a, B=a["B"][:, :, 0], C=a["C"][:, :, 0]), flags=flags)
        assert np.array_equal(y, ys) and np.array_equal(hf, hs)


def test_each_channel_reads_its_group():
    for Dm, G in ((6, 6), (8, 4), (9, 3)):
        a = synth.s6_inputs(2, 19, Dm, 4, seed=(2, G), h0=True, ngroups=G, a_log="uniform").arrays
        y, hf = oracle.s6_grouped_fwd(**a, flags=oracle.BBAR_ZOH)
        for d in range(Dm):
            ys, hs = oracle.s6_fwd(**_one_channel(a, d, d * G // Dm), flags=oracle.BBAR_ZOH)
            assert np.array_equal(y[:, :, d], ys[:, :, 0]), (Dm, G, d)
            assert np.array_equal(hf[:, d], hs[:, 0]), (Dm, G, d)


def test_equal_rows_give_the_shared_result():
    a = synth.s6_inputs(1, 30, 5, 6, seed=(3,), h0=True, ngroups=5).arrays
    shared = dict(a, B=a["B"][:, :, 0], C=a["C"][:, :, 0])
    a["B"] = np.repeat(shared["B"][:, :, None], 5, axis=2)
    a["C"] = np.repeat(shared["C"][:, :, None], 5, axis=2)
    y, hf = oracle.s6_grouped_fwd(**a)
    ys, hs = oracle.s6_fwd(**shared)
    assert np.array_equal(y, ys) and np.array_equal(hf, hs)


# ---- the backward (s6_grouped_bwd), by the shared-B backward oracle on one-channel slices

GR = ("du", "ddt", "dB", "dC", "dA_log", "dD", "ddt_bias", "dh0")


def _cot(a, seed):
    rng = np.random.default_rng(seed)
    batch, L, Dm = a["u"].shape
    N = a["A_log"].shape[1]
    return (rng.standard_normal((batch, L, Dm)).astype(np.float32),
            rng.standard_normal((batch, Dm, N)).astype(np.float32))


def test_backward_one_group_is_the_shared_oracle():
    for flags in (oracle.BBAR_ZOH, oracle.BBAR_DT, oracle.BBAR_ONE):
        a = synth.s6_inputs(2, 21, 6, 5, seed=(11,), h0=True, ngroups=1, a_log="uniform").arrays
        dy, dhf = _cot(a, 1)
        g = oracle.s6_grouped_bwd(**a, dy=dy, dh_final=dhf, flags=flags)
        s = oracle.s6_bwd(**dict(a, B=a["B"][:, :, 0], C=a["C"][:, :, 0]), dy=dy, dh_final=dhf, flags=flags)
        for k in GR:
            ref = s[k][:, :, None] if k in ("dB", "dC") else s[k]
            assert np.array_equal(g[k], ref), (flags, k)


def test_backward_per_channel_and_groups_by_slices():
    for Dm, G in ((6, 6), (8, 4), (9, 3)):
        a = synth.s6_inputs(2, 17, Dm, 4, seed=(12, G), h0=True, ngroups=G, a_log="uniform").arrays
        dy, dhf = _cot(a, 2)
        g = oracle.s6_grouped_bwd(**a, dy=dy, dh_final=dhf)
        dBsum = np.zeros_like(g["dB"])
        dCsum = np.zeros_like(g["dC"])
        for d in range(Dm):
            gi = d * G // Dm
            one = _one_channel(a, d, gi)
            s = oracle.s6_bwd(**one, dy=dy[:, :, d:d + 1], dh_final=dhf[:, d:d + 1])
            for k in ("du", "ddt"):
                np.testing.assert_allclose(g[k][:, :, d], s[k][:, :, 0], rtol=1e-12, atol=1e-14)
            for k in ("dA_log", "dD", "ddt_bias"):
                np.testing.assert_allclose(g[k][d], s[k][0], rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(g["dh0"][:, d], s["dh0"][:, 0], rtol=1e-12, atol=1e-14)
            dBsum[:, :, gi] += s["dB"]
            dCsum[:, :, gi] += s["dC"]
        np.testing.assert_allclose(g["dB"], dBsum, rtol=1e-10, atol=1e-12 * np.abs(dBsum).max())
        np.testing.assert_allclose(g["dC"], dCsum, rtol=1e-10, atol=1e-12 * np.abs(dCsum).max())
