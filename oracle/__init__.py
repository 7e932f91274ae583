"""fp64 CPU oracle for the forward selective scans -- TEST INFRASTRUCTURE.

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this module.  The product path (the HIP library and its binding)
never does, and this module imports nothing from the product package.

The arithmetic lives in ``ssm_oracle.c`` (plain C, double precision, the
sequential recurrence exactly as defined on the pages); this file only builds
and loads it and marshals numpy arrays.  Inputs are float32 (bf16 inputs are
passed as their exactly-widened float32 values); outputs are float64.

Parity status of each function (what pins it is listed in the tests):
  s6_fwd    pinned: exact-fraction hand cases, A->0 cumulative-sum limit,
            closed-form brute force, carry composition, linearity.
  s6_segmented_fwd  an internal cross-check of the associative carry (numpy):
            pinned to s6_fwd for segment lengths 1, 7, 64, L and > L, and its
            segment decay to the closed form exp(A * sum of delta); with the page's
            printed combine it departs from s6_fwd (reading R6).
  ssd_fwd   pinned: brute-force semiseparable matrix, chunked algebra,
            reduction to S6, group replication, hand case.
  cssd_fwd  pinned: reduction to the real SSD at zero phase, L=1 closed form,
            brute-force complex semiseparable matrix, conjugate-C identity.
  s6_bwd    pinned: exact adjoint identities for the inputs the outputs are
            linear in (u, B, C, D, h0) and central finite differences of
            s6_fwd for the rest (dt, dt_bias, A_log), in all beta modes.
  ssd_bwd   pinned: the same two kinds of checks against ssd_fwd (with groups
            and h0), and equality with s6_bwd on the SSD shapes that are an S6
            scan (headdim 1, one group, A shared over the states).
  trap_fwd  pinned: reduction to ssd_fwd at trap = 1, brute-force semiseparable
            matrix (diagonal gamma, off-diagonal gamma + next step's
            dt (1 - trap)), hand case, carry composition across calls.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# flag values of the library interface (restated by value)
BBAR_ZOH, BBAR_DT, BBAR_ONE = 0x0, 0x1, 0x2
CPLX_STABLE, CPLX_DOC, CPLX_CODE, CPLX_CONJ_C = 0x0, 0x4, 0x8, 0x10


def build() -> str:
    """Compile the oracle with gcc (IEEE double, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
           "-o", _LIB, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    I = ctypes.c_int64
    common = [P] * 8
    lib.oracle_s6_fwd.argtypes = common + [I, I, I, I, ctypes.c_uint32, P, I, P, P, ctypes.c_int]
    lib.oracle_ssd_fwd.argtypes = common + [I, I, I, I, I, I, ctypes.c_uint32, P, I, P, P, ctypes.c_int]
    lib.oracle_cssd_fwd.argtypes = common + [I, I, I, I, I, I, ctypes.c_uint32, P, I, P, P, ctypes.c_int]
    lib.oracle_cssd_mimo_fwd.argtypes = [P] * 8 + [I] * 7 + [ctypes.c_uint32, P, I, P, P, ctypes.c_int]
    lib.oracle_s6_bwd.argtypes = [P] * 10 + [I, I, I, I, ctypes.c_uint32, I, I, I, I] + [P] * 8 + [ctypes.c_int]
    lib.oracle_s6_grouped_bwd.argtypes = [P] * 10 + [I, I, I, I, I, ctypes.c_uint32, I, I, I, I] + [P] * 8 + \
        [ctypes.c_int]
    lib.oracle_ssd_bwd.argtypes = [P] * 10 + [I] * 6 + [ctypes.c_uint32, P, I] + [P] * 8 + [ctypes.c_int]
    lib.oracle_trap_fwd.argtypes = [P] * 10 + [I] * 5 + [P, I, P, P, ctypes.c_int]
    lib.oracle_trap_rotate.argtypes = [P] * 5 + [I] * 5 + [P] * 3
    lib.oracle_trap_bwd.argtypes = [P] * 12 + [I] * 5 + [P, I] + [P] * 10 + [ctypes.c_int]
    lib.oracle_s6_grouped_fwd.argtypes = common + [I, I, I, I, I, ctypes.c_uint32, P, I, P, P, ctypes.c_int]
    lib.oracle_s6_layer_fwd.argtypes = [P] * 12 + [I] * 5 + [ctypes.c_uint32, P, I] + [P] * 4 + [ctypes.c_int]
    for f in (lib.oracle_s6_fwd, lib.oracle_ssd_fwd, lib.oracle_cssd_fwd, lib.oracle_s6_bwd,
              lib.oracle_ssd_bwd, lib.oracle_trap_fwd):
        f.restype = None
    lib.oracle_dphi1.argtypes = [ctypes.c_double]
    lib.oracle_dphi1.restype = ctypes.c_double
    lib.oracle_softplus.argtypes = [ctypes.c_double]
    lib.oracle_softplus.restype = ctypes.c_double
    lib.oracle_phi1.argtypes = [ctypes.c_double]
    lib.oracle_phi1.restype = ctypes.c_double
    _lib = lib
    return lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _f32(a):
    if a is None:
        return None
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def softplus(x: float) -> float:
    return _load().oracle_softplus(float(x))


def phi1(z: float) -> float:
    return _load().oracle_phi1(float(z))


def dphi1(z: float) -> float:
    return _load().oracle_dphi1(float(z))


def _units(units, n0, n1):
    if units is None:
        bb, ii = np.meshgrid(np.arange(n0), np.arange(n1), indexing="ij")
        return np.ascontiguousarray(np.stack([bb.ravel(), ii.ravel()], 1).astype(np.int64)), True
    u = np.ascontiguousarray(np.asarray(units, dtype=np.int64).reshape(-1, 2))
    if u.size and (u[:, 0].min() < 0 or u[:, 0].max() >= n0 or u[:, 1].min() < 0 or u[:, 1].max() >= n1):
        raise ValueError("unit index out of range")
    return u, False


def s6_fwd(u, dt, dt_bias, A_log, B, C, D, h0=None, flags=BBAR_ZOH, units=None, nthreads=None):
    """Sequential S6 recurrence in fp64.

    u, dt: (batch, L, d_inner); dt_bias, D: (d_inner,) or None (zero);
    A_log: (d_inner, N); B, C: (batch, L, N); h0: (batch, d_inner, N) or None.
    ``units``: optional (b, d) pairs; then y is (n_units, L) and h_final
    (n_units, N).  Without units: y (batch, L, d_inner), h_final (batch, d_inner, N).
    """
    u, dt, dt_bias, A_log, B, C, D, h0 = map(_f32, (u, dt, dt_bias, A_log, B, C, D, h0))
    batch, L, Dm = u.shape
    N = A_log.shape[1]
    uu, full = _units(units, batch, Dm)
    nu = uu.shape[0]
    y = np.empty((nu, L), np.float64)
    hf = np.empty((nu, N), np.float64)
    _load().oracle_s6_fwd(_ptr(u), _ptr(dt), _ptr(dt_bias), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D),
                          _ptr(h0), batch, L, Dm, N, flags, _ptr(uu), nu, _ptr(y), _ptr(hf),
                          nthreads or default_threads())
    if full:
        return (y.reshape(batch, Dm, L).transpose(0, 2, 1).copy(), hf.reshape(batch, Dm, N))
    return y, hf


def _s6_coeffs_np(u, dt, dt_bias, A_log, B, flags):
    """Per-step decay and input of the S6 recurrence in fp64 numpy (the definitions of
    selective_scan.js softplus, discretise_A, discretise_B; readings R2-R5):
    Abar[b,t,d,n] = exp(delta A), inp[b,t,d,n] = beta B[b,t,n] u[b,t,d]."""
    x = dt.astype(np.float64) + (0.0 if dt_bias is None else dt_bias.astype(np.float64))
    delta = np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))
    A = -np.exp(A_log.astype(np.float64))
    z = delta[..., None] * A
    Abar = np.exp(z)
    mode = flags & 0x3
    if mode == BBAR_ZOH:
        zs = np.where(z == 0.0, 1.0, z)
        beta = delta[..., None] * np.where(z == 0.0, 1.0, np.expm1(zs) / zs)
    elif mode == BBAR_DT:
        beta = np.broadcast_to(delta[..., None], z.shape)
    else:
        beta = np.ones_like(z)
    inp = beta * B.astype(np.float64)[:, :, None, :] * u.astype(np.float64)[..., None]
    return Abar, inp


def s6_segmented_fwd(u, dt, dt_bias, A_log, B, C, D, h0=None, flags=BBAR_ZOH, seg_len=64,
                     order="earlier_first"):
    """The S6 recurrence computed by time segments joined with the associative carry, in
    fp64 numpy: an oracle-internal cross-check of the carry algebra the segmented kernel
    uses (the parity reference stays s6_fwd, the plain sequential recurrence).

    Each step is the affine map h -> Abar h + inp.  A segment of steps composes into one
    map (P, c): P the product of its Abar, c its final state from a zero state.  Two maps
    run one after the other compose as (P2 P1, P2 c1 + c2), the earlier one first
    (order="earlier_first").  order="page" uses the combine printed in
    builderforce-memory-engine selective_scan.js (forward_scan comment and code),
    (P1 P2, P1 c2 + c1), which applies the earlier decay to the later input -- kept to show
    that it is not the recurrence.  The entering state of every segment comes from an
    inclusive Hillis-Steele scan of (0, h0), (P_0, c_0), ... (the pairs composed in a tree,
    not a left fold), then every segment runs again from its entering state.
    Returns y (batch, L, d_inner) and h_final (batch, d_inner, N), float64."""
    u, dt, dt_bias, A_log, B, C, D, h0 = map(_f32, (u, dt, dt_bias, A_log, B, C, D, h0))
    batch, L, Dm = u.shape
    N = A_log.shape[1]
    Abar, inp = _s6_coeffs_np(u, dt, dt_bias, A_log, B, flags)
    starts = list(range(0, L, seg_len))
    # segment maps: (P, c) with c the final state from zero
    pairs = [(np.zeros((batch, Dm, N)), np.zeros((batch, Dm, N)) if h0 is None else h0.astype(np.float64))]
    for s0 in starts[:-1]:
        P = np.ones((batch, Dm, N))
        c = np.zeros((batch, Dm, N))
        for t in range(s0, min(s0 + seg_len, L)):
            c = Abar[:, t] * c + inp[:, t]
            P = P * Abar[:, t]
        pairs.append((P, c))

    def compose(e, l):   # e runs first, then l
        if order == "earlier_first":
            return (l[0] * e[0], l[0] * e[1] + l[1])
        return (e[0] * l[0], e[0] * l[1] + e[1])

    scan = list(pairs)
    k = 1
    while k < len(scan):
        scan = [scan[i] if i < k else compose(scan[i - k], scan[i]) for i in range(len(scan))]
        k *= 2
    y = np.empty((batch, L, Dm))
    Cd = C.astype(np.float64)
    Dv = np.zeros(Dm) if D is None else D.astype(np.float64)
    h = None
    for si, s0 in enumerate(starts):
        h = scan[si][1].copy()
        for t in range(s0, min(s0 + seg_len, L)):
            h = Abar[:, t] * h + inp[:, t]
            y[:, t] = np.einsum("bdn,bn->bd", h, Cd[:, t]) + Dv * u[:, t].astype(np.float64)
    return y, h


def s6_grouped_fwd(u, dt, dt_bias, A_log, B, C, D, h0=None, flags=BBAR_ZOH, units=None, nthreads=None):
    """The S6 recurrence in fp64 with B, C (batch, L, G, N) per group of channels: channel d
    reads group d * G // d_inner (G = d_inner: per channel).  Returns as s6_fwd."""
    u, dt, dt_bias, A_log, B, C, D, h0 = map(_f32, (u, dt, dt_bias, A_log, B, C, D, h0))
    batch, L, Dm = u.shape
    N = A_log.shape[1]
    G = B.shape[2]
    assert B.shape == (batch, L, G, N) and C.shape == B.shape and Dm % G == 0
    uu, full = _units(units, batch, Dm)
    nu = uu.shape[0]
    y = np.empty((nu, L), np.float64)
    hf = np.empty((nu, N), np.float64)
    _load().oracle_s6_grouped_fwd(_ptr(u), _ptr(dt), _ptr(dt_bias), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D),
                                  _ptr(h0), batch, L, Dm, N, G, flags, _ptr(uu), nu, _ptr(y), _ptr(hf),
                                  nthreads or default_threads())
    if full:
        return (y.reshape(batch, Dm, L).transpose(0, 2, 1).copy(), hf.reshape(batch, Dm, N))
    return y, hf


def s6_layer_fwd(x, conv_w, conv_b, dt, dt_bias, A_log, B, C, D, h0=None, conv_state=None, z=None,
                 flags=BBAR_ZOH, units=None, nthreads=None):
    """Causal depthwise conv1d + SiLU, the S6 scan, and SiLU(z) gating, in fp64.

    x, dt, z: (batch, L, d_inner); conv_w (d_inner, K); conv_b (d_inner,) or None;
    conv_state (batch, d_inner, K-1) or None (zeros); other inputs as s6_fwd.
    Returns y, h_final, u (the scan's input), conv_state_out: full arrays
    (batch, L, d_inner), (batch, d_inner, N), (batch, L, d_inner), (batch, d_inner, K-1),
    or per-unit arrays (n, L), (n, N), (n, L), (n, K-1) with (b, d) units."""
    x, conv_w, conv_b, conv_state, z, dt, dt_bias, A_log, B, C, D, h0 = map(
        _f32, (x, conv_w, conv_b, conv_state, z, dt, dt_bias, A_log, B, C, D, h0))
    batch, L, Dm = x.shape
    N, K = A_log.shape[1], conv_w.shape[1]
    assert conv_w.shape == (Dm, K) and K >= 1
    uu, full = _units(units, batch, Dm)
    nu = uu.shape[0]
    y = np.empty((nu, L), np.float64)
    hf = np.empty((nu, N), np.float64)
    u = np.empty((nu, L), np.float64)
    cs = np.empty((nu, max(K - 1, 1)), np.float64)
    _load().oracle_s6_layer_fwd(_ptr(x), _ptr(conv_w), _ptr(conv_b), _ptr(conv_state), _ptr(z),
                                _ptr(dt), _ptr(dt_bias), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D),
                                _ptr(h0), batch, L, Dm, N, K, flags, _ptr(uu), nu, _ptr(y), _ptr(hf),
                                _ptr(u), _ptr(cs) if K > 1 else None, nthreads or default_threads())
    cs = cs[:, :K - 1]
    if full:
        return (y.reshape(batch, Dm, L).transpose(0, 2, 1).copy(), hf.reshape(batch, Dm, N),
                u.reshape(batch, Dm, L).transpose(0, 2, 1).copy(), cs.reshape(batch, Dm, K - 1))
    return y, hf, u, cs


def causal_conv1d(x, w, b=None, state=None, silu=False):
    """Causal depthwise conv1d in fp64 (builderforce-memory-engine conv1d.ts header and
    conv1d_forward; mamba-rs 0.4.0 forward.rs F4a for the fused SiLU and the carried state):
        y[b,t,c] = bias[c] + sum_{k<K} w[c,k] x[b,t-k,c],  x[b,t',c] for t' < 0 from
        state[b,c,K-1+t'] (oldest first) or 0;  then SiLU if silu.
    x (batch, L, D); w (D, K); b (D,) or None; state (batch, D, K-1) or None.
    Returns y (batch, L, D) and the outgoing state (batch, D, K-1) (the last K-1 inputs)."""
    x, w, b, state = map(_f32, (x, w, b, state))
    batch, L, Dc = x.shape
    K = w.shape[1]
    prev = (state.astype(np.float64).transpose(0, 2, 1) if state is not None
            else np.zeros((batch, K - 1, Dc)))
    xe = np.concatenate([prev, x.astype(np.float64)], axis=1)        # times -(K-1) .. L-1
    y = np.zeros((batch, L, Dc)) + (b.astype(np.float64) if b is not None else 0.0)
    for k in range(K):             # tap k multiplies x[t - k]
        y += w[:, k].astype(np.float64) * xe[:, K - 1 - k:K - 1 - k + L, :]
    if silu:
        y = y / (1.0 + np.exp(-y))
    return y, xe[:, L:, :].transpose(0, 2, 1).copy()


def ssd_fwd(x, dt, dt_bias, A_log, B, C, D, h0=None, ngroups=1, flags=BBAR_DT, units=None,
            nthreads=None):
    """Sequential SSD (scalar A per head) recurrence in fp64.

    x: (batch, L, H, P); dt: (batch, L, H); dt_bias, A_log, D: (H,);
    B, C: (batch, L, G, N); h0: (batch, H, P, N) or None.
    Without units: y (batch, L, H, P), h_final (batch, H, P, N); with (b, h)
    units: y (n_units, L, P), h_final (n_units, P, N).
    """
    x, dt, dt_bias, A_log, B, C, D, h0 = map(_f32, (x, dt, dt_bias, A_log, B, C, D, h0))
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    assert G == ngroups
    uu, full = _units(units, batch, H)
    nu = uu.shape[0]
    y = np.empty((nu, L, P), np.float64)
    hf = np.empty((nu, P, N), np.float64)
    _load().oracle_ssd_fwd(_ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D),
                           _ptr(h0), batch, L, H, P, N, G, flags, _ptr(uu), nu, _ptr(y), _ptr(hf),
                           nthreads or default_threads())
    if full:
        return (y.reshape(batch, H, L, P).transpose(0, 2, 1, 3).copy(), hf.reshape(batch, H, P, N))
    return y, hf


def trap_fwd(x, k, q, dt, a, trap, D=None, h0=None, k_prev=None, x_prev=None, units=None,
             nthreads=None):
    """Sequential Mamba-3 trapezoidal recurrence in fp64 (per-head k, q).

    x: (batch, L, H, P); k, q: (batch, L, H, N); dt, a, trap: (batch, L, H);
    D: (H,); h0: (batch, H, P, N); k_prev: (batch, H, N); x_prev: (batch, H, P).
    Returns y (batch, L, H, P), h_final (batch, H, P, N), or per-unit arrays."""
    x, k, q, dt, a, trap, D, h0, k_prev, x_prev = map(
        _f32, (x, k, q, dt, a, trap, D, h0, k_prev, x_prev))
    batch, L, H, P = x.shape
    N = k.shape[3]
    uu, full = _units(units, batch, H)
    nu = uu.shape[0]
    y = np.empty((nu, L, P), np.float64)
    hf = np.empty((nu, P, N), np.float64)
    _load().oracle_trap_fwd(_ptr(x), _ptr(k), _ptr(q), _ptr(dt), _ptr(a), _ptr(trap), _ptr(D),
                            _ptr(h0), _ptr(k_prev), _ptr(x_prev), batch, L, H, P, N, _ptr(uu), nu,
                            _ptr(y), _ptr(hf), nthreads or default_threads())
    if full:
        return (y.reshape(batch, H, L, P).transpose(0, 2, 1, 3).copy(), hf.reshape(batch, H, P, N))
    return y, hf


def trap_rotate(k, q, angles, dt, angle_state=None):
    """Data-dependent rotation of k and q in fp64 (Mamba-3 angle accumulation + RoPE).

    k, q: (batch, L, H, N); angles: (batch, L, n_angles), 2 n_angles <= N; dt: (batch, L, H);
    angle_state: (batch, H, n_angles) or None.  Returns k', q' (batch, L, H, N) and the
    final angles (batch, H, n_angles)."""
    k, q, angles, dt, angle_state = map(_f32, (k, q, angles, dt, angle_state))
    batch, L, H, N = k.shape
    NA = angles.shape[2]
    assert 2 * NA <= N and angles.shape[:2] == (batch, L) and dt.shape == (batch, L, H)
    ko = np.empty((batch, L, H, N), np.float64)
    qo = np.empty((batch, L, H, N), np.float64)
    so = np.empty((batch, H, NA), np.float64)
    _load().oracle_trap_rotate(_ptr(k), _ptr(q), _ptr(angles), _ptr(dt), _ptr(angle_state),
                               batch, L, H, N, NA, _ptr(ko), _ptr(qo), _ptr(so))
    return ko, qo, so


def trap_bwd(x, k, q, dt, a, trap, D, h0, k_prev, x_prev, dy, dh_final=None, units=None, nthreads=None):
    """Gradients of the Mamba-3 trapezoidal recurrence (trap_fwd) in fp64.

    dy: (batch, L, H, P); dh_final: (batch, H, P, N) or None.  Without units returns a dict
    of full gradients: dx (batch, L, H, P); dk, dq (batch, L, H, N); ddt, da, dtrap
    (batch, L, H); dD (H,) (summed over the batch); dh0 (batch, H, P, N); dx_prev
    (batch, H, P); dk_prev (batch, H, N).  With (b, h) units, the per-unit pieces
    (dD per unit)."""
    x, k, q, dt, a, trap, D, h0, k_prev, x_prev, dy, dh_final = map(
        _f32, (x, k, q, dt, a, trap, D, h0, k_prev, x_prev, dy, dh_final))
    batch, L, H, P = x.shape
    N = k.shape[3]
    uu, full = _units(units, batch, H)
    nu = uu.shape[0]
    out = dict(dx=np.empty((nu, L, P)), dk=np.empty((nu, L, N)), dq=np.empty((nu, L, N)),
               ddt=np.empty((nu, L)), da=np.empty((nu, L)), dtrap=np.empty((nu, L)),
               dh0=np.empty((nu, P, N)), dx_prev=np.empty((nu, P)), dk_prev=np.empty((nu, N)),
               dD=np.empty((nu,)))
    _load().oracle_trap_bwd(_ptr(x), _ptr(k), _ptr(q), _ptr(dt), _ptr(a), _ptr(trap), _ptr(D), _ptr(h0),
                            _ptr(k_prev), _ptr(x_prev), _ptr(dy), _ptr(dh_final), batch, L, H, P, N,
                            _ptr(uu), nu, *(_ptr(out[n]) for n in ("dx", "dk", "dq", "ddt", "da", "dtrap",
                                                                    "dh0", "dx_prev", "dk_prev", "dD")),
                            nthreads or default_threads())
    if not full:
        return out
    r = lambda v, *shape: v.reshape(batch, H, *shape)
    return dict(dx=r(out["dx"], L, P).transpose(0, 2, 1, 3).copy(), dk=r(out["dk"], L, N).transpose(0, 2, 1, 3).copy(),
                dq=r(out["dq"], L, N).transpose(0, 2, 1, 3).copy(),
                ddt=r(out["ddt"], L).transpose(0, 2, 1).copy(), da=r(out["da"], L).transpose(0, 2, 1).copy(),
                dtrap=r(out["dtrap"], L).transpose(0, 2, 1).copy(), dh0=r(out["dh0"], P, N),
                dx_prev=r(out["dx_prev"], P), dk_prev=r(out["dk_prev"], N), dD=out["dD"].reshape(batch, H).sum(0))


def s6_grouped_bwd(u, dt, dt_bias, A_log, B, C, D, h0, dy, dh_final=None, flags=BBAR_ZOH, b_range=None,
                   d_range=None, nthreads=None):
    """Gradients of s6_grouped_fwd (B, C (batch, L, G, N) per group of channels) in fp64.
    Returns as s6_bwd, with dB, dC (nb, L, G, N) summed over each group's channels in the
    unit range."""
    u, dt, dt_bias, A_log, B, C, D, h0, dy, dh_final = map(
        _f32, (u, dt, dt_bias, A_log, B, C, D, h0, dy, dh_final))
    batch, L, Dm = u.shape
    N = A_log.shape[1]
    G = B.shape[2]
    assert B.shape == (batch, L, G, N) and C.shape == B.shape and Dm % G == 0
    b_lo, b_hi = b_range if b_range is not None else (0, batch)
    d_lo, d_hi = d_range if d_range is not None else (0, Dm)
    if not (0 <= b_lo < b_hi <= batch and 0 <= d_lo < d_hi <= Dm):
        raise ValueError("unit range out of bounds")
    nb, nd = b_hi - b_lo, d_hi - d_lo
    out = dict(du=np.empty((nb, L, nd)), ddt=np.empty((nb, L, nd)), dB=np.empty((nb, L, G, N)),
               dC=np.empty((nb, L, G, N)), dA_log=np.empty((nd, N)), dD=np.empty((nd,)),
               ddt_bias=np.empty((nd,)), dh0=np.empty((nb, nd, N)))
    _load().oracle_s6_grouped_bwd(_ptr(u), _ptr(dt), _ptr(dt_bias), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D),
                                  _ptr(h0), _ptr(dy), _ptr(dh_final), batch, L, Dm, N, G, flags,
                                  b_lo, b_hi, d_lo, d_hi,
                                  *(_ptr(out[k]) for k in ("du", "ddt", "dB", "dC", "dA_log", "dD", "ddt_bias",
                                                           "dh0")),
                                  nthreads or default_threads())
    return out


def ssd_bwd(x, dt, dt_bias, A_log, B, C, D, h0, dy, dh_final=None, ngroups=1, flags=BBAR_DT,
            units=None, nthreads=None):
    """Gradients of the SSD recurrence in fp64 (reverse-time chain rule of ssd_fwd).

    dy: (batch, L, H, P) = dL/dy; dh_final: (batch, H, P, N) or None.
    Without units, returns a dict of full gradients: dx (batch, L, H, P);
    dB, dC (batch, L, G, N) (summed over each group's heads); ddt (batch, L, H);
    dA_log, dD, ddt_bias (H,) (summed over the batch); dh0 (batch, H, P, N).
    With (b, h) units, returns the per-unit pieces: dx (n, L, P), dB, dC (n, L, N)
    (that head's share), ddt (n, L), dh0 (n, P, N), dA_log, dD, ddt_bias (n,).
    """
    x, dt, dt_bias, A_log, B, C, D, h0, dy, dh_final = map(
        _f32, (x, dt, dt_bias, A_log, B, C, D, h0, dy, dh_final))
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    assert G == ngroups and H % G == 0
    uu, full = _units(units, batch, H)
    nu = uu.shape[0]
    out = dict(dx=np.empty((nu, L, P)), dB=np.empty((nu, L, N)), dC=np.empty((nu, L, N)),
               ddt=np.empty((nu, L)), dh0=np.empty((nu, P, N)), dA_log=np.empty(nu),
               dD=np.empty(nu), ddt_bias=np.empty(nu))
    _load().oracle_ssd_bwd(_ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D),
                           _ptr(h0), _ptr(dy), _ptr(dh_final), batch, L, H, P, N, G, flags,
                           _ptr(uu), nu,
                           *(_ptr(out[k]) for k in ("dx", "dB", "dC", "ddt", "dh0", "dA_log", "dD",
                                                    "ddt_bias")),
                           nthreads or default_threads())
    if not full:
        return out
    hpg = H // G
    dBu = out["dB"].reshape(batch, H, L, N)
    dCu = out["dC"].reshape(batch, H, L, N)
    return dict(
        dx=out["dx"].reshape(batch, H, L, P).transpose(0, 2, 1, 3).copy(),
        dB=dBu.reshape(batch, G, hpg, L, N).sum(2).transpose(0, 2, 1, 3).copy(),
        dC=dCu.reshape(batch, G, hpg, L, N).sum(2).transpose(0, 2, 1, 3).copy(),
        ddt=out["ddt"].reshape(batch, H, L).transpose(0, 2, 1).copy(),
        dh0=out["dh0"].reshape(batch, H, P, N),
        dA_log=out["dA_log"].reshape(batch, H).sum(0),
        dD=out["dD"].reshape(batch, H).sum(0),
        ddt_bias=out["ddt_bias"].reshape(batch, H).sum(0))


def cssd_fwd(x, dt, dt_bias, A_log, B, C, D, h0=None, ngroups=1, flags=BBAR_ZOH | CPLX_STABLE,
             units=None, nthreads=None):
    """Sequential complex-state SSD recurrence in fp64.

    x: (batch, L, H, P); dt: (batch, L, H); A_log: (H, 2) = [log|A|, arg A];
    B, C: (batch, L, G, Nc, 2) interleaved (re, im); h0: (batch, H, P, Nc, 2).
    Returns y (batch, L, H, P) and h_final (batch, H, P, Nc, 2), or per-unit
    (n_units, L, P) / (n_units, P, Nc, 2) when (b, h) units are given.
    """
    x, dt, dt_bias, A_log, B, C, D, h0 = map(_f32, (x, dt, dt_bias, A_log, B, C, D, h0))
    batch, L, H, P = x.shape
    G, Nc = B.shape[2], B.shape[3]
    assert G == ngroups and B.shape[4] == 2
    uu, full = _units(units, batch, H)
    nu = uu.shape[0]
    y = np.empty((nu, L, P), np.float64)
    hf = np.empty((nu, P, Nc, 2), np.float64)
    _load().oracle_cssd_fwd(_ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D),
                            _ptr(h0), batch, L, H, P, Nc, G, flags, _ptr(uu), nu, _ptr(y), _ptr(hf),
                            nthreads or default_threads())
    if full:
        return (y.reshape(batch, H, L, P).transpose(0, 2, 1, 3).copy(),
                hf.reshape(batch, H, P, Nc, 2))
    return y, hf


def cssd_mimo_fwd(x, dt, dt_bias, A_log, B, C, D, h0=None, ngroups=1, flags=BBAR_ZOH | CPLX_STABLE,
                  units=None, nthreads=None):
    """Multi-input multi-output complex SSD in fp64 (rank R inputs and outputs per head
    sharing one complex state; the stable reading of A).

    x: (batch, L, R, H, P); dt: (batch, L, H); A_log: (H, 2); B, C: (batch, L, R, G, Nc, 2);
    h0: (batch, H, P, Nc, 2).  Returns y (batch, L, R, H, P) and h_final (batch, H, P, Nc, 2),
    or per-unit (n_units, L, R, P) / (n_units, P, Nc, 2) with (b, h) units."""
    x, dt, dt_bias, A_log, B, C, D, h0 = map(_f32, (x, dt, dt_bias, A_log, B, C, D, h0))
    batch, L, R, H, P = x.shape
    G, Nc = B.shape[3], B.shape[4]
    assert G == ngroups and B.shape[:3] == (batch, L, R) and B.shape[5] == 2
    assert (flags & (CPLX_DOC | CPLX_CODE)) == CPLX_STABLE, "the MIMO form takes the stable reading of A"
    uu, full = _units(units, batch, H)
    nu = uu.shape[0]
    y = np.empty((nu, L, R, P), np.float64)
    hf = np.empty((nu, P, Nc, 2), np.float64)
    _load().oracle_cssd_mimo_fwd(_ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D),
                                 _ptr(h0), batch, L, R, H, P, Nc, G, flags, _ptr(uu), nu, _ptr(y), _ptr(hf),
                                 nthreads or default_threads())
    if full:
        return (y.reshape(batch, H, L, R, P).transpose(0, 2, 3, 1, 4).copy(),
                hf.reshape(batch, H, P, Nc, 2))
    return y, hf


def s6_bwd(u, dt, dt_bias, A_log, B, C, D, h0, dy, dh_final=None, flags=BBAR_ZOH, b_range=None,
           d_range=None, nthreads=None):
    """Gradients of the S6 scan in fp64 (reverse-time chain rule of s6_fwd).

    dy: (batch, L, d_inner) = dL/dy; dh_final: (batch, d_inner, N) or None.
    Units are b in b_range, d in d_range (default: all); sums over b or d run
    over those ranges.  Returns a dict: du, ddt (nb, L, nd); dB, dC (nb, L, N);
    dA_log (nd, N); dD, ddt_bias (nd,); dh0 (nb, nd, N).
    """
    u, dt, dt_bias, A_log, B, C, D, h0, dy, dh_final = map(
        _f32, (u, dt, dt_bias, A_log, B, C, D, h0, dy, dh_final))
    batch, L, Dm = u.shape
    N = A_log.shape[1]
    b_lo, b_hi = b_range if b_range is not None else (0, batch)
    d_lo, d_hi = d_range if d_range is not None else (0, Dm)
    if not (0 <= b_lo < b_hi <= batch and 0 <= d_lo < d_hi <= Dm):
        raise ValueError("unit range out of bounds")
    nb, nd = b_hi - b_lo, d_hi - d_lo
    out = dict(du=np.empty((nb, L, nd)), ddt=np.empty((nb, L, nd)), dB=np.empty((nb, L, N)),
               dC=np.empty((nb, L, N)), dA_log=np.empty((nd, N)), dD=np.empty((nd,)),
               ddt_bias=np.empty((nd,)), dh0=np.empty((nb, nd, N)))
    _load().oracle_s6_bwd(_ptr(u), _ptr(dt), _ptr(dt_bias), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D),
                          _ptr(h0), _ptr(dy), _ptr(dh_final), batch, L, Dm, N, flags,
                          b_lo, b_hi, d_lo, d_hi,
                          *(_ptr(out[k]) for k in ("du", "ddt", "dB", "dC", "dA_log", "dD", "ddt_bias", "dh0")),
                          nthreads or default_threads())
    return out
