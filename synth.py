"""Seeded synthetic inputs for the scan workloads -- shared by the tests, the
benchmark and the smoke check.

This module only draws random numbers (numpy PCG64 streams keyed by a
(workload, tensor) pair) and rounds them to the input dtype; it holds none of
the scan arithmetic.  Every array is returned as float32 holding the exact
values the device will see (bf16 inputs are rounded to nearest-even first), so
the same arrays feed the fp64 oracle and, converted, the GPU.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# Workloads.  Distributions: N(m, s) has standard deviation s; complex parts
# "N(0, 1/2)" have variance 1/2 (standard complex normal).
WORKLOADS = {
    # S6 tiny: 1 x 64 x 16, N=4, fp32
    "s6_tiny": dict(kind="s6", batch=1, L=64, d_inner=16, d_state=4, dtype="f32",
                    dt_bias="zero", D="one"),
    # S6 at a Mamba-1 layer shape: 8 x 2048 x 1536, N=16, fp32
    "s6_mamba1": dict(kind="s6", batch=8, L=2048, d_inner=1536, d_state=16, dtype="f32",
                      dt_bias="uniform", D="normal"),
    # that scan at long context for one sequence: 1 x 32768 x 1536, N=16 (the segmented scan)
    "s6_long": dict(kind="s6", batch=1, L=32768, d_inner=1536, d_state=16, dtype="f32",
                    dt_bias="uniform", D="normal"),
    # that scan with B, C per channel (d_inner groups of one): 16x the B/C bytes
    "s6_pc_mamba1": dict(kind="s6", batch=8, L=2048, d_inner=1536, d_state=16, dtype="f32",
                         dt_bias="uniform", D="normal", ngroups=1536),
    # the Mamba-1 layer around that scan: conv1d (K=4) + SiLU before, SiLU(z) gating after
    "s6_layer_mamba1": dict(kind="s6_layer", batch=8, L=2048, d_inner=1536, d_state=16, d_conv=4,
                            dtype="f32"),
    # one decode step of that layer for a serving batch of 64: L = 1, state carried in place
    "s6_decode_mamba1": dict(kind="s6_layer", batch=64, L=1, d_inner=1536, d_state=16, d_conv=4,
                             dtype="f32"),
    # SSD at a Mamba-2 layer shape: 8 x 4096, 24 heads x 64, N=128, G=1, Q=256, bf16
    "ssd_mamba2": dict(kind="ssd", batch=8, L=4096, nheads=24, headdim=64, d_state=128, ngroups=1,
                       chunk_len=256, dtype="bf16"),
    # SSD long context: 2 x 32768, 80 heads x 64, N=128, G=8, Q=256, bf16, with final state
    "ssd_long": dict(kind="ssd", batch=2, L=32768, nheads=80, headdim=64, d_state=128, ngroups=8,
                     chunk_len=256, dtype="bf16"),
    # one decode step of that layer for a serving batch of 64: L = 1, state carried in place
    "ssd_decode_mamba2": dict(kind="ssd", batch=64, L=1, nheads=24, headdim=64, d_state=128, ngroups=1,
                              chunk_len=256, dtype="bf16", carry=True),
    # the Mamba-2 layer's causal conv (K=4) + SiLU over x, B, C (1536 + 2 x 128 channels)
    "conv_mamba2": dict(kind="conv", batch=8, L=4096, channels=1792, d_conv=4, dtype="bf16", silu=True),
    # Mamba-3 trapezoidal SSD: 4 x 8192, 32 heads x 64, N=128, per-head k/q, Q=64, bf16
    "trap_mamba3": dict(kind="trap", batch=4, L=8192, nheads=32, headdim=64, d_state=128,
                        chunk_len=64, dtype="bf16"),
    # one decode step of the trapezoidal layer for a serving batch of 64 (state and the
    # previous x, k carried)
    "trap_decode_mamba3": dict(kind="trap", batch=64, L=1, nheads=32, headdim=64, d_state=128,
                               chunk_len=64, dtype="bf16", carry=True),
    # Mamba-3 rotation of k and q ahead of that scan: 64 angles (every pair of N=128 turns)
    "trap_rot_mamba3": dict(kind="trap_rot", batch=4, L=8192, nheads=32, headdim=64, d_state=128,
                            n_angles=64, chunk_len=64, dtype="bf16"),
    # complex-state SSD: 4 x 8192, 32 heads x 64, 32 complex states, Q=64, fp32
    "cssd_mamba3": dict(kind="cssd", batch=4, L=8192, nheads=32, headdim=64, n_complex=32,
                        ngroups=1, chunk_len=64, dtype="f32"),
    # its multi-input multi-output form: rank 4 (4 inputs and outputs per head and step)
    "cssd_mimo_mamba3": dict(kind="cssd_mimo", batch=4, L=4096, rank=4, nheads=32, headdim=64,
                             n_complex=32, ngroups=1, chunk_len=64, dtype="f32"),
}


def _rng(key, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng([*key, tensor_id])


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest-even), returned as float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32)
    nan = np.isnan(a)
    if nan.any():
        out = out.copy()
        out[nan] = np.nan
    return out.reshape(a.shape)


def _normal(rng, shape, mean=0.0, sd=1.0):
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if sd != 1.0:
        a *= np.float32(sd)
    if mean != 0.0:
        a += np.float32(mean)
    return a


def _uniform(rng, shape, lo, hi):
    return rng.uniform(lo, hi, size=shape).astype(np.float32)


@dataclass
class Inputs:
    kind: str
    dims: dict
    arrays: dict = field(default_factory=dict)   # name -> float32 ndarray (exact device values)
    bf16: tuple = ()                              # names whose device dtype is bfloat16

    def torch(self, device):
        """Device tensors (bf16 where the workload says so, fp32 otherwise)."""
        import torch
        out = {}
        for k, v in self.arrays.items():
            if v is None:
                out[k] = None
                continue
            t = torch.from_numpy(v)
            if k in self.bf16:
                t = t.to(torch.bfloat16)     # exact: values are already bf16-representable
            out[k] = t.to(device).contiguous()
        return out


def s6_inputs(batch, L, d_inner, d_state, *, seed=(0,), dtype="f32", dt_bias="uniform",
              D="normal", h0=False, a_log="index", ngroups=None) -> Inputs:
    """ngroups: B, C (batch, L, ngroups, d_state) per group of channels (d_inner: per
    channel) instead of one shared (batch, L, d_state)."""
    key = (1, *seed)
    u = _normal(_rng(key, 0), (batch, L, d_inner))
    dt = _normal(_rng(key, 1), (batch, L, d_inner), -3.0, 0.5)
    bshape = (batch, L, d_state) if ngroups is None else (batch, L, ngroups, d_state)
    B = _normal(_rng(key, 2), bshape)
    C = _normal(_rng(key, 3), bshape)
    if dt_bias == "uniform":
        bias = _uniform(_rng(key, 4), (d_inner,), -1.0, 0.0)
    elif dt_bias == "zero":
        bias = np.zeros((d_inner,), np.float32)
    else:
        bias = None
    if D == "normal":
        Dv = _normal(_rng(key, 5), (d_inner,), 1.0, 0.1)
    elif D == "one":
        Dv = np.ones((d_inner,), np.float32)
    else:
        Dv = None
    if a_log == "index":   # A_log[d, n] = log(n + 1), so A = -(n + 1)
        A_log = np.broadcast_to(np.log(np.arange(1, d_state + 1, dtype=np.float32)),
                                (d_inner, d_state)).astype(np.float32).copy()
    elif a_log == "uniform":
        A_log = _uniform(_rng(key, 6), (d_inner, d_state), 0.0, math.log(16.0))
    else:
        A_log = np.full((d_inner, d_state), float(a_log), np.float32)
    h0a = _normal(_rng(key, 7), (batch, d_inner, d_state)) if h0 else None
    bf = ()
    if dtype == "bf16":
        u, B, C = round_bf16(u), round_bf16(B), round_bf16(C)
        bf = ("u", "B", "C")
    dims = dict(batch=batch, L=L, d_inner=d_inner, d_state=d_state)
    if ngroups is not None:
        dims["ngroups"] = ngroups
    return Inputs("s6", dims, dict(u=u, dt=dt, dt_bias=bias, A_log=A_log, B=B, C=C, D=Dv, h0=h0a), bf)


def layer_inputs(batch, L, d_inner, d_state, d_conv=4, *, seed=(0,), dtype="f32", conv_state=True,
                 gate=True, h0=False) -> Inputs:
    """The Mamba-1 layer around the scan: s6_inputs with u renamed x (the conv's input),
    plus conv_w, conv_b ~ U(-1/sqrt(K), 1/sqrt(K)) (a depthwise conv's default init),
    conv_state (batch, d_inner, K-1) ~ N(0, 1) and the gate z ~ N(0, 1)."""
    inp = s6_inputs(batch, L, d_inner, d_state, seed=seed, dtype=dtype, h0=h0)
    a = dict(inp.arrays)
    key = (7, *seed)
    bound = 1.0 / math.sqrt(d_conv)
    a["x"] = a.pop("u")
    a["conv_w"] = _uniform(_rng(key, 0), (d_inner, d_conv), -bound, bound)
    a["conv_b"] = _uniform(_rng(key, 1), (d_inner,), -bound, bound)
    a["conv_state"] = _normal(_rng(key, 2), (batch, d_inner, d_conv - 1)) if conv_state and d_conv > 1 else None
    z = _normal(_rng(key, 3), (batch, L, d_inner)) if gate else None
    if z is not None and dtype == "bf16":
        z = round_bf16(z)
    a["z"] = z
    bf = tuple("x" if n == "u" else n for n in inp.bf16) + (("z",) if dtype == "bf16" else ())
    return Inputs("s6_layer", dict(inp.dims, d_conv=d_conv), a, bf)


def conv_inputs(batch, L, channels, d_conv=4, *, seed=(0,), dtype="bf16", state=True) -> Inputs:
    """Causal conv1d inputs: x ~ N(0, 1) (rounded to bf16 when dtype is bf16), w, bias ~
    U(-1/sqrt(K), 1/sqrt(K)), the carried state ~ N(0, 1) (fp32, holding bf16 values when x is
    bf16, as a state carried from earlier inputs would)."""
    key = (8, *seed)
    bound = 1.0 / math.sqrt(d_conv)
    x = _normal(_rng(key, 0), (batch, L, channels))
    st = _normal(_rng(key, 3), (batch, channels, d_conv - 1)) if state and d_conv > 1 else None
    if dtype == "bf16":
        x = round_bf16(x)
        st = None if st is None else round_bf16(st)
    return Inputs("conv", dict(batch=batch, L=L, channels=channels, d_conv=d_conv),
                  dict(x=x, w=_uniform(_rng(key, 1), (channels, d_conv), -bound, bound),
                       bias=_uniform(_rng(key, 2), (channels,), -bound, bound), state=st),
                  ("x",) if dtype == "bf16" else ())


def s6_cotangents(batch, L, d_inner, d_state, *, seed=(0,), dh_final=True):
    """Seeded dL/dy (batch, L, d_inner) and dL/dh_final (batch, d_inner, d_state),
    both N(0, 1) fp32, for the backward pass (dh_final None when not asked)."""
    key = (4, *seed)
    dy = _normal(_rng(key, 0), (batch, L, d_inner))
    dhf = _normal(_rng(key, 1), (batch, d_inner, d_state)) if dh_final else None
    return dy, dhf


def ssd_inputs(batch, L, nheads, headdim, d_state, ngroups, *, seed=(0,), dtype="bf16",
               h0=False, dt_bias=True, D="one") -> Inputs:
    key = (2, *seed)
    x = _normal(_rng(key, 0), (batch, L, nheads, headdim))
    dt = _normal(_rng(key, 1), (batch, L, nheads), -3.0, 0.5)
    B = _normal(_rng(key, 2), (batch, L, ngroups, d_state))
    C = _normal(_rng(key, 3), (batch, L, ngroups, d_state))
    bias = _uniform(_rng(key, 4), (nheads,), -1.0, 0.0) if dt_bias else None
    A_log = _uniform(_rng(key, 5), (nheads,), 0.0, math.log(16.0))
    if D == "one":
        Dv = np.ones((nheads,), np.float32)
    elif D == "normal":
        Dv = _normal(_rng(key, 6), (nheads,), 1.0, 0.1)
    else:
        Dv = None
    h0a = _normal(_rng(key, 7), (batch, nheads, headdim, d_state)) if h0 else None
    bf = ()
    if dtype == "bf16":
        x, B, C = round_bf16(x), round_bf16(B), round_bf16(C)
        bf = ("x", "B", "C")
    return Inputs("ssd", dict(batch=batch, L=L, nheads=nheads, headdim=headdim, d_state=d_state,
                              ngroups=ngroups),
                  dict(x=x, dt=dt, dt_bias=bias, A_log=A_log, B=B, C=C, D=Dv, h0=h0a), bf)


def cssd_inputs(batch, L, nheads, headdim, n_complex, ngroups, *, seed=(0,), h0=False,
                phase=True) -> Inputs:
    key = (3, *seed)
    x = _normal(_rng(key, 0), (batch, L, nheads, headdim))
    dt = _normal(_rng(key, 1), (batch, L, nheads), -3.0, 0.5)
    sd = np.float32(math.sqrt(0.5))
    B = _normal(_rng(key, 2), (batch, L, ngroups, n_complex, 2), 0.0, sd)
    C = _normal(_rng(key, 3), (batch, L, ngroups, n_complex, 2), 0.0, sd)
    bias = _uniform(_rng(key, 4), (nheads,), -1.0, 0.0)
    A_log = np.stack([_uniform(_rng(key, 5), (nheads,), -2.0, 1.0),
                      _uniform(_rng(key, 6), (nheads,), -math.pi, math.pi) if phase
                      else np.zeros((nheads,), np.float32)], axis=1).astype(np.float32)
    Dv = np.ones((nheads,), np.float32)
    h0a = _normal(_rng(key, 7), (batch, nheads, headdim, n_complex, 2), 0.0, sd) if h0 else None
    return Inputs("cssd", dict(batch=batch, L=L, nheads=nheads, headdim=headdim,
                               n_complex=n_complex, ngroups=ngroups),
                  dict(x=x, dt=dt, dt_bias=bias, A_log=A_log, B=B, C=C, D=Dv, h0=h0a), ())


def mimo_inputs(batch, L, rank, nheads, headdim, n_complex, ngroups=1, *, seed=(0,), h0=False) -> Inputs:
    """Multi-input multi-output complex SSD inputs: the complex SSD recipe with a rank
    axis on x (batch, L, rank, nheads, headdim) and on B, C (batch, L, rank, ngroups,
    n_complex, 2); B, C entries N(0, 1/2) per part, so |B_n|^2 has mean 1."""
    key = (11, *seed)
    x = _normal(_rng(key, 0), (batch, L, rank, nheads, headdim))
    dt = _normal(_rng(key, 1), (batch, L, nheads), -3.0, 0.5)
    sd = np.float32(math.sqrt(0.5))
    B = _normal(_rng(key, 2), (batch, L, rank, ngroups, n_complex, 2), 0.0, sd)
    C = _normal(_rng(key, 3), (batch, L, rank, ngroups, n_complex, 2), 0.0, sd)
    bias = _uniform(_rng(key, 4), (nheads,), -1.0, 0.0)
    A_log = np.stack([_uniform(_rng(key, 5), (nheads,), -2.0, 1.0),
                      _uniform(_rng(key, 6), (nheads,), -math.pi, math.pi)], axis=1).astype(np.float32)
    Dv = np.ones((nheads,), np.float32)
    h0a = _normal(_rng(key, 7), (batch, nheads, headdim, n_complex, 2), 0.0, sd) if h0 else None
    return Inputs("cssd_mimo", dict(batch=batch, L=L, rank=rank, nheads=nheads, headdim=headdim,
                                    n_complex=n_complex, ngroups=ngroups),
                  dict(x=x, dt=dt, dt_bias=bias, A_log=A_log, B=B, C=C, D=Dv, h0=h0a), ())


def trap_inputs(batch, L, nheads, headdim, d_state, *, seed=(0,), h0=False, prev=False,
                D="normal", trap="uniform") -> Inputs:
    """Mamba-3 trapezoidal inputs: dt log-uniform on [1e-3, 1e-1] (a positive step, as
    after softplus), a = -exp(U(0, log 16)) per step, trap U(0, 1) (as after a sigmoid)
    or the constant 0 / 1; x, k, q, x_prev, k_prev N(0, 1) rounded to bf16.  k and q are
    the scan's inputs (already rotated); rotation_inputs draws the angles for them."""
    key = (5, *seed)
    x = round_bf16(_normal(_rng(key, 0), (batch, L, nheads, headdim)))
    k = round_bf16(_normal(_rng(key, 1), (batch, L, nheads, d_state)))
    q = round_bf16(_normal(_rng(key, 2), (batch, L, nheads, d_state)))
    dt = np.exp(_uniform(_rng(key, 3), (batch, L, nheads), math.log(1e-3), math.log(1e-1)))
    a = -np.exp(_uniform(_rng(key, 4), (batch, L, nheads), 0.0, math.log(16.0)))
    if trap == "uniform":
        tr = _uniform(_rng(key, 5), (batch, L, nheads), 0.0, 1.0)
    else:
        tr = np.full((batch, L, nheads), float(trap), np.float32)
    Dv = _normal(_rng(key, 6), (nheads,), 1.0, 0.1) if D == "normal" else None
    h0a = _normal(_rng(key, 7), (batch, nheads, headdim, d_state)) if h0 else None
    kp = round_bf16(_normal(_rng(key, 8), (batch, nheads, d_state))) if prev else None
    xp = round_bf16(_normal(_rng(key, 9), (batch, nheads, headdim))) if prev else None
    return Inputs("trap", dict(batch=batch, L=L, nheads=nheads, headdim=headdim, d_state=d_state),
                  dict(x=x, k=k, q=q, dt=dt.astype(np.float32), a=a.astype(np.float32), trap=tr,
                       D=Dv, h0=h0a, k_prev=kp, x_prev=xp),
                  ("x", "k", "q", "k_prev", "x_prev"))


def rotation_inputs(batch, L, nheads, n_angles, *, seed=(0,), angle_state=True):
    """Angles for the Mamba-3 rotation of k and q: per-step angles U(-pi, pi) shared by the
    heads (batch, L, n_angles) and an entering angle state U(-pi, pi) (batch, nheads, n_angles)."""
    key = (6, *seed)
    ang = _uniform(_rng(key, 0), (batch, L, n_angles), -math.pi, math.pi)
    st = _uniform(_rng(key, 1), (batch, nheads, n_angles), -math.pi, math.pi) if angle_state else None
    return ang, st


def workload_inputs(name: str, seed=(0,)) -> Inputs:
    w = dict(WORKLOADS[name])
    kind = w.pop("kind")
    if kind == "s6":
        return s6_inputs(w["batch"], w["L"], w["d_inner"], w["d_state"], seed=seed,
                         dtype=w["dtype"], dt_bias=w["dt_bias"], D=w["D"], ngroups=w.get("ngroups"))
    if kind == "ssd":
        return ssd_inputs(w["batch"], w["L"], w["nheads"], w["headdim"], w["d_state"],
                          w["ngroups"], seed=seed, dtype=w["dtype"], h0=w.get("carry", False))
    if kind == "conv":
        return conv_inputs(w["batch"], w["L"], w["channels"], w["d_conv"], seed=seed, dtype=w["dtype"])
    if kind == "s6_layer":
        return layer_inputs(w["batch"], w["L"], w["d_inner"], w["d_state"], w["d_conv"], seed=seed,
                            dtype=w["dtype"], h0=True)
    if kind in ("trap", "trap_rot"):
        carry = w.get("carry", False)
        return trap_inputs(w["batch"], w["L"], w["nheads"], w["headdim"], w["d_state"], seed=seed,
                           h0=carry, prev=carry)
    if kind == "cssd_mimo":
        return mimo_inputs(w["batch"], w["L"], w["rank"], w["nheads"], w["headdim"], w["n_complex"],
                           w["ngroups"], seed=seed)
    return cssd_inputs(w["batch"], w["L"], w["nheads"], w["headdim"], w["n_complex"],
                       w["ngroups"], seed=seed)


def max_rel_err(got, ref, floor_frac=0.01) -> float:
    """Elementwise relative error with a floor of floor_frac * rms(ref):
    max |g - o| / (|o| + floor_frac * rms(o)).  (Comparison metric, not scan arithmetic.)"""
    g = np.asarray(got, dtype=np.float64)
    o = np.asarray(ref, dtype=np.float64)
    if o.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(o * o)))
    den = np.abs(o) + floor_frac * rms
    den = np.where(den == 0, 1.0, den)
    return float(np.max(np.abs(g - o) / den))
