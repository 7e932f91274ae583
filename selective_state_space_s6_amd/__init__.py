"""MI355X-native forward selective state-space scans (S6, SSD, complex SSD).

Thin Python binding over ``libssmscan.so`` (include/ssm_scan.h).  The functions
carry the names of the C entry points and only marshal arguments: they check
dtypes, shapes and contiguity, allocate outputs and workspace with torch (when
the caller does not pass them), and hand device pointers plus the current HIP
stream to the library.  Every step of the computation runs in the HIP kernels;
there is no fallback path: if the library is missing, importing this package
fails.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "ssm_s6_scan_fwd", "ssm_s6_scan_grouped_fwd", "ssm_s6_scan_bwd", "ssm_s6_scan_fwd_save",
    "ssm_s6_scan_bwd_saved", "ssm_s6_scan_checkpoint_size", "ssm_s6_scan_grouped_bwd",
    "ssm_s6_scan_grouped_bwd_workspace_size", "ssm_s6_fused_fwd", "ssm_causal_conv1d_fwd", "ssd_chunk_scan_fwd",
    "ssd_chunk_scan_bwd",
    "ssd_cplx_chunk_scan_fwd", "ssd_trap_chunk_scan_fwd", "ssm_s6_scan_fwd_workspace_size",
    "ssm_s6_scan_bwd_workspace_size", "ssd_trap_chunk_scan_fwd_workspace_size",
    "ssd_trap_rotate_qk", "ssd_trap_rotate_qk_workspace_size", "ssd_trap_chunk_scan_bwd",
    "ssd_trap_chunk_scan_bwd_workspace_size",
    "ssd_chunk_scan_bwd_workspace_size", "ssd_chunk_scan_fwd_workspace_size",
    "ssd_cplx_chunk_scan_fwd_workspace_size", "ssd_cplx_mimo_chunk_scan_fwd",
    "ssd_cplx_mimo_chunk_scan_fwd_workspace_size", "ssm_last_error", "SsmError", "LIB_PATH",
    "ssd_chunk_scan_fwd_noalloc",
    "SSM_BBAR_ZOH", "SSM_BBAR_DT", "SSM_BBAR_ONE", "SSM_CPLX_STABLE", "SSM_CPLX_DOC",
    "SSM_CPLX_CODE", "SSM_CPLX_CONJ_C", "SSM_F32", "SSM_BF16",
]

SSM_F32, SSM_BF16 = 0, 1
SSM_BBAR_ZOH, SSM_BBAR_DT, SSM_BBAR_ONE = 0x0, 0x1, 0x2
SSM_CPLX_STABLE, SSM_CPLX_DOC, SSM_CPLX_CODE, SSM_CPLX_CONJ_C = 0x0, 0x4, 0x8, 0x10

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libssmscan.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python selective_state_space_s6_amd/build.py` "
        "(there is no non-HIP fallback)")

_lib = ctypes.CDLL(LIB_PATH)
_P, _I, _Z = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
_lib.ssm_last_error.restype = ctypes.c_char_p
_lib.ssm_s6_scan_fwd_workspace_size.argtypes = [_I] * 4
_lib.ssm_s6_scan_fwd_workspace_size.restype = _Z
_lib.ssm_s6_scan_fwd.argtypes = [_P] * 10 + [_I] * 4 + [ctypes.c_int, ctypes.c_uint32, _P, _Z, _P]
_lib.ssm_s6_scan_fwd.restype = ctypes.c_int
_lib.ssm_s6_scan_grouped_fwd.argtypes = [_P] * 10 + [_I] * 5 + [ctypes.c_int, ctypes.c_uint32, _P]
_lib.ssm_s6_scan_grouped_fwd.restype = ctypes.c_int
_lib.ssm_s6_fused_fwd.argtypes = [_P] * 16 + [_I] * 5 + [ctypes.c_int, ctypes.c_uint32, _P]
_lib.ssm_s6_fused_fwd.restype = ctypes.c_int
_lib.ssm_causal_conv1d_fwd.argtypes = [_P] * 6 + [_I] * 4 + [ctypes.c_int, ctypes.c_int, _P]
_lib.ssm_causal_conv1d_fwd.restype = ctypes.c_int
_lib.ssm_s6_scan_bwd_workspace_size.argtypes = [_I] * 4
_lib.ssm_s6_scan_bwd_workspace_size.restype = _Z
_lib.ssm_s6_scan_bwd.argtypes = [_P] * 18 + [_I] * 4 + [ctypes.c_int, ctypes.c_uint32, _P, _Z, _P]
_lib.ssm_s6_scan_bwd.restype = ctypes.c_int
_lib.ssm_s6_scan_bwd_saved.argtypes = [_P] * 19 + [_I] * 4 + [ctypes.c_int, ctypes.c_uint32, _P, _Z, _P]
_lib.ssm_s6_scan_bwd_saved.restype = ctypes.c_int
_lib.ssm_s6_scan_fwd_save.argtypes = [_P] * 11 + [_I] * 4 + [ctypes.c_int, ctypes.c_uint32, _P]
_lib.ssm_s6_scan_fwd_save.restype = ctypes.c_int
_lib.ssm_s6_scan_grouped_bwd.argtypes = [_P] * 18 + [_I] * 5 + [ctypes.c_int, ctypes.c_uint32, _P, _Z, _P]
_lib.ssm_s6_scan_grouped_bwd.restype = ctypes.c_int
_lib.ssm_s6_scan_grouped_bwd_workspace_size.argtypes = [_I] * 5
_lib.ssm_s6_scan_grouped_bwd_workspace_size.restype = _Z
_lib.ssm_s6_scan_checkpoint_size.argtypes = [_I] * 4
_lib.ssm_s6_scan_grouped_fwd_save.argtypes = [_P] * 11 + [_I] * 5 + [ctypes.c_int, ctypes.c_uint32, _P]
_lib.ssm_s6_scan_grouped_bwd_saved.argtypes = [_P] * 19 + [_I] * 5 + [ctypes.c_int, ctypes.c_uint32, _P, _Z, _P]
_lib.ssm_s6_scan_checkpoint_size.restype = _Z
_lib.ssd_chunk_scan_fwd_workspace_size.argtypes = [_I] * 7
_lib.ssd_chunk_scan_fwd_workspace_size.restype = _Z
_lib.ssd_chunk_scan_fwd.argtypes = [_P] * 10 + [_I] * 7 + [ctypes.c_int, ctypes.c_uint32, _P, _Z, _P]
_lib.ssd_chunk_scan_fwd.restype = ctypes.c_int
_lib.ssd_chunk_scan_fwd_noalloc.argtypes = [_P] * 10 + [_I] * 7 + [ctypes.c_int, ctypes.c_uint32, _P]
_lib.ssd_chunk_scan_fwd_noalloc.restype = ctypes.c_int
_lib.ssd_chunk_scan_bwd_workspace_size.argtypes = [_I] * 7
_lib.ssd_chunk_scan_bwd_workspace_size.restype = _Z
_lib.ssd_chunk_scan_bwd.argtypes = [_P] * 18 + [_I] * 7 + [ctypes.c_int, ctypes.c_uint32, _P, _Z, _P]
_lib.ssd_chunk_scan_bwd.restype = ctypes.c_int
_lib.ssd_trap_chunk_scan_fwd_workspace_size.argtypes = [_I] * 6
_lib.ssd_trap_chunk_scan_fwd_workspace_size.restype = _Z
_lib.ssd_trap_chunk_scan_fwd.argtypes = [_P] * 12 + [_I] * 6 + [ctypes.c_int, _P, _Z, _P]
_lib.ssd_trap_chunk_scan_fwd.restype = ctypes.c_int
_lib.ssd_trap_rotate_qk_workspace_size.argtypes = [_I] * 5
_lib.ssd_trap_rotate_qk_workspace_size.restype = _Z
_lib.ssd_trap_rotate_qk.argtypes = [_P] * 8 + [_I] * 5 + [ctypes.c_int, _P, _Z, _P]
_lib.ssd_trap_rotate_qk.restype = ctypes.c_int
_lib.ssd_trap_chunk_scan_bwd_workspace_size.argtypes = [_I] * 6
_lib.ssd_trap_chunk_scan_bwd_workspace_size.restype = _Z
_lib.ssd_trap_chunk_scan_bwd.argtypes = [_P] * 22 + [_I] * 6 + [ctypes.c_int, _P, _Z, _P]
_lib.ssd_trap_chunk_scan_bwd.restype = ctypes.c_int
_lib.ssd_cplx_chunk_scan_fwd_workspace_size.argtypes = [_I] * 7
_lib.ssd_cplx_chunk_scan_fwd_workspace_size.restype = _Z
_lib.ssd_cplx_chunk_scan_fwd.argtypes = [_P] * 10 + [_I] * 7 + [ctypes.c_uint32, _P, _Z, _P]
_lib.ssd_cplx_chunk_scan_fwd.restype = ctypes.c_int
_lib.ssd_cplx_mimo_chunk_scan_fwd_workspace_size.argtypes = [_I] * 8
_lib.ssd_cplx_mimo_chunk_scan_fwd_workspace_size.restype = _Z
_lib.ssd_cplx_mimo_chunk_scan_fwd.argtypes = [_P] * 10 + [_I] * 8 + [ctypes.c_uint32, _P, _Z, _P]
_lib.ssd_cplx_mimo_chunk_scan_fwd.restype = ctypes.c_int


class SsmError(RuntimeError):
    """A library call returned a negative status; ``code`` holds it."""

    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


def ssm_last_error() -> str:
    return _lib.ssm_last_error().decode()


def _check(rc: int) -> None:
    if rc != 0:
        raise SsmError(rc, ssm_last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _req(t, name, dtype, shape, device):
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t


def _opt(t, name, dtype, shape, device):
    return None if t is None else _req(t, name, dtype, shape, device)


def _in_dtype(t):
    if t.dtype == torch.float32:
        return SSM_F32
    if t.dtype == torch.bfloat16:
        return SSM_BF16
    raise TypeError(f"input dtype {t.dtype}: expected float32 or bfloat16")


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def ssm_s6_scan_fwd_workspace_size(batch, L, d_inner, d_state) -> int:
    return int(_lib.ssm_s6_scan_fwd_workspace_size(batch, L, d_inner, d_state))


def ssm_s6_scan_bwd_workspace_size(batch, L, d_inner, d_state) -> int:
    return int(_lib.ssm_s6_scan_bwd_workspace_size(batch, L, d_inner, d_state))


def ssd_chunk_scan_fwd_workspace_size(batch, L, nheads, headdim, d_state, ngroups, chunk_len) -> int:
    return int(_lib.ssd_chunk_scan_fwd_workspace_size(batch, L, nheads, headdim, d_state, ngroups,
                                                      chunk_len))


def ssd_chunk_scan_bwd_workspace_size(batch, L, nheads, headdim, d_state, ngroups, chunk_len) -> int:
    return int(_lib.ssd_chunk_scan_bwd_workspace_size(batch, L, nheads, headdim, d_state, ngroups,
                                                      chunk_len))


def ssd_trap_chunk_scan_fwd_workspace_size(batch, L, nheads, headdim, d_state, chunk_len) -> int:
    return int(_lib.ssd_trap_chunk_scan_fwd_workspace_size(batch, L, nheads, headdim, d_state,
                                                           chunk_len))


def ssd_cplx_chunk_scan_fwd_workspace_size(batch, L, nheads, headdim, n_complex, ngroups,
                                           chunk_len) -> int:
    return int(_lib.ssd_cplx_chunk_scan_fwd_workspace_size(batch, L, nheads, headdim, n_complex,
                                                           ngroups, chunk_len))


def ssm_s6_scan_fwd(u, dt, dt_bias, A_log, B, C, D, h0=None, *, flags=SSM_BBAR_ZOH,
                    return_final=False, y=None, h_final=None, workspace="auto"):
    """S6 forward scan.  u (batch, L, d_inner) fp32|bf16; dt fp32 (same shape);
    dt_bias, D (d_inner) fp32 or None; A_log (d_inner, d_state) fp32;
    B, C (batch, L, d_state) in u's dtype; h0 (batch, d_inner, d_state) fp32 or None.
    workspace: "auto" allocates the size the library asks for (nonzero only for
    long sequences over few channels, which then take the segmented scan), None
    walks the sequence in one pass, or a uint8 device tensor.
    Returns y (fp32), or (y, h_final) when return_final."""
    dev = u.device
    batch, L, Dm = u.shape
    N = A_log.shape[1]
    dty = u.dtype
    _req(u, "u", dty, (batch, L, Dm), dev)
    _req(dt, "dt", torch.float32, (batch, L, Dm), dev)
    _opt(dt_bias, "dt_bias", torch.float32, (Dm,), dev)
    _req(A_log, "A_log", torch.float32, (Dm, N), dev)
    _req(B, "B", dty, (batch, L, N), dev)
    _req(C, "C", dty, (batch, L, N), dev)
    _opt(D, "D", torch.float32, (Dm,), dev)
    _opt(h0, "h0", torch.float32, (batch, Dm, N), dev)
    if y is None:
        y = torch.empty((batch, L, Dm), dtype=torch.float32, device=dev)
    _req(y, "y", torch.float32, (batch, L, Dm), dev)
    if return_final and h_final is None:
        h_final = torch.empty((batch, Dm, N), dtype=torch.float32, device=dev)
    _opt(h_final, "h_final", torch.float32, (batch, Dm, N), dev)
    if isinstance(workspace, str):
        ws_n = ssm_s6_scan_fwd_workspace_size(batch, L, Dm, N)
        workspace = torch.empty(ws_n, dtype=torch.uint8, device=dev) if ws_n > 0 else None
    ws_ptr, ws_n = (None, 0) if workspace is None else (_ptr(workspace), workspace.numel())
    rc = _lib.ssm_s6_scan_fwd(_ptr(u), _ptr(dt), _ptr(dt_bias), _ptr(A_log), _ptr(B), _ptr(C),
                              _ptr(D), _ptr(y), _ptr(h0), _ptr(h_final), batch, L, Dm, N,
                              _in_dtype(u), flags, ws_ptr, ws_n, _stream(dev))
    _check(rc)
    return (y, h_final) if (return_final or h_final is not None) else y


def ssm_s6_scan_grouped_fwd(u, dt, dt_bias, A_log, B, C, D, h0=None, *, flags=SSM_BBAR_ZOH,
                            return_final=False, y=None, h_final=None):
    """S6 forward scan with B, C (batch, L, ngroups, d_state) per group of channels
    (ngroups = d_inner: per channel); the rest as ssm_s6_scan_fwd."""
    dev = u.device
    batch, L, Dm = u.shape
    N = A_log.shape[1]
    G = B.shape[2]
    dty = u.dtype
    _req(u, "u", dty, (batch, L, Dm), dev)
    _req(dt, "dt", torch.float32, (batch, L, Dm), dev)
    _opt(dt_bias, "dt_bias", torch.float32, (Dm,), dev)
    _req(A_log, "A_log", torch.float32, (Dm, N), dev)
    _req(B, "B", dty, (batch, L, G, N), dev)
    _req(C, "C", dty, (batch, L, G, N), dev)
    _opt(D, "D", torch.float32, (Dm,), dev)
    _opt(h0, "h0", torch.float32, (batch, Dm, N), dev)
    if y is None:
        y = torch.empty((batch, L, Dm), dtype=torch.float32, device=dev)
    _req(y, "y", torch.float32, (batch, L, Dm), dev)
    if return_final and h_final is None:
        h_final = torch.empty((batch, Dm, N), dtype=torch.float32, device=dev)
    _opt(h_final, "h_final", torch.float32, (batch, Dm, N), dev)
    rc = _lib.ssm_s6_scan_grouped_fwd(_ptr(u), _ptr(dt), _ptr(dt_bias), _ptr(A_log), _ptr(B), _ptr(C),
                                      _ptr(D), _ptr(y), _ptr(h0), _ptr(h_final), batch, L, Dm, N, G,
                                      _in_dtype(u), flags, _stream(dev))
    _check(rc)
    return (y, h_final) if (return_final or h_final is not None) else y


def ssm_s6_fused_fwd(x, conv_w, conv_b, dt, dt_bias, A_log, B, C, D, h0=None, conv_state=None, z=None,
                     *, flags=SSM_BBAR_ZOH, return_final=False, y=None, h_final=None, u_out=None,
                     conv_state_out=None):
    """Causal conv1d + SiLU, the S6 scan and SiLU(z) gating in one pass.
    x, z (batch, L, d_inner) fp32|bf16 (z may be None); conv_w (d_inner, d_conv) fp32;
    conv_b (d_inner,) fp32 or None; conv_state (batch, d_inner, d_conv-1) fp32 or None;
    the rest as ssm_s6_scan_fwd.  Returns y, or (y, h_final, conv_state_out) when
    return_final (h_final=h0 and conv_state_out=conv_state carry in place).
    u_out (batch, L, d_inner) fp32 receives the scan's input when given."""
    dev = x.device
    batch, L, Dm = x.shape
    N, K = A_log.shape[1], conv_w.shape[1]
    dty = x.dtype
    _req(x, "x", dty, (batch, L, Dm), dev)
    _req(conv_w, "conv_w", torch.float32, (Dm, K), dev)
    _opt(conv_b, "conv_b", torch.float32, (Dm,), dev)
    _opt(conv_state, "conv_state", torch.float32, (batch, Dm, K - 1), dev)
    _opt(z, "z", dty, (batch, L, Dm), dev)
    _req(dt, "dt", torch.float32, (batch, L, Dm), dev)
    _opt(dt_bias, "dt_bias", torch.float32, (Dm,), dev)
    _req(A_log, "A_log", torch.float32, (Dm, N), dev)
    _req(B, "B", dty, (batch, L, N), dev)
    _req(C, "C", dty, (batch, L, N), dev)
    _opt(D, "D", torch.float32, (Dm,), dev)
    _opt(h0, "h0", torch.float32, (batch, Dm, N), dev)
    if y is None:
        y = torch.empty((batch, L, Dm), dtype=torch.float32, device=dev)
    _req(y, "y", torch.float32, (batch, L, Dm), dev)
    if return_final:
        if h_final is None:
            h_final = torch.empty((batch, Dm, N), dtype=torch.float32, device=dev)
        if conv_state_out is None and K > 1:
            conv_state_out = torch.empty((batch, Dm, K - 1), dtype=torch.float32, device=dev)
    _opt(h_final, "h_final", torch.float32, (batch, Dm, N), dev)
    _opt(u_out, "u_out", torch.float32, (batch, L, Dm), dev)
    _opt(conv_state_out, "conv_state_out", torch.float32, (batch, Dm, K - 1), dev)
    rc = _lib.ssm_s6_fused_fwd(_ptr(x), _ptr(conv_w), _ptr(conv_b), _ptr(conv_state), _ptr(z), _ptr(dt),
                               _ptr(dt_bias), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D), _ptr(y), _ptr(h0),
                               _ptr(h_final), _ptr(u_out), _ptr(conv_state_out), batch, L, Dm, N, K,
                               _in_dtype(x), flags, _stream(dev))
    _check(rc)
    return (y, h_final, conv_state_out) if return_final else y


def ssm_causal_conv1d_fwd(x, w, bias=None, state_in=None, *, silu=False, y=None, state_out=None,
                          return_state=False):
    """Causal depthwise conv1d (+ SiLU).  x (batch, L, channels) fp32|bf16; w (channels, K)
    fp32; bias (channels,) fp32 or None; state_in (batch, channels, K-1) fp32 or None.
    Returns y (x's dtype), or (y, state_out) when return_state or state_out is given
    (state_out=state_in updates the state in place)."""
    dev = x.device
    batch, L, Dc = x.shape
    K = w.shape[1]
    _req(x, "x", x.dtype, (batch, L, Dc), dev)
    _req(w, "w", torch.float32, (Dc, K), dev)
    _opt(bias, "bias", torch.float32, (Dc,), dev)
    _opt(state_in, "state_in", torch.float32, (batch, Dc, K - 1), dev)
    if y is None:
        y = torch.empty_like(x)
    _req(y, "y", x.dtype, (batch, L, Dc), dev)
    if return_state and state_out is None and K > 1:
        state_out = torch.empty((batch, Dc, K - 1), dtype=torch.float32, device=dev)
    _opt(state_out, "state_out", torch.float32, (batch, Dc, K - 1), dev)
    rc = _lib.ssm_causal_conv1d_fwd(_ptr(x), _ptr(w), _ptr(bias), _ptr(state_in), _ptr(y), _ptr(state_out),
                                    batch, L, Dc, K, int(bool(silu)), _in_dtype(x), _stream(dev))
    _check(rc)
    return (y, state_out) if (return_state or state_out is not None) else y


_S6_GRADS = ("du", "ddt", "dB", "dC", "dA_log", "dD", "ddt_bias", "dh0")


def ssm_s6_scan_grouped_bwd_workspace_size(batch, L, d_inner, d_state, ngroups) -> int:
    return int(_lib.ssm_s6_scan_grouped_bwd_workspace_size(batch, L, d_inner, d_state, ngroups))


def ssm_s6_scan_grouped_bwd(u, dt, dt_bias, A_log, B, C, D, h0, dy, dh_final=None, *, flags=SSM_BBAR_ZOH,
                            out=None, workspace=None, _checkpoints=None):
    """Gradients of ssm_s6_scan_grouped_fwd.  Inputs as there, plus dy (batch, L, d_inner) fp32 and
    dh_final (batch, d_inner, d_state) fp32 or None.  Returns a dict as ssm_s6_scan_bwd, with
    dB, dC (batch, L, ngroups, d_state)."""
    dev = u.device
    batch, L, Dm = u.shape
    N = A_log.shape[1]
    G = B.shape[2]
    dty = u.dtype
    _req(u, "u", dty, (batch, L, Dm), dev)
    _req(dt, "dt", torch.float32, (batch, L, Dm), dev)
    _opt(dt_bias, "dt_bias", torch.float32, (Dm,), dev)
    _req(A_log, "A_log", torch.float32, (Dm, N), dev)
    _req(B, "B", dty, (batch, L, G, N), dev)
    _req(C, "C", dty, (batch, L, G, N), dev)
    _opt(D, "D", torch.float32, (Dm,), dev)
    _opt(h0, "h0", torch.float32, (batch, Dm, N), dev)
    _req(dy, "dy", torch.float32, (batch, L, Dm), dev)
    _opt(dh_final, "dh_final", torch.float32, (batch, Dm, N), dev)
    shapes = dict(du=(batch, L, Dm), ddt=(batch, L, Dm), dB=(batch, L, G, N), dC=(batch, L, G, N),
                  dA_log=(Dm, N), dD=(Dm,), ddt_bias=(Dm,), dh0=(batch, Dm, N))
    g = dict(out or {})
    for k in _S6_GRADS:
        if g.get(k) is None:
            g[k] = torch.empty(shapes[k], dtype=torch.float32, device=dev)
        _req(g[k], k, torch.float32, shapes[k], dev)
    need = ssm_s6_scan_grouped_bwd_workspace_size(batch, L, Dm, N, G)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    if _checkpoints is not None:
        _req(_checkpoints, "checkpoints", torch.float32, (batch, (L + 15) // 16, Dm, N), dev)
        rc = _lib.ssm_s6_scan_grouped_bwd_saved(_ptr(u), _ptr(dt), _ptr(dt_bias), _ptr(A_log), _ptr(B), _ptr(C),
                                                _ptr(D), _ptr(h0), _ptr(dy), _ptr(dh_final), _ptr(_checkpoints),
                                                *(_ptr(g[k]) for k in _S6_GRADS), batch, L, Dm, N, G,
                                                _in_dtype(u), flags, _ptr(workspace),
                                                workspace.numel() * workspace.element_size(), _stream(dev))
    else:
        rc = _lib.ssm_s6_scan_grouped_bwd(_ptr(u), _ptr(dt), _ptr(dt_bias), _ptr(A_log), _ptr(B), _ptr(C),
                                          _ptr(D), _ptr(h0), _ptr(dy), _ptr(dh_final),
                                          *(_ptr(g[k]) for k in _S6_GRADS), batch, L, Dm, N, G, _in_dtype(u),
                                          flags, _ptr(workspace), workspace.numel() * workspace.element_size(),
                                          _stream(dev))
    _check(rc)
    return g


def ssm_s6_scan_grouped_fwd_save(u, dt, dt_bias, A_log, B, C, D, h0=None, *, flags=SSM_BBAR_ZOH, y=None,
                                 h_final=None, checkpoints=None):
    """ssm_s6_scan_grouped_fwd that also saves the state entering every 16-step tile for
    the backward (d_state <= 16).  Returns (y, h_final, checkpoints); checkpoints is
    (batch, ceil(L/16), d_inner, d_state) fp32."""
    dev = u.device
    batch, L, Dm = u.shape
    N = A_log.shape[1]
    G = B.shape[2]
    dty = u.dtype
    _req(u, "u", dty, (batch, L, Dm), dev)
    _req(dt, "dt", torch.float32, (batch, L, Dm), dev)
    _opt(dt_bias, "dt_bias", torch.float32, (Dm,), dev)
    _req(A_log, "A_log", torch.float32, (Dm, N), dev)
    _req(B, "B", dty, (batch, L, G, N), dev)
    _req(C, "C", dty, (batch, L, G, N), dev)
    _opt(D, "D", torch.float32, (Dm,), dev)
    _opt(h0, "h0", torch.float32, (batch, Dm, N), dev)
    if y is None:
        y = torch.empty((batch, L, Dm), dtype=torch.float32, device=dev)
    _req(y, "y", torch.float32, (batch, L, Dm), dev)
    if h_final is None:
        h_final = torch.empty((batch, Dm, N), dtype=torch.float32, device=dev)
    _req(h_final, "h_final", torch.float32, (batch, Dm, N), dev)
    ck_shape = (batch, (L + 15) // 16, Dm, N)
    if checkpoints is None:
        checkpoints = torch.empty(ck_shape, dtype=torch.float32, device=dev)
    _req(checkpoints, "checkpoints", torch.float32, ck_shape, dev)
    rc = _lib.ssm_s6_scan_grouped_fwd_save(_ptr(u), _ptr(dt), _ptr(dt_bias), _ptr(A_log), _ptr(B), _ptr(C),
                                           _ptr(D), _ptr(y), _ptr(h0), _ptr(h_final), _ptr(checkpoints),
                                           batch, L, Dm, N, G, _in_dtype(u), flags, _stream(dev))
    _check(rc)
    return y, h_final, checkpoints


def ssm_s6_scan_grouped_bwd_saved(u, dt, dt_bias, A_log, B, C, D, h0, dy, dh_final, checkpoints, *,
                                  flags=SSM_BBAR_ZOH, out=None, workspace=None):
    """ssm_s6_scan_grouped_bwd reading the states ssm_s6_scan_grouped_fwd_save wrote (same
    inputs as that forward) instead of recomputing them."""
    if checkpoints is None:
        raise ValueError("checkpoints are required")
    return ssm_s6_scan_grouped_bwd(u, dt, dt_bias, A_log, B, C, D, h0, dy, dh_final, flags=flags, out=out,
                                   workspace=workspace, _checkpoints=checkpoints)


def ssm_s6_scan_checkpoint_size(batch, L, d_inner, d_state) -> int:
    return int(_lib.ssm_s6_scan_checkpoint_size(batch, L, d_inner, d_state))


def ssm_s6_scan_fwd_save(u, dt, dt_bias, A_log, B, C, D, h0=None, *, flags=SSM_BBAR_ZOH, y=None,
                         h_final=None, checkpoints=None):
    """ssm_s6_scan_fwd that also saves the state entering every 16-step tile for the
    backward (d_state <= 16).  Returns (y, h_final, checkpoints); checkpoints is
    (batch, ceil(L/16), d_inner, d_state) fp32."""
    dev = u.device
    batch, L, Dm = u.shape
    N = A_log.shape[1]
    dty = u.dtype
    _req(u, "u", dty, (batch, L, Dm), dev)
    _req(dt, "dt", torch.float32, (batch, L, Dm), dev)
    _opt(dt_bias, "dt_bias", torch.float32, (Dm,), dev)
    _req(A_log, "A_log", torch.float32, (Dm, N), dev)
    _req(B, "B", dty, (batch, L, N), dev)
    _req(C, "C", dty, (batch, L, N), dev)
    _opt(D, "D", torch.float32, (Dm,), dev)
    _opt(h0, "h0", torch.float32, (batch, Dm, N), dev)
    if y is None:
        y = torch.empty((batch, L, Dm), dtype=torch.float32, device=dev)
    _req(y, "y", torch.float32, (batch, L, Dm), dev)
    if h_final is None:
        h_final = torch.empty((batch, Dm, N), dtype=torch.float32, device=dev)
    _req(h_final, "h_final", torch.float32, (batch, Dm, N), dev)
    ck_shape = (batch, (L + 15) // 16, Dm, N)
    if checkpoints is None:
        checkpoints = torch.empty(ck_shape, dtype=torch.float32, device=dev)
    _req(checkpoints, "checkpoints", torch.float32, ck_shape, dev)
    rc = _lib.ssm_s6_scan_fwd_save(_ptr(u), _ptr(dt), _ptr(dt_bias), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D),
                                   _ptr(y), _ptr(h0), _ptr(h_final), _ptr(checkpoints), batch, L, Dm, N,
                                   _in_dtype(u), flags, _stream(dev))
    _check(rc)
    return y, h_final, checkpoints


def ssm_s6_scan_bwd_saved(u, dt, dt_bias, A_log, B, C, D, h0, dy, dh_final, checkpoints, *,
                          flags=SSM_BBAR_ZOH, out=None, workspace=None):
    """ssm_s6_scan_bwd reading the states ssm_s6_scan_fwd_save wrote (same inputs as that
    forward) instead of recomputing them."""
    if checkpoints is None:
        raise ValueError("checkpoints are required")
    return ssm_s6_scan_bwd(u, dt, dt_bias, A_log, B, C, D, h0, dy, dh_final, flags=flags, out=out,
                           workspace=workspace, _checkpoints=checkpoints)


def ssm_s6_scan_bwd(u, dt, dt_bias, A_log, B, C, D, h0, dy, dh_final=None, *, flags=SSM_BBAR_ZOH,
                    out=None, workspace=None, _checkpoints=None):
    """Gradients of the S6 forward scan.  Inputs as ssm_s6_scan_fwd, plus
    dy (batch, L, d_inner) fp32 and dh_final (batch, d_inner, d_state) fp32 or None.
    Returns a dict of fp32 tensors: du, ddt (batch, L, d_inner); dB, dC
    (batch, L, d_state); dA_log (d_inner, d_state); dD, ddt_bias (d_inner);
    dh0 (batch, d_inner, d_state).  `out` may hold preallocated tensors under
    those names; `workspace` a uint8 tensor of ssm_s6_scan_bwd_workspace_size bytes."""
    dev = u.device
    batch, L, Dm = u.shape
    N = A_log.shape[1]
    dty = u.dtype
    _req(u, "u", dty, (batch, L, Dm), dev)
    _req(dt, "dt", torch.float32, (batch, L, Dm), dev)
    _opt(dt_bias, "dt_bias", torch.float32, (Dm,), dev)
    _req(A_log, "A_log", torch.float32, (Dm, N), dev)
    _req(B, "B", dty, (batch, L, N), dev)
    _req(C, "C", dty, (batch, L, N), dev)
    _opt(D, "D", torch.float32, (Dm,), dev)
    _opt(h0, "h0", torch.float32, (batch, Dm, N), dev)
    _req(dy, "dy", torch.float32, (batch, L, Dm), dev)
    _opt(dh_final, "dh_final", torch.float32, (batch, Dm, N), dev)
    shapes = dict(du=(batch, L, Dm), ddt=(batch, L, Dm), dB=(batch, L, N), dC=(batch, L, N),
                  dA_log=(Dm, N), dD=(Dm,), ddt_bias=(Dm,), dh0=(batch, Dm, N))
    g = dict(out or {})
    for k in _S6_GRADS:
        if g.get(k) is None:
            g[k] = torch.empty(shapes[k], dtype=torch.float32, device=dev)
        _req(g[k], k, torch.float32, shapes[k], dev)
    need = ssm_s6_scan_bwd_workspace_size(batch, L, Dm, N)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    if _checkpoints is not None:
        _req(_checkpoints, "checkpoints", torch.float32, (batch, (L + 15) // 16, Dm, N), dev)
        rc = _lib.ssm_s6_scan_bwd_saved(_ptr(u), _ptr(dt), _ptr(dt_bias), _ptr(A_log), _ptr(B), _ptr(C),
                                        _ptr(D), _ptr(h0), _ptr(dy), _ptr(dh_final), _ptr(_checkpoints),
                                        *(_ptr(g[k]) for k in _S6_GRADS), batch, L, Dm, N, _in_dtype(u),
                                        flags, _ptr(workspace), workspace.numel() * workspace.element_size(),
                                        _stream(dev))
    else:
        rc = _lib.ssm_s6_scan_bwd(_ptr(u), _ptr(dt), _ptr(dt_bias), _ptr(A_log), _ptr(B), _ptr(C),
                                  _ptr(D), _ptr(h0), _ptr(dy), _ptr(dh_final),
                                  *(_ptr(g[k]) for k in _S6_GRADS), batch, L, Dm, N, _in_dtype(u),
                                  flags, _ptr(workspace), workspace.numel() * workspace.element_size(),
                                  _stream(dev))
    _check(rc)
    return g


def ssd_chunk_scan_fwd(x, dt, dt_bias, A_log, B, C, D, h0=None, *, chunk_len=256,
                       flags=SSM_BBAR_DT, return_final=False, y=None, h_final=None, workspace=None):
    """SSD chunked forward scan.  x (batch, L, H, P) bf16; dt (batch, L, H) fp32;
    dt_bias, A_log, D (H,) fp32 (dt_bias, D may be None); B, C (batch, L, G, N) in x's
    dtype; h0 (batch, H, P, N) fp32 or None.  Returns y fp32 (and h_final)."""
    dev = x.device
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    dty = x.dtype
    _req(x, "x", dty, (batch, L, H, P), dev)
    _req(dt, "dt", torch.float32, (batch, L, H), dev)
    _opt(dt_bias, "dt_bias", torch.float32, (H,), dev)
    _req(A_log, "A_log", torch.float32, (H,), dev)
    _req(B, "B", dty, (batch, L, G, N), dev)
    _req(C, "C", dty, (batch, L, G, N), dev)
    _opt(D, "D", torch.float32, (H,), dev)
    _opt(h0, "h0", torch.float32, (batch, H, P, N), dev)
    if y is None:
        y = torch.empty((batch, L, H, P), dtype=torch.float32, device=dev)
    _req(y, "y", torch.float32, (batch, L, H, P), dev)
    if return_final and h_final is None:
        h_final = torch.empty((batch, H, P, N), dtype=torch.float32, device=dev)
    _opt(h_final, "h_final", torch.float32, (batch, H, P, N), dev)
    ws = ssd_chunk_scan_fwd_workspace_size(batch, L, H, P, N, G, chunk_len)
    if workspace is None:
        workspace = torch.empty((max(ws, 1),), dtype=torch.uint8, device=dev)
    rc = _lib.ssd_chunk_scan_fwd(_ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A_log), _ptr(B), _ptr(C),
                                 _ptr(D), _ptr(y), _ptr(h0), _ptr(h_final), batch, L, H, P, N, G,
                                 chunk_len, _in_dtype(x), flags, _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(dev))
    _check(rc)
    return (y, h_final) if (return_final or h_final is not None) else y


def ssd_chunk_scan_fwd_noalloc(x, dt, dt_bias, A_log, B, C, D, h0=None, *, chunk_len=256,
                               flags=SSM_BBAR_DT, return_final=False, y=None, h_final=None):
    """ssd_chunk_scan_fwd without a workspace: the segment states live in the library's
    static device scratch (32 MiB per GPU), so the call allocates nothing when y (and
    h_final) are given.  Calls that overlap on one GPU race on the scratch."""
    dev = x.device
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    dty = x.dtype
    _req(x, "x", dty, (batch, L, H, P), dev)
    _req(dt, "dt", torch.float32, (batch, L, H), dev)
    _opt(dt_bias, "dt_bias", torch.float32, (H,), dev)
    _req(A_log, "A_log", torch.float32, (H,), dev)
    _req(B, "B", dty, (batch, L, G, N), dev)
    _req(C, "C", dty, (batch, L, G, N), dev)
    _opt(D, "D", torch.float32, (H,), dev)
    _opt(h0, "h0", torch.float32, (batch, H, P, N), dev)
    if y is None:
        y = torch.empty((batch, L, H, P), dtype=torch.float32, device=dev)
    _req(y, "y", torch.float32, (batch, L, H, P), dev)
    if return_final and h_final is None:
        h_final = torch.empty((batch, H, P, N), dtype=torch.float32, device=dev)
    _opt(h_final, "h_final", torch.float32, (batch, H, P, N), dev)
    rc = _lib.ssd_chunk_scan_fwd_noalloc(_ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A_log), _ptr(B), _ptr(C),
                                         _ptr(D), _ptr(y), _ptr(h0), _ptr(h_final), batch, L, H, P, N, G,
                                         chunk_len, _in_dtype(x), flags, _stream(dev))
    _check(rc)
    return (y, h_final) if (return_final or h_final is not None) else y


def ssd_trap_chunk_scan_fwd(x, k, q, dt, a, trap, D=None, h0=None, k_prev=None, x_prev=None, *,
                            chunk_len=64, return_final=False, y=None, h_final=None, workspace=None):
    """Mamba-3 trapezoidal SSD forward.  x (batch, L, H, P) bf16; k, q (batch, L, H, N)
    bf16; dt, a, trap (batch, L, H) fp32 (dt positive, used as given); D (H,) fp32 or
    None; h0 (batch, H, P, N) fp32 or None; k_prev (batch, H, N), x_prev (batch, H, P)
    bf16, both or neither.  Returns y fp32 (and h_final)."""
    dev = x.device
    batch, L, H, P = x.shape
    N = k.shape[3]
    dty = x.dtype
    _req(x, "x", dty, (batch, L, H, P), dev)
    _req(k, "k", dty, (batch, L, H, N), dev)
    _req(q, "q", dty, (batch, L, H, N), dev)
    for t, nm in ((dt, "dt"), (a, "a"), (trap, "trap")):
        _req(t, nm, torch.float32, (batch, L, H), dev)
    _opt(D, "D", torch.float32, (H,), dev)
    _opt(h0, "h0", torch.float32, (batch, H, P, N), dev)
    _opt(k_prev, "k_prev", dty, (batch, H, N), dev)
    _opt(x_prev, "x_prev", dty, (batch, H, P), dev)
    if y is None:
        y = torch.empty((batch, L, H, P), dtype=torch.float32, device=dev)
    _req(y, "y", torch.float32, (batch, L, H, P), dev)
    if return_final and h_final is None:
        h_final = torch.empty((batch, H, P, N), dtype=torch.float32, device=dev)
    _opt(h_final, "h_final", torch.float32, (batch, H, P, N), dev)
    ws = ssd_trap_chunk_scan_fwd_workspace_size(batch, L, H, P, N, chunk_len)
    if workspace is None:
        workspace = torch.empty((max(ws, 1),), dtype=torch.uint8, device=dev)
    rc = _lib.ssd_trap_chunk_scan_fwd(_ptr(x), _ptr(k), _ptr(q), _ptr(dt), _ptr(a), _ptr(trap),
                                      _ptr(D), _ptr(y), _ptr(h0), _ptr(k_prev), _ptr(x_prev),
                                      _ptr(h_final), batch, L, H, P, N, chunk_len, _in_dtype(x),
                                      _ptr(workspace), workspace.numel() * workspace.element_size(),
                                      _stream(dev))
    _check(rc)
    return (y, h_final) if (return_final or h_final is not None) else y


def ssd_trap_rotate_qk_workspace_size(batch, L, nheads, d_state, n_angles) -> int:
    return int(_lib.ssd_trap_rotate_qk_workspace_size(batch, L, nheads, d_state, n_angles))


def ssd_trap_rotate_qk(k_raw, q_raw, angles, dt, angle_state=None, *, k=None, q=None,
                       angle_state_out=None, return_state=False, workspace=None):
    """Mamba-3 data-dependent rotation of k and q.  k_raw, q_raw (batch, L, H, N) bf16;
    angles (batch, L, n_angles) fp32 (2 n_angles <= N); dt (batch, L, H) fp32; angle_state
    (batch, H, n_angles) fp32 or None.  Returns (k, q), or (k, q, angle_state_out) when
    return_state.  k=k_raw, q=q_raw and angle_state_out=angle_state update in place."""
    dev = k_raw.device
    batch, L, H, N = k_raw.shape
    NA = angles.shape[2]
    _req(k_raw, "k_raw", torch.bfloat16, (batch, L, H, N), dev)
    _req(q_raw, "q_raw", torch.bfloat16, (batch, L, H, N), dev)
    _req(angles, "angles", torch.float32, (batch, L, NA), dev)
    _req(dt, "dt", torch.float32, (batch, L, H), dev)
    _opt(angle_state, "angle_state", torch.float32, (batch, H, NA), dev)
    k = torch.empty_like(k_raw) if k is None else k
    q = torch.empty_like(q_raw) if q is None else q
    _req(k, "k", torch.bfloat16, (batch, L, H, N), dev)
    _req(q, "q", torch.bfloat16, (batch, L, H, N), dev)
    if return_state and angle_state_out is None:
        angle_state_out = torch.empty((batch, H, NA), dtype=torch.float32, device=dev)
    _opt(angle_state_out, "angle_state_out", torch.float32, (batch, H, NA), dev)
    ws = ssd_trap_rotate_qk_workspace_size(batch, L, H, N, NA)
    if workspace is None:
        workspace = torch.empty((max(ws, 1),), dtype=torch.uint8, device=dev)
    rc = _lib.ssd_trap_rotate_qk(_ptr(k_raw), _ptr(q_raw), _ptr(angles), _ptr(dt), _ptr(angle_state),
                                 _ptr(k), _ptr(q), _ptr(angle_state_out), batch, L, H, N, NA,
                                 _in_dtype(k_raw), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(dev))
    _check(rc)
    return (k, q, angle_state_out) if (return_state or angle_state_out is not None) else (k, q)


def ssd_trap_chunk_scan_bwd_workspace_size(batch, L, nheads, headdim, d_state, chunk_len=64) -> int:
    return int(_lib.ssd_trap_chunk_scan_bwd_workspace_size(batch, L, nheads, headdim, d_state, chunk_len))


_TRAP_GRADS = ("dx", "dk", "dq", "ddt", "da", "dtrap", "dD", "dh0", "dk_prev", "dx_prev")


def ssd_trap_chunk_scan_bwd(x, k, q, dt, a, trap, D, h0, k_prev, x_prev, dy, dh_final=None, *, chunk_len=64,
                            out=None, workspace=None):
    """Gradients of ssd_trap_chunk_scan_fwd.  Inputs as there, plus dy (batch, L, H, P) fp32
    and dh_final (batch, H, P, N) fp32 or None.  Returns a dict of fp32 tensors: dx; dk, dq;
    ddt, da, dtrap; dD (H,); dh0 (batch, H, P, N); dk_prev, dx_prev (when the carried pair
    is given, else None)."""
    dev = x.device
    batch, L, H, P = x.shape
    N = k.shape[3]
    dty = x.dtype
    _req(x, "x", dty, (batch, L, H, P), dev)
    _req(k, "k", dty, (batch, L, H, N), dev)
    _req(q, "q", dty, (batch, L, H, N), dev)
    for t_, nm in ((dt, "dt"), (a, "a"), (trap, "trap")):
        _req(t_, nm, torch.float32, (batch, L, H), dev)
    _opt(D, "D", torch.float32, (H,), dev)
    _opt(h0, "h0", torch.float32, (batch, H, P, N), dev)
    _opt(k_prev, "k_prev", dty, (batch, H, N), dev)
    _opt(x_prev, "x_prev", dty, (batch, H, P), dev)
    _req(dy, "dy", torch.float32, (batch, L, H, P), dev)
    _opt(dh_final, "dh_final", torch.float32, (batch, H, P, N), dev)
    prev = k_prev is not None
    shapes = dict(dx=(batch, L, H, P), dk=(batch, L, H, N), dq=(batch, L, H, N), ddt=(batch, L, H),
                  da=(batch, L, H), dtrap=(batch, L, H), dD=(H,), dh0=(batch, H, P, N),
                  dk_prev=(batch, H, N) if prev else None, dx_prev=(batch, H, P) if prev else None)
    g = dict(out or {})
    for n_ in _TRAP_GRADS:
        if shapes[n_] is None:
            g[n_] = None
            continue
        if g.get(n_) is None:
            g[n_] = torch.empty(shapes[n_], dtype=torch.float32, device=dev)
        _req(g[n_], n_, torch.float32, shapes[n_], dev)
    ws = ssd_trap_chunk_scan_bwd_workspace_size(batch, L, H, P, N, chunk_len)
    if workspace is None:
        workspace = torch.empty((max(ws, 1),), dtype=torch.uint8, device=dev)
    rc = _lib.ssd_trap_chunk_scan_bwd(_ptr(x), _ptr(k), _ptr(q), _ptr(dt), _ptr(a), _ptr(trap), _ptr(D),
                                      _ptr(h0), _ptr(k_prev), _ptr(x_prev), _ptr(dy), _ptr(dh_final),
                                      *(_ptr(g[n_]) for n_ in _TRAP_GRADS), batch, L, H, P, N, chunk_len,
                                      _in_dtype(x), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                      _stream(dev))
    _check(rc)
    return g


_SSD_GRADS = ("dx", "ddt", "dB", "dC", "dA_log", "dD", "ddt_bias", "dh0")


def ssd_chunk_scan_bwd(x, dt, dt_bias, A_log, B, C, D, h0, dy, dh_final=None, *, chunk_len=256,
                       flags=SSM_BBAR_DT, out=None, workspace=None):
    """Gradients of the SSD forward scan.  Inputs as ssd_chunk_scan_fwd (bf16 x, B, C),
    plus dy (batch, L, H, P) fp32 and dh_final (batch, H, P, N) fp32 or None.
    Returns a dict of fp32 tensors: dx (batch, L, H, P); ddt (batch, L, H);
    dB, dC (batch, L, G, N); dA_log, dD, ddt_bias (H,); dh0 (batch, H, P, N).
    `out` may hold preallocated tensors under those names; `workspace` a uint8
    tensor of ssd_chunk_scan_bwd_workspace_size bytes."""
    dev = x.device
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    dty = x.dtype
    _req(x, "x", dty, (batch, L, H, P), dev)
    _req(dt, "dt", torch.float32, (batch, L, H), dev)
    _opt(dt_bias, "dt_bias", torch.float32, (H,), dev)
    _req(A_log, "A_log", torch.float32, (H,), dev)
    _req(B, "B", dty, (batch, L, G, N), dev)
    _req(C, "C", dty, (batch, L, G, N), dev)
    _opt(D, "D", torch.float32, (H,), dev)
    _opt(h0, "h0", torch.float32, (batch, H, P, N), dev)
    _req(dy, "dy", torch.float32, (batch, L, H, P), dev)
    _opt(dh_final, "dh_final", torch.float32, (batch, H, P, N), dev)
    shapes = dict(dx=(batch, L, H, P), ddt=(batch, L, H), dB=(batch, L, G, N), dC=(batch, L, G, N),
                  dA_log=(H,), dD=(H,), ddt_bias=(H,), dh0=(batch, H, P, N))
    g = dict(out or {})
    for k in _SSD_GRADS:
        if g.get(k) is None:
            g[k] = torch.empty(shapes[k], dtype=torch.float32, device=dev)
        _req(g[k], k, torch.float32, shapes[k], dev)
    need = ssd_chunk_scan_bwd_workspace_size(batch, L, H, P, N, G, chunk_len)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    rc = _lib.ssd_chunk_scan_bwd(_ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A_log), _ptr(B), _ptr(C),
                                 _ptr(D), _ptr(h0), _ptr(dy), _ptr(dh_final),
                                 *(_ptr(g[k]) for k in _SSD_GRADS), batch, L, H, P, N, G, chunk_len,
                                 _in_dtype(x), flags, _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(dev))
    _check(rc)
    return g


def ssd_cplx_chunk_scan_fwd(x, dt, dt_bias, A_log, B, C, D, h0=None, *, chunk_len=64,
                            flags=SSM_BBAR_ZOH | SSM_CPLX_STABLE, return_final=False, y=None,
                            h_final=None, workspace=None):
    """Complex-state SSD forward scan.  x (batch, L, H, P) fp32; dt (batch, L, H);
    A_log (H, 2) = [log|A|, arg A]; B, C (batch, L, G, Nc, 2) fp32 interleaved (re, im);
    h0 (batch, H, P, Nc, 2) or None.  Returns y (and h_final)."""
    dev = x.device
    batch, L, H, P = x.shape
    G, Nc = B.shape[2], B.shape[3]
    f32 = torch.float32
    _req(x, "x", f32, (batch, L, H, P), dev)
    _req(dt, "dt", f32, (batch, L, H), dev)
    _opt(dt_bias, "dt_bias", f32, (H,), dev)
    _req(A_log, "A_log", f32, (H, 2), dev)
    _req(B, "B", f32, (batch, L, G, Nc, 2), dev)
    _req(C, "C", f32, (batch, L, G, Nc, 2), dev)
    _opt(D, "D", f32, (H,), dev)
    _opt(h0, "h0", f32, (batch, H, P, Nc, 2), dev)
    if y is None:
        y = torch.empty((batch, L, H, P), dtype=f32, device=dev)
    _req(y, "y", f32, (batch, L, H, P), dev)
    if return_final and h_final is None:
        h_final = torch.empty((batch, H, P, Nc, 2), dtype=f32, device=dev)
    _opt(h_final, "h_final", f32, (batch, H, P, Nc, 2), dev)
    ws = ssd_cplx_chunk_scan_fwd_workspace_size(batch, L, H, P, Nc, G, chunk_len)
    if workspace is None:
        workspace = torch.empty((max(ws, 1),), dtype=torch.uint8, device=dev)
    rc = _lib.ssd_cplx_chunk_scan_fwd(_ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A_log), _ptr(B),
                                      _ptr(C), _ptr(D), _ptr(y), _ptr(h0), _ptr(h_final), batch, L,
                                      H, P, Nc, G, chunk_len, flags, _ptr(workspace),
                                      workspace.numel() * workspace.element_size(), _stream(dev))
    _check(rc)
    return (y, h_final) if (return_final or h_final is not None) else y


def ssd_cplx_mimo_chunk_scan_fwd_workspace_size(batch, L, rank, nheads, headdim, n_complex, ngroups,
                                                chunk_len) -> int:
    return int(_lib.ssd_cplx_mimo_chunk_scan_fwd_workspace_size(batch, L, rank, nheads, headdim, n_complex,
                                                                ngroups, chunk_len))


def ssd_cplx_mimo_chunk_scan_fwd(x, dt, dt_bias, A_log, B, C, D, h0=None, *, chunk_len=64,
                                 flags=SSM_BBAR_ZOH | SSM_CPLX_STABLE, return_final=False, y=None,
                                 h_final=None, workspace=None):
    """Multi-input multi-output complex SSD forward scan.  x (batch, L, R, H, P) fp32;
    dt (batch, L, H); A_log (H, 2); B, C (batch, L, R, G, Nc, 2) fp32 interleaved (re, im);
    h0 (batch, H, P, Nc, 2) or None.  Returns y (batch, L, R, H, P) (and h_final)."""
    dev = x.device
    batch, L, R, H, P = x.shape
    G, Nc = B.shape[3], B.shape[4]
    f32 = torch.float32
    _req(x, "x", f32, (batch, L, R, H, P), dev)
    _req(dt, "dt", f32, (batch, L, H), dev)
    _opt(dt_bias, "dt_bias", f32, (H,), dev)
    _req(A_log, "A_log", f32, (H, 2), dev)
    _req(B, "B", f32, (batch, L, R, G, Nc, 2), dev)
    _req(C, "C", f32, (batch, L, R, G, Nc, 2), dev)
    _opt(D, "D", f32, (H,), dev)
    _opt(h0, "h0", f32, (batch, H, P, Nc, 2), dev)
    if y is None:
        y = torch.empty((batch, L, R, H, P), dtype=f32, device=dev)
    _req(y, "y", f32, (batch, L, R, H, P), dev)
    if return_final and h_final is None:
        h_final = torch.empty((batch, H, P, Nc, 2), dtype=f32, device=dev)
    _opt(h_final, "h_final", f32, (batch, H, P, Nc, 2), dev)
    ws = ssd_cplx_mimo_chunk_scan_fwd_workspace_size(batch, L, R, H, P, Nc, G, chunk_len)
    if workspace is None:
        workspace = torch.empty((max(ws, 1),), dtype=torch.uint8, device=dev)
    rc = _lib.ssd_cplx_mimo_chunk_scan_fwd(_ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A_log), _ptr(B),
                                           _ptr(C), _ptr(D), _ptr(y), _ptr(h0), _ptr(h_final), batch, L,
                                           R, H, P, Nc, G, chunk_len, flags, _ptr(workspace),
                                           workspace.numel() * workspace.element_size(), _stream(dev))
    _check(rc)
    return (y, h_final) if (return_final or h_final is not None) else y
