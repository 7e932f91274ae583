"""The C interface of libssmscan.so without a GPU: every symbol the header
declares is exported, workspace sizes, and every argument check returns its
error code and message before any HIP call (fake, aligned pointers are never
dereferenced on these paths)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm_scan.h")
LIB = os.path.join(ROOT, "selective_state_space_s6_amd", "libssmscan.so")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3
FAKE = ctypes.c_void_p(0x100000)      # aligned, never dereferenced by the checks
MIS = ctypes.c_void_p(0x100004)       # misaligned


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from selective_state_space_s6_amd import build as b  # noqa: F401  (import builds nothing)
        pytest.skip("libssmscan.so not built")
    L = ctypes.CDLL(LIB)
    L.ssm_last_error.restype = ctypes.c_char_p
    I, P, Z = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    L.ssm_s6_scan_fwd.argtypes = [P] * 10 + [I] * 4 + [ctypes.c_int, ctypes.c_uint32, P, Z, P]
    L.ssd_chunk_scan_fwd.argtypes = [P] * 10 + [I] * 7 + [ctypes.c_int, ctypes.c_uint32, P, Z, P]
    L.ssd_cplx_chunk_scan_fwd.argtypes = [P] * 10 + [I] * 7 + [ctypes.c_uint32, P, Z, P]
    for f in ("ssm_s6_scan_fwd_workspace_size",):
        getattr(L, f).argtypes = [I] * 4
        getattr(L, f).restype = Z
    for f in ("ssd_chunk_scan_fwd_workspace_size", "ssd_cplx_chunk_scan_fwd_workspace_size"):
        getattr(L, f).argtypes = [I] * 7
        getattr(L, f).restype = Z
    return L


def test_every_declared_symbol_is_exported(lib):
    text = open(HEADER).read()
    names = set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, re.M))
    names = {n for n in names if n.startswith(("ssm_", "ssd_"))}
    assert names == {"ssm_last_error", "ssm_s6_scan_fwd_workspace_size", "ssm_s6_scan_fwd",
                     "ssd_chunk_scan_fwd_workspace_size", "ssd_chunk_scan_fwd",
                     "ssd_cplx_chunk_scan_fwd_workspace_size", "ssd_cplx_chunk_scan_fwd"}
    for n in names:
        assert hasattr(lib, n), n


def _s6(lib, u=FAKE, dt=FAKE, A_log=FAKE, B=FAKE, C=FAKE, y=FAKE, dims=(2, 8, 16, 4), dtype=0,
        flags=0, dt_bias=None, D=None, h0=None, hf=None):
    return lib.ssm_s6_scan_fwd(u, dt, dt_bias, A_log, B, C, D, y, h0, hf, *dims, dtype, flags,
                               None, 0, None)


def _err(lib):
    return lib.ssm_last_error().decode()


def test_s6_argument_checks(lib):
    assert _s6(lib, u=None) == INVALID and "u is NULL" in _err(lib)
    assert _s6(lib, y=None) == INVALID and "y is NULL" in _err(lib)
    assert _s6(lib, dims=(0, 8, 16, 4)) == INVALID and "batch" in _err(lib)
    assert _s6(lib, dims=(1, -3, 16, 4)) == INVALID and "L" in _err(lib)
    assert _s6(lib, dims=(1, 8, 16, 300)) == UNSUPPORTED and "d_state" in _err(lib)
    assert _s6(lib, dtype=7) == INVALID and "in_dtype" in _err(lib)
    assert _s6(lib, flags=0x3) == INVALID and "flags" in _err(lib)
    assert _s6(lib, flags=0x4) == INVALID
    assert _s6(lib, B=MIS) == UNSUPPORTED and "aligned" in _err(lib)
    assert _s6(lib, y=FAKE, u=FAKE) == INVALID and "alias" in _err(lib)
    assert lib.ssm_s6_scan_fwd_workspace_size(8, 2048, 1536, 16) == 0


def _ssd(lib, dims=(2, 300, 4, 64, 128, 2, 256), dtype=1, flags=1, ws=FAKE, wsb=1 << 40, x=FAKE,
         y=ctypes.c_void_p(0x200000)):
    return lib.ssd_chunk_scan_fwd(x, FAKE, None, FAKE, FAKE, FAKE, None, y, None, None, *dims, dtype,
                                  flags, ws, wsb, None)


def test_ssd_argument_checks(lib):
    assert _ssd(lib, x=None) == INVALID and "x is NULL" in _err(lib)
    assert _ssd(lib, dims=(2, 300, 6, 64, 128, 4, 256)) == INVALID and "ngroups" in _err(lib)
    assert _ssd(lib, dims=(2, 300, 4, 48, 128, 2, 256)) == UNSUPPORTED and "headdim" in _err(lib)
    assert _ssd(lib, dims=(2, 300, 4, 64, 100, 2, 256)) == UNSUPPORTED and "d_state" in _err(lib)
    assert _ssd(lib, dims=(2, 300, 4, 64, 512, 2, 256)) == UNSUPPORTED
    assert _ssd(lib, dims=(2, 300, 4, 64, 128, 2, 100)) == UNSUPPORTED and "chunk_len" in _err(lib)
    assert _ssd(lib, dims=(2, 300, 4, 64, 128, 2, 0)) == INVALID
    assert _ssd(lib, dtype=0) == UNSUPPORTED and "bf16" in _err(lib)
    assert _ssd(lib, flags=0x8) == INVALID
    # short sequences run as one segment (no workspace); long ones keep one
    # (P x N) fp32 state per (batch, head, segment) plus a decay per segment
    assert lib.ssd_chunk_scan_fwd_workspace_size(2, 300, 4, 64, 128, 2, 256) == 0
    ws = lib.ssd_chunk_scan_fwd_workspace_size(8, 4096, 24, 64, 128, 1, 256)
    assert ws >= 8 * 24 * 2 * 64 * 128 * 4 and ws % 4 == 0
    assert lib.ssd_chunk_scan_fwd_workspace_size(0, 300, 4, 64, 128, 2, 256) == 0


def _cssd(lib, dims=(2, 100, 4, 64, 32, 2, 64), flags=0, ws=FAKE, wsb=1 << 40):
    return lib.ssd_cplx_chunk_scan_fwd(FAKE, FAKE, None, FAKE, FAKE, FAKE, None,
                                       ctypes.c_void_p(0x200000), None, None, *dims, flags, ws, wsb,
                                       None)


def test_cssd_argument_checks(lib):
    assert _cssd(lib, dims=(2, 100, 4, 64, 32, 3, 64)) == INVALID
    assert _cssd(lib, dims=(2, 100, 4, 40, 32, 2, 64)) == UNSUPPORTED and "headdim" in _err(lib)
    assert _cssd(lib, dims=(2, 100, 4, 64, 30, 2, 64)) == UNSUPPORTED and "n_complex" in _err(lib)
    assert _cssd(lib, dims=(2, 100, 4, 64, 32, 2, 256)) == UNSUPPORTED and "chunk_len" in _err(lib)
    assert _cssd(lib, flags=0x8 | 0x1) == INVALID and "CODE" in _err(lib)
    assert _cssd(lib, flags=0xC) == INVALID
    assert _cssd(lib, flags=0x20) == INVALID
    assert _cssd(lib, dims=(2, 100, 4, 64, 72, 2, 64)) == UNSUPPORTED and "n_complex" in _err(lib)
    # long sequences are cut into segments whose states go through the workspace
    long_dims = (4, 8192, 32, 64, 32, 1, 64)
    need = lib.ssd_cplx_chunk_scan_fwd_workspace_size(*long_dims)
    assert need >= 4 * 32 * 2 * 64 * 32 * 2 * 4
    assert lib.ssd_cplx_chunk_scan_fwd_workspace_size(2, 100, 4, 64, 32, 2, 64) == 0
    assert _cssd(lib, dims=long_dims, ws=None) == WORKSPACE
    assert _cssd(lib, dims=long_dims, wsb=need - 1) == WORKSPACE
