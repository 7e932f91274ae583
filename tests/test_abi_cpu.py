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
    L.ssm_s6_scan_grouped_fwd.argtypes = [P] * 10 + [I] * 5 + [ctypes.c_int, ctypes.c_uint32, P]
    L.ssm_s6_scan_fwd_save.argtypes = [P] * 11 + [I] * 4 + [ctypes.c_int, ctypes.c_uint32, P]
    L.ssm_s6_scan_bwd_saved.argtypes = [P] * 19 + [I] * 4 + [ctypes.c_int, ctypes.c_uint32, P, Z, P]
    L.ssm_s6_scan_grouped_fwd_save.argtypes = [P] * 11 + [I] * 5 + [ctypes.c_int, ctypes.c_uint32, P]
    L.ssm_s6_scan_grouped_bwd_saved.argtypes = [P] * 19 + [I] * 5 + [ctypes.c_int, ctypes.c_uint32, P, Z, P]
    L.ssm_s6_scan_grouped_bwd.argtypes = [P] * 18 + [I] * 5 + [ctypes.c_int, ctypes.c_uint32, P, Z, P]
    L.ssm_s6_scan_grouped_bwd_workspace_size.argtypes = [I] * 5
    L.ssm_s6_scan_grouped_bwd_workspace_size.restype = Z
    L.ssm_s6_scan_checkpoint_size.argtypes = [I] * 4
    L.ssm_s6_scan_checkpoint_size.restype = Z
    L.ssd_chunk_scan_fwd.argtypes = [P] * 10 + [I] * 7 + [ctypes.c_int, ctypes.c_uint32, P, Z, P]
    L.ssd_cplx_chunk_scan_fwd.argtypes = [P] * 10 + [I] * 7 + [ctypes.c_uint32, P, Z, P]
    L.ssd_cplx_mimo_chunk_scan_fwd.argtypes = [P] * 10 + [I] * 8 + [ctypes.c_uint32, P, Z, P]
    L.ssd_cplx_mimo_chunk_scan_fwd_workspace_size.argtypes = [I] * 8
    L.ssd_cplx_mimo_chunk_scan_fwd_workspace_size.restype = Z
    L.ssm_s6_scan_bwd.argtypes = [P] * 18 + [I] * 4 + [ctypes.c_int, ctypes.c_uint32, P, Z, P]
    L.ssd_chunk_scan_bwd.argtypes = [P] * 18 + [I] * 7 + [ctypes.c_int, ctypes.c_uint32, P, Z, P]
    L.ssd_trap_chunk_scan_fwd.argtypes = [P] * 12 + [I] * 6 + [ctypes.c_int, P, Z, P]
    L.ssd_trap_chunk_scan_fwd_workspace_size.argtypes = [I] * 6
    L.ssd_trap_chunk_scan_fwd_workspace_size.restype = Z
    L.ssd_trap_rotate_qk.argtypes = [P] * 8 + [I] * 5 + [ctypes.c_int, P, Z, P]
    L.ssm_s6_fused_fwd.argtypes = [P] * 16 + [I] * 5 + [ctypes.c_int, ctypes.c_uint32, P]
    L.ssm_causal_conv1d_fwd.argtypes = [P] * 6 + [I] * 4 + [ctypes.c_int, ctypes.c_int, P]
    L.ssd_trap_chunk_scan_bwd.argtypes = [P] * 22 + [I] * 6 + [ctypes.c_int, P, Z, P]
    L.ssd_trap_chunk_scan_bwd_workspace_size.argtypes = [I] * 6
    L.ssd_trap_chunk_scan_bwd_workspace_size.restype = Z
    L.ssd_trap_rotate_qk_workspace_size.argtypes = [I] * 5
    L.ssd_trap_rotate_qk_workspace_size.restype = Z
    for f in ("ssm_s6_scan_fwd_workspace_size", "ssm_s6_scan_bwd_workspace_size"):
        getattr(L, f).argtypes = [I] * 4
        getattr(L, f).restype = Z
    for f in ("ssd_chunk_scan_fwd_workspace_size", "ssd_cplx_chunk_scan_fwd_workspace_size",
              "ssd_chunk_scan_bwd_workspace_size"):
        getattr(L, f).argtypes = [I] * 7
        getattr(L, f).restype = Z
    return L


def test_every_declared_symbol_is_exported(lib):
    text = open(HEADER).read()
    names = set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, re.M))
    names = {n for n in names if n.startswith(("ssm_", "ssd_"))}
    assert names == {"ssm_last_error", "ssm_s6_scan_fwd_workspace_size", "ssm_s6_scan_fwd",
                     "ssm_s6_scan_grouped_fwd", "ssm_s6_scan_fwd_save", "ssm_s6_scan_bwd_saved",
                     "ssm_s6_scan_checkpoint_size", "ssm_s6_scan_grouped_bwd",
                     "ssm_s6_scan_grouped_fwd_save", "ssm_s6_scan_grouped_bwd_saved",
                     "ssm_s6_scan_grouped_bwd_workspace_size",
                     "ssm_s6_fused_fwd", "ssm_causal_conv1d_fwd",
                     "ssm_s6_scan_bwd_workspace_size", "ssm_s6_scan_bwd",
                     "ssd_chunk_scan_fwd_workspace_size", "ssd_chunk_scan_fwd", "ssd_chunk_scan_fwd_noalloc",
                     "ssd_chunk_scan_bwd_workspace_size", "ssd_chunk_scan_bwd",
                     "ssd_trap_chunk_scan_fwd_workspace_size", "ssd_trap_chunk_scan_fwd",
                     "ssd_trap_rotate_qk_workspace_size", "ssd_trap_rotate_qk",
                     "ssd_trap_chunk_scan_bwd_workspace_size", "ssd_trap_chunk_scan_bwd",
                     "ssd_cplx_chunk_scan_fwd_workspace_size", "ssd_cplx_chunk_scan_fwd",
                     "ssd_cplx_mimo_chunk_scan_fwd_workspace_size", "ssd_cplx_mimo_chunk_scan_fwd"}
    for n in names:
        assert hasattr(lib, n), n


def _s6(lib, u=FAKE, dt=FAKE, A_log=FAKE, B=FAKE, C=FAKE, y=FAKE, dims=(2, 8, 16, 4), dtype=0,
        flags=0, dt_bias=None, D=None, h0=None, hf=None, ws=None, wsb=0):
    return lib.ssm_s6_scan_fwd(u, dt, dt_bias, A_log, B, C, D, y, h0, hf, *dims, dtype, flags,
                               ws, wsb, None)


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
    # the Mamba-1 layer shape fills the chip: the sequential walk, no workspace
    assert lib.ssm_s6_scan_fwd_workspace_size(8, 2048, 1536, 16) == 0
    # one batch row at long context: 8 segments of 4096 steps, 96 blocks of 16 channels;
    # workspace = local states (7 segments) + sums of delta + entering states (8 segments)
    need = lib.ssm_s6_scan_fwd_workspace_size(1, 32768, 1536, 16)
    assert need == 7 * 1536 * 16 * 4 + 7 * 1536 * 8 + 8 * 1536 * 16 * 4
    assert lib.ssm_s6_scan_fwd_workspace_size(2, 8192, 1536, 16) > 0
    assert lib.ssm_s6_scan_fwd_workspace_size(1, 1000, 1536, 16) == 0      # too short to split
    assert lib.ssm_s6_scan_fwd_workspace_size(1, 32768, 1536, 32) == 0     # d_state > 16: walk
    dims = (1, 32768, 1536, 16)
    distinct = {n: ctypes.c_void_p(0x100000 * (i + 2)) for i, n in enumerate(("u", "dt", "A_log", "B", "C", "y"))}
    assert _s6(lib, dims=dims, ws=FAKE, wsb=need - 1, **distinct) == WORKSPACE and "workspace" in _err(lib)
    assert _s6(lib, dims=dims, ws=MIS, wsb=need, **distinct) == UNSUPPORTED and "aligned" in _err(lib)


def _s6b(lib, dims=(2, 40, 20, 16), dtype=0, flags=0, ws=ctypes.c_void_p(0x900000), wsb=1 << 40,
         **kw):
    names = ["u", "dt", "dt_bias", "A_log", "B", "C", "D", "h0", "dy", "dh_final",
             "du", "ddt", "dB", "dC", "dA_log", "dD", "ddt_bias", "dh0"]
    required = {"u", "dt", "A_log", "B", "C", "dy", "du", "ddt", "dB", "dC", "dA_log"}
    # distinct aligned fake addresses for the required pointers, NULL for the optional ones
    ptrs = {n: (ctypes.c_void_p(0x100000 * (i + 1)) if n in required else None)
            for i, n in enumerate(names)}
    ptrs.update(kw)
    return lib.ssm_s6_scan_bwd(*(ptrs[n] for n in names), *dims, dtype, flags, ws, wsb, None)


def test_s6_bwd_argument_checks(lib):
    assert _s6b(lib, dy=None) == INVALID and "dy is NULL" in _err(lib)
    assert _s6b(lib, dA_log=None) == INVALID and "dA_log is NULL" in _err(lib)
    assert _s6b(lib, dims=(0, 40, 20, 16)) == INVALID and "batch" in _err(lib)
    assert _s6b(lib, dims=(2, 40, 20, 17)) == UNSUPPORTED and "d_state" in _err(lib)
    assert _s6b(lib, dtype=3) == INVALID and "in_dtype" in _err(lib)
    assert _s6b(lib, flags=0x3) == INVALID and "flags" in _err(lib)
    assert _s6b(lib, dB=MIS) == UNSUPPORTED and "aligned" in _err(lib)
    assert _s6b(lib, du=ctypes.c_void_p(0x100000)) == INVALID and "alias" in _err(lib)   # du == u
    assert _s6b(lib, dD=ctypes.c_void_p(0xB00000)) == INVALID and "alias" in _err(lib)   # dD == du
    need = lib.ssm_s6_scan_bwd_workspace_size(2, 40, 20, 16)
    # the state entering each of the 3 tiles of 16 steps, per (batch, channel, state)
    assert need >= 2 * 3 * 20 * 16 * 4 and need % 256 == 0
    assert _s6b(lib, ws=None) == WORKSPACE and "workspace" in _err(lib)
    assert _s6b(lib, wsb=need - 1) == WORKSPACE
    assert lib.ssm_s6_scan_bwd_workspace_size(0, 40, 20, 16) == 0
    assert lib.ssm_s6_scan_bwd_workspace_size(8, 2048, 1536, 16) >= 8 * 128 * 1536 * 16 * 4


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
    assert _ssd(lib, dims=(1, 64, 1 << 18, 128, 128, 1, 256)) == UNSUPPORTED and "2^24" in _err(lib)
    assert _ssd(lib, dtype=0) == UNSUPPORTED and "bf16" in _err(lib)
    assert _ssd(lib, flags=0x8) == INVALID
    # short sequences run as one segment (no workspace); long ones keep one
    # (P x N) fp32 state per (batch, head, segment) plus a decay per segment
    assert lib.ssd_chunk_scan_fwd_workspace_size(2, 300, 4, 64, 128, 2, 256) == 0
    ws = lib.ssd_chunk_scan_fwd_workspace_size(8, 4096, 24, 64, 128, 1, 256)
    assert ws >= 8 * 24 * 2 * 64 * 128 * 4 and ws % 4 == 0
    assert lib.ssd_chunk_scan_fwd_workspace_size(0, 300, 4, 64, 128, 2, 256) == 0


def _ssdb(lib, dims=(2, 300, 4, 64, 128, 2, 256), dtype=1, flags=1, ws=ctypes.c_void_p(0x9000000),
          wsb=1 << 40, **kw):
    names = ["x", "dt", "dt_bias", "A_log", "B", "C", "D", "h0", "dy", "dh_final",
             "dx", "ddt", "dB", "dC", "dA_log", "dD", "ddt_bias", "dh0"]
    required = {"x", "dt", "A_log", "B", "C", "dy", "dx", "ddt", "dB", "dC", "dA_log"}
    ptrs = {n: (ctypes.c_void_p(0x100000 * (i + 1)) if n in required else None)
            for i, n in enumerate(names)}
    ptrs.update(kw)
    return lib.ssd_chunk_scan_bwd(*(ptrs[n] for n in names), *dims, dtype, flags, ws, wsb, None)


def test_ssd_bwd_argument_checks(lib):
    assert _ssdb(lib, dy=None) == INVALID and "dy is NULL" in _err(lib)
    assert _ssdb(lib, dims=(2, 300, 6, 64, 128, 4, 256)) == INVALID and "ngroups" in _err(lib)
    assert _ssdb(lib, dims=(2, 300, 4, 48, 128, 2, 256)) == UNSUPPORTED and "headdim" in _err(lib)
    assert _ssdb(lib, dims=(2, 300, 4, 64, 256, 2, 256)) == UNSUPPORTED and "d_state" in _err(lib)
    assert _ssdb(lib, dims=(2, 300, 4, 64, 128, 2, 100)) == UNSUPPORTED and "chunk_len" in _err(lib)
    assert _ssdb(lib, dtype=0) == UNSUPPORTED and "bf16" in _err(lib)
    assert _ssdb(lib, flags=0x3) == INVALID
    assert _ssdb(lib, dx=ctypes.c_void_p(0x100000)) == INVALID and "alias" in _err(lib)   # dx == x
    need = lib.ssd_chunk_scan_bwd_workspace_size(2, 300, 4, 64, 128, 2, 256)
    # each head's share of dB and dC: 2 * batch * L * H * N fp32
    assert need >= 2 * 2 * 300 * 4 * 128 * 4
    assert _ssdb(lib, ws=None) == WORKSPACE
    assert _ssdb(lib, wsb=need - 1) == WORKSPACE and "workspace" in _err(lib)


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
    # the workspace holds a 528-byte chunk record and 3 KiB of M tiles per (batch, head,
    # 32-step chunk), and, for long sequences, the segment states
    short = lib.ssd_cplx_chunk_scan_fwd_workspace_size(2, 100, 4, 64, 32, 2, 64)
    assert short >= 2 * 4 * 4 * (528 + 3072)
    assert _cssd(lib, ws=None) == WORKSPACE
    assert _cssd(lib, wsb=short - 1) == WORKSPACE
    long_dims = (4, 8192, 32, 64, 32, 1, 64)
    need = lib.ssd_cplx_chunk_scan_fwd_workspace_size(*long_dims)
    assert need >= 4 * 32 * 2 * 64 * 32 * 2 * 4 + 4 * 32 * 256 * (528 + 3072)
    assert _cssd(lib, dims=long_dims, ws=None) == WORKSPACE
    assert _cssd(lib, dims=long_dims, wsb=need - 1) == WORKSPACE
    # within the element limits, but the per-chunk prep pass would need more than 2^31 - 1
    # work groups (2^32 chunks x 8 groups): refused before any launch
    assert _cssd(lib, dims=(1, 1 << 37, 8, 32, 8, 8, 64)) == UNSUPPORTED and "too large" in _err(lib)


def _s6g(lib, dims=(2, 8, 16, 16, 16), dtype=0, flags=0, y=FAKE, u=FAKE, B=FAKE):
    return lib.ssm_s6_scan_grouped_fwd(u, FAKE, None, FAKE, B, FAKE, None, y, None, None, *dims, dtype, flags,
                                       None)


def test_s6_grouped_argument_checks(lib):
    # every case below fails before any launch (the pointers are fake)
    assert _s6g(lib, dims=(2, 8, 16, 16, 3)) == INVALID and "multiple" in _err(lib)
    assert _s6g(lib, dims=(2, 8, 16, 16, 0)) == INVALID
    assert _s6g(lib, dims=(2, 8, 16, 33, 16)) == UNSUPPORTED and "d_state" in _err(lib)
    assert _s6g(lib, dims=(2, 8, 16, 257, 1)) == UNSUPPORTED and "d_state" in _err(lib)
    assert _s6g(lib, dims=(2, 0, 16, 16, 16)) == INVALID
    assert _s6g(lib, dtype=7) == INVALID and "in_dtype" in _err(lib)
    assert _s6g(lib, flags=0x3) == INVALID
    assert _s6g(lib, flags=0x4) == INVALID
    assert _s6g(lib, y=None) == INVALID
    assert _s6g(lib, y=FAKE, u=FAKE, B=FAKE, flags=0x8) == INVALID


def _fsave(lib, dims=(2, 40, 16, 16), ck=ctypes.c_void_p(0x7000000), y=ctypes.c_void_p(0x6000000), flags=0):
    return lib.ssm_s6_scan_fwd_save(FAKE, FAKE, None, FAKE, FAKE, FAKE, None, y, None, None, ck, *dims, 0, flags,
                                    None)


def _bsaved(lib, ck=ctypes.c_void_p(0xA000000), dims=(2, 40, 16, 16)):
    # a one-byte workspace: a call that passes every other check is refused for it
    o = [ctypes.c_void_p(0x1000000 * (i + 1)) for i in range(8)]
    return lib.ssm_s6_scan_bwd_saved(FAKE, FAKE, None, FAKE, FAKE, FAKE, None, None, FAKE, None, ck, *o, *dims, 0, 0,
                                     ctypes.c_void_p(0x9000000), 1, None)


def test_s6_saved_argument_checks(lib):
    # every case below fails before any launch (the pointers are fake)
    assert lib.ssm_s6_scan_checkpoint_size(2, 40, 16, 16) == 2 * 3 * 16 * 16 * 4
    assert lib.ssm_s6_scan_checkpoint_size(1, 16, 5, 3) == 1 * 1 * 5 * 3 * 4
    assert lib.ssm_s6_scan_checkpoint_size(0, 16, 5, 3) == 0
    assert _fsave(lib, ck=None) == INVALID and "checkpoints" in _err(lib)
    assert _fsave(lib, dims=(2, 40, 16, 17)) == UNSUPPORTED and "d_state" in _err(lib)
    assert _fsave(lib, flags=0x3) == INVALID
    assert _fsave(lib, ck=ctypes.c_void_p(0x6000000)) == INVALID and "alias" in _err(lib)
    assert _fsave(lib, ck=ctypes.c_void_p(0x7000004)) == UNSUPPORTED and "align" in _err(lib)
    assert _bsaved(lib, ck=None) == INVALID and "checkpoints" in _err(lib)
    # a workspace of 1 byte is refused before anything runs
    assert _bsaved(lib) == WORKSPACE and "ssm_s6_scan_bwd_saved" in _err(lib)


def _gbwd(lib, dims=(2, 40, 32, 16, 32), wsb=1, dtype=0):
    o = [ctypes.c_void_p(0x1000000 * (i + 1)) for i in range(8)]
    return lib.ssm_s6_scan_grouped_bwd(FAKE, FAKE, None, FAKE, FAKE, FAKE, None, None, FAKE, None, *o, *dims, dtype,
                                       0, ctypes.c_void_p(0x9000000), wsb, None)


def test_s6_grouped_bwd_argument_checks(lib):
    # every case below fails before any launch (the pointers are fake)
    assert _gbwd(lib, dims=(2, 40, 32, 16, 5)) == INVALID and "multiple" in _err(lib)
    assert _gbwd(lib, dims=(2, 40, 32, 17, 32)) == UNSUPPORTED and "d_state" in _err(lib)
    assert _gbwd(lib, dims=(2, 40, 32, 16, 0)) == INVALID
    assert _gbwd(lib, dtype=5) == INVALID
    assert _gbwd(lib) == WORKSPACE and "ssm_s6_scan_grouped_bwd" in _err(lib)
    # per channel: checkpoints and partials; groups of several channels add the shares
    pc = lib.ssm_s6_scan_grouped_bwd_workspace_size(2, 40, 32, 16, 32)
    grp = lib.ssm_s6_scan_grouped_bwd_workspace_size(2, 40, 32, 16, 8)
    assert pc >= 2 * 3 * 32 * 16 * 4 and grp >= pc + 2 * 2 * 40 * 32 * 16 * 4
    assert lib.ssm_s6_scan_grouped_bwd_workspace_size(2, 40, 32, 16, 1) == lib.ssm_s6_scan_bwd_workspace_size(
        2, 40, 32, 16)


def _mimo(lib, dims=(2, 100, 4, 4, 64, 32, 2, 64), flags=0, ws=FAKE, wsb=1 << 40):
    return lib.ssd_cplx_mimo_chunk_scan_fwd(FAKE, FAKE, None, FAKE, FAKE, FAKE, None,
                                            ctypes.c_void_p(0x200000), None, None, *dims, flags, ws, wsb,
                                            None)


def test_cssd_mimo_argument_checks(lib):
    # every case below fails before any launch (the pointers are fake)
    assert _mimo(lib, dims=(2, 100, 3, 4, 64, 32, 2, 64)) == UNSUPPORTED and "rank" in _err(lib)
    assert _mimo(lib, dims=(2, 100, 32, 4, 64, 32, 2, 64)) == UNSUPPORTED and "rank" in _err(lib)
    assert _mimo(lib, dims=(2, 100, 0, 4, 64, 32, 2, 64)) == UNSUPPORTED
    assert _mimo(lib, dims=(2, 100, 4, 4, 64, 32, 3, 64)) == INVALID
    assert _mimo(lib, dims=(2, 100, 4, 4, 40, 32, 2, 64)) == UNSUPPORTED and "headdim" in _err(lib)
    assert _mimo(lib, dims=(2, 100, 4, 4, 64, 30, 2, 64)) == UNSUPPORTED and "n_complex" in _err(lib)
    assert _mimo(lib, dims=(2, 100, 4, 4, 64, 32, 2, 256)) == UNSUPPORTED and "chunk_len" in _err(lib)
    assert _mimo(lib, dims=(2, 0, 4, 4, 64, 32, 2, 64)) == INVALID
    assert _mimo(lib, flags=0x4) == INVALID and "stable" in _err(lib)
    assert _mimo(lib, flags=0x8) == INVALID
    assert _mimo(lib, flags=0x3) == INVALID
    # the workspace covers L x rank rows: the complex SSD's over that length
    dims = (4, 2048, 4, 32, 64, 32, 1, 64)
    need = lib.ssd_cplx_mimo_chunk_scan_fwd_workspace_size(*dims)
    assert need == lib.ssd_cplx_chunk_scan_fwd_workspace_size(4, 8192, 32, 64, 32, 1, 64) > 0
    assert (lib.ssd_cplx_mimo_chunk_scan_fwd_workspace_size(2, 25, 4, 4, 64, 32, 2, 64) ==
            lib.ssd_cplx_chunk_scan_fwd_workspace_size(2, 100, 4, 64, 32, 2, 64))
    assert _mimo(lib, dims=dims, ws=None) == WORKSPACE
    assert _mimo(lib, dims=dims, wsb=need - 1) == WORKSPACE
    assert _mimo(lib, dims=(1, 1 << 35, 4, 8, 32, 8, 8, 64)) == UNSUPPORTED and "too large" in _err(lib)


def _trap(lib, dims=(2, 300, 4, 64, 128, 64), dtype=1, ws=ctypes.c_void_p(0x9000000), wsb=1 << 40,
          **kw):
    names = ["x", "k", "q", "dt", "a", "trap", "D", "y", "h0", "k_prev", "x_prev", "h_final"]
    required = {"x", "k", "q", "dt", "a", "trap", "y"}
    ptrs = {n: (ctypes.c_void_p(0x100000 * (i + 1)) if n in required else None)
            for i, n in enumerate(names)}
    ptrs.update(kw)
    return lib.ssd_trap_chunk_scan_fwd(*(ptrs[n] for n in names), *dims, dtype, ws, wsb, None)


def test_trap_argument_checks(lib):
    assert _trap(lib, trap=None) == INVALID and "trap is NULL" in _err(lib)
    assert _trap(lib, q=None) == INVALID and "q is NULL" in _err(lib)
    assert _trap(lib, dims=(2, 0, 4, 64, 128, 64)) == INVALID and "L" in _err(lib)
    assert _trap(lib, dims=(2, 300, 4, 48, 128, 64)) == UNSUPPORTED and "headdim" in _err(lib)
    assert _trap(lib, dims=(2, 300, 4, 64, 96 + 8, 64)) == UNSUPPORTED and "d_state" in _err(lib)
    assert _trap(lib, dims=(2, 300, 4, 64, 128, 32)) == UNSUPPORTED and "chunk_len" in _err(lib)
    assert _trap(lib, dtype=0) == UNSUPPORTED and "bf16" in _err(lib)
    assert _trap(lib, dtype=5) == INVALID and "in_dtype" in _err(lib)
    # the carried previous input comes as a pair
    assert _trap(lib, k_prev=ctypes.c_void_p(0xA000000)) == INVALID and "together" in _err(lib)
    assert _trap(lib, a=MIS) == UNSUPPORTED and "aligned" in _err(lib)
    assert _trap(lib, y=ctypes.c_void_p(0x200000)) == INVALID and "alias" in _err(lib)       # y == k
    assert _trap(lib, h_final=ctypes.c_void_p(0x600000)) == INVALID and "alias" in _err(lib)  # == trap
    need = lib.ssd_trap_chunk_scan_fwd_workspace_size(2, 300, 4, 64, 128, 64)
    # always at least the entering state with the carried input folded in
    assert need >= 2 * 4 * 64 * 128 * 4
    assert _trap(lib, ws=None) == WORKSPACE and "workspace" in _err(lib)
    assert _trap(lib, wsb=need - 1) == WORKSPACE
    assert lib.ssd_trap_chunk_scan_fwd_workspace_size(2, 0, 4, 64, 128, 64) == 0


def _rot(lib, dims=(2, 300, 4, 128, 64), dtype=1, ws=ctypes.c_void_p(0x9000000), wsb=1 << 40, **kw):
    names = ["k_raw", "q_raw", "angles", "dt", "angle_state", "k", "q", "angle_state_out"]
    required = {"k_raw", "q_raw", "angles", "dt", "k", "q"}
    ptrs = {n: (ctypes.c_void_p(0x100000 * (i + 1)) if n in required else None)
            for i, n in enumerate(names)}
    ptrs.update(kw)
    return lib.ssd_trap_rotate_qk(*(ptrs[n] for n in names), *dims, dtype, ws, wsb, None)


def test_rotate_argument_checks(lib):
    assert _rot(lib, dt=None) == INVALID and "dt is NULL" in _err(lib)
    assert _rot(lib, angles=None) == INVALID and "angles is NULL" in _err(lib)
    assert _rot(lib, dims=(2, 300, 4, 127, 60)) == UNSUPPORTED and "even" in _err(lib)
    assert _rot(lib, dims=(2, 300, 4, 128, 65)) == INVALID and "n_angles" in _err(lib)
    assert _rot(lib, dims=(2, 300, 4, 128, -1)) == INVALID and "n_angles" in _err(lib)
    assert _rot(lib, dims=(2, 0, 4, 128, 64)) == INVALID
    assert _rot(lib, dtype=0) == UNSUPPORTED and "bf16" in _err(lib)
    assert _rot(lib, k=ctypes.c_void_p(0x700000)) == INVALID and "k aliases" in _err(lib)      # k == q
    assert _rot(lib, q=ctypes.c_void_p(0x100000)) == INVALID and "q aliases" in _err(lib)      # q == k_raw
    assert _rot(lib, angle_state_out=ctypes.c_void_p(0x400000)) == INVALID                      # == dt
    assert _rot(lib, angles=MIS) == UNSUPPORTED and "aligned" in _err(lib)
    need = lib.ssd_trap_rotate_qk_workspace_size(2, 300, 4, 128, 64)
    assert need >= 2 * 4 * 64 * 4
    assert _rot(lib, ws=None) == WORKSPACE and "workspace" in _err(lib)
    assert _rot(lib, wsb=need - 1) == WORKSPACE
    assert lib.ssd_trap_rotate_qk_workspace_size(2, 300, 4, 128, -1) == 0


def _fused(lib, dims=(2, 40, 20, 16, 4), dtype=0, flags=0, **kw):
    names = ["x", "conv_w", "conv_b", "conv_state", "z", "dt", "dt_bias", "A_log", "B", "C", "D", "y",
             "h0", "h_final", "u_out", "conv_state_out"]
    required = {"x", "conv_w", "dt", "A_log", "B", "C", "y"}
    ptrs = {n: (ctypes.c_void_p(0x100000 * (i + 1)) if n in required else None)
            for i, n in enumerate(names)}
    ptrs.update(kw)
    return lib.ssm_s6_fused_fwd(*(ptrs[n] for n in names), *dims, dtype, flags, None)


def test_fused_argument_checks(lib):
    assert _fused(lib, conv_w=None) == INVALID and "conv_w is NULL" in _err(lib)
    assert _fused(lib, x=None) == INVALID and "x is NULL" in _err(lib)
    assert _fused(lib, dims=(2, 40, 20, 16, 0)) == INVALID and "d_conv" in _err(lib)
    assert _fused(lib, dims=(2, 40, 20, 16, 5)) == UNSUPPORTED and "d_conv" in _err(lib)
    assert _fused(lib, dims=(2, 40, 20, 300, 4)) == UNSUPPORTED and "d_state" in _err(lib)
    assert _fused(lib, dtype=4) == INVALID and "in_dtype" in _err(lib)
    assert _fused(lib, flags=0x3) == INVALID and "flags" in _err(lib)
    assert _fused(lib, z=MIS) == UNSUPPORTED and "aligned" in _err(lib)
    assert _fused(lib, y=ctypes.c_void_p(0x100000)) == INVALID and "alias" in _err(lib)            # y == x
    assert _fused(lib, u_out=ctypes.c_void_p(0xC00000)) == INVALID and "alias" in _err(lib)        # == y
    assert _fused(lib, conv_state_out=ctypes.c_void_p(0x200000)) == INVALID and "alias" in _err(lib)  # == conv_w


def _conv(lib, dims=(2, 40, 24, 4), silu=1, dtype=1, **kw):
    names = ["x", "w", "bias", "state_in", "y", "state_out"]
    required = {"x", "w", "y"}
    ptrs = {n: (ctypes.c_void_p(0x100000 * (i + 1)) if n in required else None) for i, n in enumerate(names)}
    ptrs.update(kw)
    return lib.ssm_causal_conv1d_fwd(*(ptrs[n] for n in names), *dims, silu, dtype, None)


def test_conv1d_argument_checks(lib):
    assert _conv(lib, w=None) == INVALID and "w is NULL" in _err(lib)
    assert _conv(lib, dims=(2, 40, 24, 0)) == INVALID and "d_conv" in _err(lib)
    assert _conv(lib, dims=(2, 40, 24, 5)) == UNSUPPORTED and "d_conv" in _err(lib)
    assert _conv(lib, dims=(2, 0, 24, 4)) == INVALID
    assert _conv(lib, silu=2) == INVALID and "silu" in _err(lib)
    assert _conv(lib, dtype=9) == INVALID and "dtype" in _err(lib)
    assert _conv(lib, bias=MIS) == UNSUPPORTED and "aligned" in _err(lib)
    assert _conv(lib, y=ctypes.c_void_p(0x100000)) == INVALID and "alias" in _err(lib)            # y == x
    assert _conv(lib, state_out=ctypes.c_void_p(0x500000)) == INVALID and "alias" in _err(lib)    # == y


def _trapb(lib, dims=(2, 300, 4, 64, 128, 64), dtype=1, ws=ctypes.c_void_p(0x9000000), wsb=1 << 40, **kw):
    names = ["x", "k", "q", "dt", "a", "trap", "D", "h0", "k_prev", "x_prev", "dy", "dh_final",
             "dx", "dk", "dq", "ddt", "da", "dtrap", "dD", "dh0", "dk_prev", "dx_prev"]
    required = {"x", "k", "q", "dt", "a", "trap", "dy", "dx", "dk", "dq", "ddt", "da", "dtrap"}
    ptrs = {n: (ctypes.c_void_p(0x100000 * (i + 1)) if n in required else None) for i, n in enumerate(names)}
    ptrs.update(kw)
    return lib.ssd_trap_chunk_scan_bwd(*(ptrs[n] for n in names), *dims, dtype, ws, wsb, None)


def test_trap_bwd_argument_checks(lib):
    assert _trapb(lib, dy=None) == INVALID and "dy is NULL" in _err(lib)
    assert _trapb(lib, dtrap=None) == INVALID and "dtrap is NULL" in _err(lib)
    assert _trapb(lib, dims=(2, 300, 4, 48, 128, 64)) == UNSUPPORTED and "headdim" in _err(lib)
    assert _trapb(lib, dims=(2, 300, 4, 64, 256, 64)) == UNSUPPORTED and "d_state" in _err(lib)
    assert _trapb(lib, dims=(2, 300, 4, 64, 128, 32)) == UNSUPPORTED and "chunk_len" in _err(lib)
    assert _trapb(lib, dtype=0) == UNSUPPORTED and "bf16" in _err(lib)
    assert _trapb(lib, x_prev=ctypes.c_void_p(0xA000000)) == INVALID and "together" in _err(lib)
    assert _trapb(lib, dx=ctypes.c_void_p(0x100000)) == INVALID and "alias" in _err(lib)      # dx == x
    assert _trapb(lib, da=MIS) == UNSUPPORTED and "aligned" in _err(lib)
    need = lib.ssd_trap_chunk_scan_bwd_workspace_size(2, 300, 4, 64, 128, 64)
    assert need >= 2 * 2 * 4 * 64 * 128 * 4
    assert _trapb(lib, ws=None) == WORKSPACE
    assert _trapb(lib, wsb=need - 1) == WORKSPACE and "workspace" in _err(lib)


def _gfsave(lib, dims=(2, 40, 32, 16, 32), ck=ctypes.c_void_p(0x7000000), y=ctypes.c_void_p(0x6000000)):
    return lib.ssm_s6_scan_grouped_fwd_save(FAKE, FAKE, None, FAKE, FAKE, FAKE, None, y, None, None, ck, *dims, 0,
                                            0, None)


def _gbsaved(lib, ck=ctypes.c_void_p(0xA000000), dims=(2, 40, 32, 16, 32)):
    # a one-byte workspace: a call that passes every other check is refused for it
    o = [ctypes.c_void_p(0x1000000 * (i + 1)) for i in range(8)]
    return lib.ssm_s6_scan_grouped_bwd_saved(FAKE, FAKE, None, FAKE, FAKE, FAKE, None, None, FAKE, None, ck, *o,
                                             *dims, 0, 0, ctypes.c_void_p(0x9000000), 1, None)


def test_s6_grouped_saved_argument_checks(lib):
    # every case below fails before any launch (the pointers are fake)
    assert _gfsave(lib, dims=(2, 40, 32, 16, 5)) == INVALID and "multiple" in _err(lib)
    assert _gfsave(lib, dims=(2, 40, 32, 17, 32)) == UNSUPPORTED and "d_state" in _err(lib)
    assert _gfsave(lib, dims=(2, 40, 32, 16, 0)) == INVALID
    assert _gfsave(lib, ck=None) == INVALID and "checkpoints" in _err(lib)
    assert _gfsave(lib, ck=ctypes.c_void_p(0x6000000)) == INVALID and "alias" in _err(lib)
    assert _gfsave(lib, ck=ctypes.c_void_p(0x7000004)) == UNSUPPORTED and "align" in _err(lib)
    assert "ssm_s6_scan_grouped_fwd_save" in _err(lib)
    assert _gbsaved(lib, ck=None) == INVALID and "checkpoints" in _err(lib)
    assert _gbsaved(lib, dims=(2, 40, 32, 16, 5)) == INVALID and "multiple" in _err(lib)
    assert _gbsaved(lib) == WORKSPACE and "ssm_s6_scan_grouped_bwd_saved" in _err(lib)


def test_ssd_noalloc_argument_checks(lib):
    """The no-allocation SSD entry validates like ssd_chunk_scan_fwd, and a shape whose
    segment states exceed the static scratch is rejected before any HIP call."""
    P = ctypes.c_void_p
    lib.ssd_chunk_scan_fwd_noalloc.argtypes = [P] * 10 + [ctypes.c_int64] * 7 + [ctypes.c_int, ctypes.c_uint32, P]
    lib.ssd_chunk_scan_fwd_noalloc.restype = ctypes.c_int
    ptr = {n: ctypes.c_void_p(0x100000 * (i + 2)) for i, n in enumerate(("x", "dt", "A_log", "B", "C", "y"))}

    def call(dims, dtype=1, flags=1, **kw):
        p = dict(ptr, **kw)
        return lib.ssd_chunk_scan_fwd_noalloc(p["x"], p["dt"], None, p["A_log"], p["B"], p["C"], None, p["y"],
                                              None, None, *dims, dtype, flags, None)
    # the long-context shape needs ~100 MB of segment states: more than the 32 MiB scratch
    long_dims = (2, 32768, 80, 64, 128, 8, 256)
    need = lib.ssd_chunk_scan_fwd_workspace_size(*long_dims)
    assert need > 32 << 20
    assert call(long_dims) == WORKSPACE and "scratch" in _err(lib)
    assert call((1, 64, 2, 64, 128, 1, 256), x=None) == INVALID and "x is NULL" in _err(lib)
    assert call((1, 64, 3, 64, 128, 2, 256)) == INVALID                       # nheads % ngroups
    assert call((1, 64, 2, 48, 128, 1, 256)) == UNSUPPORTED and "headdim" in _err(lib)
    assert call((1, 64, 2, 64, 128, 1, 256), dtype=0) == UNSUPPORTED
    assert call((1, 64, 2, 64, 128, 1, 256), y=ptr["x"]) == INVALID and "alias" in _err(lib)
