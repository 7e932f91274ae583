"""Build libssmscan.so (gfx950) from the HIP sources in csrc/.

Usage: python selective_state_space_s6_amd/build.py   (or __graft_entry__.build())
Each source is compiled to an object in parallel, then linked into a shared
library next to this file.  Always recompiles (no staleness heuristics).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libssmscan.so")
SOURCES = ["abi.hip", "s6_scan.hip", "s6_seg.hip", "s6_fused.hip", "s6_decode.hip", "s6_bwd.hip", "ssd_scan.hip", "ssd_decode.hip", "ssd_bwd.hip", "cssd_scan.hip",
           "trap_rotate.hip", "conv1d.hip", "s6_grouped.hip", "scratch.hip"]
ARCH = os.environ.get("SSM_OFFLOAD_ARCH", "gfx950")
# Packed fp32 ops are switched off: the compiler must not emit v_pk_{add,mul,fma}_f32.
# MFMA accumulators are kept in ordinary VGPRs, so the fp32 state that the SSD
# kernels scale and split between contractions needs no AGPR round trips.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-mfma-vgpr-form=1",
          "-Wno-unused-command-line-argument"]


def _hipcc() -> str:
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str, obj: str) -> None:
    cmd = [_hipcc(), *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")


def build(verbose: bool = True) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, s.replace(".hip", ".o")) for s in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        list(ex.map(lambda so: _compile(*so), zip(SOURCES, objs)))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
