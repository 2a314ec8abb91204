"""Build the native library ``libmamba_scan.so`` in-tree with hipcc for gfx950.

Each source is compiled to an object in ``_build/`` in parallel and the
objects are linked into ``selective_state_space_56_amd/libmamba_scan.so``.
Packed-FP32 instructions are disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmamba_scan.so")
ARCH = "gfx950"

SOURCES = ["api.cpp", "scan_fwd.hip", "scan_split.hip", "scan_bwd.hip", "state_update.hip", "conv1d.hip", "ssd.hip"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]
DEVICE = ["-x", "hip", "--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", "-ffp-contract=fast"]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found; the HIP toolchain is required to build libmamba_scan.so")
    return p


def rocm_path() -> str:
    return os.environ.get("ROCM_PATH", "/opt/rocm")


def _stale(src: str, obj: str) -> bool:
    """Whether obj is older than src or any header under csrc/ or include/."""
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    deps = [os.path.join(CSRC, src)] + [os.path.join(d, f) for d in (CSRC, INCLUDE)
                                        for f in os.listdir(d) if f.endswith(".h")]
    return any(os.path.getmtime(p) > t for p in deps)


def _compile(src: str, incremental: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    if incremental and not _stale(src, obj):
        return obj
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [hipcc()] + COMMON + DEVICE + ["-c", path, "-o", obj]
    else:
        cmd = [hipcc()] + COMMON + ["-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I",
                                    os.path.join(rocm_path(), "include"), "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, incremental: bool = False) -> str:
    """Compile every source (with incremental=True only those newer than
    their object) and link the shared library. Returns its path."""
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, incremental), SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, incremental="--incremental" in sys.argv)
    sys.exit(0)
