"""Build libdita.so (HIP for gfx950 + host C++) in-tree with hipcc.

Usage: ``python partial_state_reuse_amd/build.py [-v]`` (run as a script, so that
importing the package -- which loads the library -- is never needed to build
it), or ``build()`` after loading this file by path.  Every call recompiles
every source, then checks that the linked library leaves no symbol of its own
undefined.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdita.so")

HIP_SOURCES = ["api.hip", "attn_bf16.hip", "attn_f32.hip", "compact.hip", "merge.hip", "stats.hip"]
CXX_SOURCES = ["planner.cpp", "error_planner.cpp"]
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    # Keep the compiler from forming packed fp32 VALU ops (v_pk_*_f32).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
CXX_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-Wall"]


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else (shutil.which("hipcc") or "hipcc")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(ln for ln in r.stdout.splitlines() if "packed-fp32-ops" not in ln)
    return r.returncode, out, cmd


def build(verbose: bool = False, extra_hip_flags=()) -> str:
    os.makedirs(OBJ, exist_ok=True)
    hipcc = _hipcc()
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(OBJ, src + ".o")
        jobs.append([hipcc, *HIP_FLAGS, *extra_hip_flags, "-c", os.path.join(CSRC, src), "-o", obj])
    for src in CXX_SOURCES:
        obj = os.path.join(OBJ, src + ".o")
        jobs.append(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        results = list(ex.map(_run, jobs))
    for rc, out, cmd in results:
        if verbose or rc:
            sys.stderr.write(" ".join(cmd) + "\n" + out + "\n")
        if rc:
            raise RuntimeError(f"compile failed: {cmd[-3]}")
    objs = [os.path.join(OBJ, s + ".o") for s in HIP_SOURCES + CXX_SOURCES]
    tmp = LIB + ".tmp"
    rc, out, cmd = _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-o", tmp, *objs])
    if rc:
        sys.stderr.write(out + "\n")
        raise RuntimeError("link failed")
    _check_symbols(tmp)
    os.replace(tmp, LIB)
    return LIB


def _check_symbols(lib: str) -> None:
    """Fail on undefined symbols of the library's own (e.g. a kernel launch stub the
    host pass did not emit): dlopen would reject such a library at run time."""
    r = subprocess.run(["nm", "-u", "-C", lib], stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True)
    bad = [ln.strip() for ln in r.stdout.splitlines()
           if "dita" in ln or "__device_stub" in ln]
    if r.returncode or bad:
        raise RuntimeError("libdita.so has undefined symbols of its own:\n" + "\n".join(bad))


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
