"""Build the gfx950 shared library ``libpa_mi355x.so`` in-tree with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(HERE, "libpa_mi355x.so")
SOURCES = [os.path.join(CSRC, "pa_kernels.hip"), os.path.join(CSRC, "pa_api.cpp"), os.path.join(CSRC, "pa_noalloc.hip")]
HEADERS = [os.path.join(CSRC, "pa_internal.h"), os.path.join(INCLUDE, "pa.h")]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def command(out: str) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            # no packed-fp32 instructions in the device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC, *SOURCES, "-o", out]


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 into ``libpa_mi355x.so`` (always recompiles)."""
    tmp = LIB_PATH + ".tmp"
    proc = subprocess.run(command(tmp), capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + proc.stdout + proc.stderr)
    if verbose:
        print(proc.stdout + proc.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def is_stale() -> bool:
    if not os.path.exists(LIB_PATH):
        return True
    t = os.path.getmtime(LIB_PATH)
    return any(os.path.getmtime(p) > t for p in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose=True))
