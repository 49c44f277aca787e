"""Build libsmla.so (HIP kernels + C ABI) in-tree for gfx950.

    python -m sparse_mla_decode_fp8_amd.build          # or build.build()

The library is written next to this file; the Python binding loads it from
there.  Every call recompiles (a few seconds).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsmla.so")
SOURCES = ["smla_kernels.hip", "smla_wide.hip", "smla_wide64.hip", "smla_v41.hip", "smla_noalloc.hip", "smla_qk_probe.hip", "smla_api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsmla.so)")


def command(out: str, extra=()) -> list:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # packed fp32 VALU forms are kept out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
        # scalar kernel arguments are preloaded into SGPRs at wave launch
        "-mllvm", "-amdgpu-kernarg-preload-count=16",
        "-I", INCLUDE, "-I", CSRC,
        *[os.path.join(CSRC, s) for s in SOURCES],
        *extra,
        "-o", out,
    ]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if res.returncode != 0:
        raise RuntimeError(f"libsmla build failed:\n{' '.join(cmd)}\n{msgs}")
    if verbose and msgs:
        print(msgs, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
