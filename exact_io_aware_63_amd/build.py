"""Build libfa.so in-tree with hipcc for gfx950.

Run ``python exact_io_aware_63_amd/build.py`` (or ``__graft_entry__.build()``).
It imports nothing from the package, so it runs before libfa.so exists.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfa.so")
SOURCES = ["fa_api.cpp", "fa_fwd_bf16.hip", "fa_fwd_fp32.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 VALU ops are kept off (v_pk_* fp32 forms are not used)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every HIP/C++ source of the library into ``libfa.so``."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *(extra_flags or []), "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    noise = [ln for ln in (res.stdout + res.stderr).splitlines()
             if ln.strip() and "packed-fp32-ops" not in ln and "not a recognized feature" not in ln]
    if verbose and noise:
        print("\n".join(noise))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
