"""Build libfa.so in-tree with hipcc for gfx950.

Run ``python exact_io_aware_63_amd/build.py`` (or ``__graft_entry__.build()``).
It imports nothing from the package, so it runs before libfa.so exists.
Each source is compiled to its own object in ``_build/`` (in parallel), then
the objects are linked into the shared library.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfa.so")
OBJ_DIR = os.path.join(os.path.dirname(PKG), "_build")
# (source, object name, extra defines): each bf16 kernel source is compiled
# once per (head width, causal) instance.
SOURCES = [("fa_api.cpp", "fa_api", []), ("fa_fwd_fp32.hip", "fa_fwd_fp32", [])] + [
    (f"fa_{pas}_bf16.hip", f"fa_{pas}_bf16_d{d}_c{c}", [f"-DFA_BF16_D={d}", f"-DFA_BF16_CAUSAL={c}"])
    for pas in ("fwd", "bwd") for d in (128, 64) for c in (1, 0)] + [
    ("fa_decode_bf16.hip", "fa_decode_bf16", []), ("fa_fwd_fp8.hip", "fa_fwd_fp8", [])]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # packed fp32 VALU ops are kept off (v_pk_* fp32 forms are not used)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def _noise_free(text: str) -> str:
    return "\n".join(ln for ln in text.splitlines()
                     if ln.strip() and "packed-fp32-ops" not in ln
                     and "not a recognized feature" not in ln)


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every HIP/C++ source of the library and link ``libfa.so``."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    procs = []
    objs = []
    for src, name, defines in SOURCES:
        obj = os.path.join(OBJ_DIR, name + ".o")
        cmd = [HIPCC, *FLAGS, *defines, *(extra_flags or []), "-c", "-o", obj,
               os.path.join(CSRC, src)]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((name, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                            text=True)))
        objs.append(obj)
    failed = []
    for src, proc in procs:
        out, _ = proc.communicate()
        msg = _noise_free(out)
        if proc.returncode != 0:
            failed.append(src)
            sys.stderr.write(out)
        elif verbose and msg:
            print(msg)
    if failed:
        raise RuntimeError(f"hipcc failed on {', '.join(failed)}")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc link failed with exit code {res.returncode}")
    os.replace(tmp, LIB)
    return LIB


SANITIZED_LIB = os.path.join(OBJ_DIR, "libfa_sanitized.so")


def build_sanitized(verbose: bool = False) -> str:
    """Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the C
    ABI layer: ``fa_api.cpp`` is compiled with g++ and the sanitizers (host
    code only; the kernel objects of ``build()`` are linked as they are) into
    ``_build/libfa_sanitized.so``. Load it with the ASan runtime preloaded and
    ``FA_LIBRARY`` pointing at it to run the ABI tests under the sanitizers."""
    objs = [os.path.join(OBJ_DIR, name + ".o") for _, name, _ in SOURCES if name != "fa_api"]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        raise FileNotFoundError(f"kernel objects missing (run build() first): {missing[:2]}")
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(HIPCC)))
    api_obj = os.path.join(OBJ_DIR, "fa_api_sanitized.o")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer"]
    steps = [
        ["g++", "-std=c++17", "-O1", "-g", "-fPIC", *san, "-D__HIP_PLATFORM_AMD__",
         f"-I{rocm}/include", "-c", "-o", api_obj, os.path.join(CSRC, "fa_api.cpp")],
        ["g++", "-shared", "-fPIC", *san, "-o", SANITIZED_LIB, api_obj, *objs,
         f"-L{rocm}/lib", "-lamdhip64", f"-Wl,-rpath,{rocm}/lib"],
    ]
    for cmd in steps:
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"sanitized build failed: {cmd[0]} exit {res.returncode}")
    return SANITIZED_LIB


if __name__ == "__main__":
    build(verbose=True)
