"""The C ABI tests again, against a build of the host layer with
AddressSanitizer and UndefinedBehaviorSanitizer (g++, host code only), so
that an out-of-bounds host access, a signed overflow or a misaligned load in
the argument checks fails the run. CPU only: no kernel is launched."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_tests_pass_under_host_sanitizers():
    import shutil
    if shutil.which("g++") is None:
        pytest.skip("g++ not found")
    asan = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("no AddressSanitizer runtime")
    sys.path.insert(0, os.path.join(ROOT, "exact_io_aware_63_amd"))
    try:
        import build as fa_build
    finally:
        sys.path.pop(0)
    try:
        lib = fa_build.build_sanitized()
    except FileNotFoundError as e:
        pytest.skip(str(e))
    env = dict(os.environ)
    env["FA_LIBRARY"] = lib
    # the ASan runtime must come first among preloaded libraries
    env["LD_PRELOAD"] = " ".join(x for x in (asan, env.get("LD_PRELOAD", "")) if x)
    # the interpreter itself is not instrumented: leak reports would be its own
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py")], env=env, cwd=ROOT,
                         capture_output=True, text=True, timeout=600)
    tail = (res.stdout + res.stderr)[-3000:]
    assert res.returncode == 0, tail
    assert "passed" in res.stdout
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, tail
