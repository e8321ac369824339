"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the
CPU: the oracle (every function on edge inputs, tests/sanitize/
oracle_checks.c) and the C ABI's argument checks (zs_abi.hip built
host-only, every rejected call and zero-length no-op, with launchers that
abort if reached, tests/sanitize/abi_checks.cpp).  Any out-of-bounds access,
leak (oracle), or undefined behaviour fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(exe, env):
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr[-4000:]
    return r.stdout


def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_checks")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-I", os.path.join(ROOT, "oracle"), os.path.join(ROOT, "oracle", "oracle.c"),
                    os.path.join(SAN, "oracle_checks.c"), "-lm", "-o", exe], check=True)
    _run(exe, ENV)


def test_abi_argument_checks_under_asan_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    exe = str(tmp_path / "abi_checks")
    csrc = os.path.join(ROOT, "zero_sharded_mixed_step_amd", "csrc")
    # host code only (no kernels in zs_abi.hip); each sanitizer flag goes to
    # the host compilation alone
    subprocess.run([HIPCC, "--cuda-host-only", "-O1", "-g", "-std=c++17",
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    "-Xarch_host", "-fno-sanitize-recover=all",
                    "-I", os.path.join(ROOT, "include"), "-I", csrc,
                    os.path.join(csrc, "zs_abi.hip"), os.path.join(SAN, "abi_checks.cpp"),
                    "-o", exe], check=True, capture_output=True)
    # the HIP runtime's own allocations are not the library's: no leak check
    _run(exe, dict(ENV, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1"))
