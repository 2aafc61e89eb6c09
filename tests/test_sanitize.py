"""CPU sanitizer tier: the oracle and the C ABI's host code built with host
sanitizers and driven on the CPU.

  - oracle/llref.c with AddressSanitizer + UndefinedBehaviorSanitizer (gcc),
    every entry point on small and degenerate shapes (tests/sanitize/oracle_driver.c);
  - fenwick_tree_linear_amd/csrc/api.cpp (validation, workspace planning, the
    launch sequence, kernel timing) with AddressSanitizer + UBSan and, in a
    second build, ThreadSanitizer, the kernel launchers replaced by stubs that
    report a failed launch (tests/sanitize/launch_stubs.cpp), so no GPU is
    touched; the driver (tests/sanitize/abi_driver.cpp) hits every validation
    error and toggles kernel timing from one thread while another calls.

The sanitizers instrument host code only (each -fsanitize= follows
-Xarch_host on the hipcc lines); no GPU code is built with them.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "fenwick_tree_linear_amd", "csrc")
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    return r.returncode, r.stdout + r.stderr


def test_oracle_under_asan_ubsan(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_san")
    rc, out = run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                   "-fno-sanitize-recover=undefined", "-std=c11", "-fopenmp", "-o", exe,
                   os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "llref.c"), "-lm"])
    assert rc == 0, out
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", OMP_NUM_THREADS="4")
    rc, out = run([exe], env=env)
    assert rc == 0 and "Sanitizer" not in out and "runtime error" not in out, out


def _build_abi(tmp_path, name, sanitizers):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / name)
    flags = []
    for s in sanitizers:
        flags += ["-Xarch_host", f"-fsanitize={s}"]
    cmd = [HIPCC, "-O1", "-g", "-std=c++17", "--offload-arch=gfx950", "-x", "hip", *flags,
           "-Xarch_host", "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "api.cpp"), os.path.join(SAN, "launch_stubs.cpp"), os.path.join(SAN, "abi_driver.cpp"),
           "-o", exe, *flags]
    rc, out = run(cmd)
    assert rc == 0, out
    return exe


def test_abi_host_code_under_asan_ubsan(tmp_path):
    exe = _build_abi(tmp_path, "abi_asan", ["address", "undefined"])
    rc, out = run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1"))
    assert rc == 0 and "Sanitizer" not in out and "runtime error" not in out, out


def test_abi_host_code_under_tsan(tmp_path):
    exe = _build_abi(tmp_path, "abi_tsan", ["thread"])
    rc, out = run([exe], env=dict(os.environ, TSAN_OPTIONS="halt_on_error=1"))
    assert rc == 0 and "ThreadSanitizer" not in out, out
