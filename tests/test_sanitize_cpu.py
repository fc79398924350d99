"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only,
no GPU call):

* the oracle (oracle/oracle.c, gcc) over small problems of every operator,
  their degenerate shapes and their error returns, with leak checking;
* the C ABI's argument validation (abi.cpp, its host code instrumented)
  over rejection cases of every entry point, the workspace queries and the
  status strings, linked against the library's device objects.

Each runs as its own executable (tests/sanitize/*_driver.*); a sanitizer
report or a wrong return code fails the test.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVERS = os.path.join(ROOT, "tests", "sanitize")
BUILD = os.path.join(ROOT, "computation_collective_amd", "_build")
DEVICE_OBJECTS = ["gemm_rs.o", "gemv_ar.o", "ag_gemm.o", "embbag_a2a.o", "gemm_a2a.o", "a2a_gemm.o"]
# sanitizers on the host side of hipcc's compilation only
HOST_SAN = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-omit-frame-pointer".split()
ENV = dict(os.environ, ASAN_OPTIONS="halt_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
           OMP_NUM_THREADS="4")


def _run(cmd, env=None, timeout=300):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    return r.returncode, r.stdout + r.stderr


def _hipcc():
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    rc, out = _run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                    "-fopenmp", "-ffp-contract=off", os.path.join(ROOT, "oracle", "oracle.c"),
                    os.path.join(DRIVERS, "oracle_driver.c"), "-lm", "-o", exe])
    assert rc == 0, out
    rc, out = _run([exe], env=ENV)
    assert rc == 0 and "0 failures" in out, out
    assert "Sanitizer" not in out and "runtime error" not in out, out


def test_abi_validation_under_asan_and_ubsan(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not found")
    objs = [os.path.join(BUILD, o) for o in DEVICE_OBJECTS]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("the library's objects are not built (computation_collective_amd/build.py)")
    flags = ["-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-I", os.path.join(ROOT, "include"), "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    abi_o, drv_o, exe = str(tmp_path / "abi.o"), str(tmp_path / "drv.o"), str(tmp_path / "abi_driver")
    for src, obj in ((os.path.join(ROOT, "computation_collective_amd", "csrc", "abi.cpp"), abi_o),
                     (os.path.join(DRIVERS, "abi_driver.cpp"), drv_o)):
        rc, out = _run([hipcc] + flags + HOST_SAN + ["-c", src, "-o", obj])
        assert rc == 0, out
    rc, out = _run([hipcc, "--offload-arch=gfx950"] + HOST_SAN + [drv_o, abi_o] + objs + ["-o", exe])
    assert rc == 0, out
    # (leak checking off: the HIP runtime's own allocations live until exit)
    rc, out = _run([exe], env=dict(ENV, ASAN_OPTIONS="halt_on_error=1:detect_leaks=0"))
    assert rc == 0 and "0 failures" in out, out
    assert "Sanitizer" not in out and "runtime error" not in out, out
