"""CPU runs of the oracle and of the library's host-side validation under
AddressSanitizer and UndefinedBehaviorSanitizer (no GPU needed).

* The oracle (oracle/la_oracle.c) is compiled with gcc and the sanitizers into
  one program with tests/sanitize/oracle_driver.c, which calls every oracle
  function on small seeded shapes (one token, ragged chunks, every feature
  map, with and without starting states) and checks agreements the
  definitions fix; leak detection is on.
* la_api.hip (argument validation, segment plans, workspace layouts) is
  compiled with the sanitizers on its host code only and linked with the
  other library objects and tests/sanitize/validate_driver.cpp, which calls
  every entry point with arguments validation must reject and the host
  queries over a sweep of shapes; no call reaches a device.
A sanitizer report makes the program exit non-zero (no recovery).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
ROCM_CLANG = "/opt/rocm/lib/llvm/bin/clang++"


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr[-4000:]}"
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_asan")
    _run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fopenmp", "-std=c11", os.path.join(ROOT, "oracle", "la_oracle.c"),
          os.path.join(SAN, "oracle_driver.c"), "-o", exe, "-lm"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS="2")
    r = _run([exe], env=env)
    assert "all agreements hold" in r.stdout


def test_host_validation_under_asan_ubsan(tmp_path):
    from kernelized_linear_attention_la_amd import build as hip_build
    if not os.path.exists(ROCM_CLANG):
        pytest.skip("ROCm clang not found")
    others = [os.path.join(hip_build.BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in hip_build.SOURCES
              if s != "la_api.hip"]
    if not all(os.path.exists(o) for o in others):
        hip_build.build()
    api_o, drv_o, exe = str(tmp_path / "la_api_san.o"), str(tmp_path / "drv.o"), str(tmp_path / "validate_san")
    # host code of la_api.hip with the sanitizers (device code built as usual)
    _run([hip_build.hipcc()] + [f for f in hip_build.compile_flags() if f != "-O3"] +
         ["-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
          "-c", os.path.join(hip_build.CSRC, "la_api.hip"), "-o", api_o])
    san = "-fsanitize=address,undefined"
    _run([ROCM_CLANG, "-O1", "-g", "-std=c++17", san, "-fno-sanitize-recover=all", "-I", hip_build.INCLUDE,
          "-c", os.path.join(SAN, "validate_driver.cpp"), "-o", drv_o])
    _run([ROCM_CLANG, san, drv_o, api_o] + others + ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib",
                                                    "-o", exe])
    # the HIP runtime's own allocations are not this library's: leak checks off here
    r = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1"))
    assert "all statuses as expected" in r.stdout
