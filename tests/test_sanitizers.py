"""AddressSanitizer + UndefinedBehaviorSanitizer runs of the CPU code (CPU only).

* The oracle (oracle/tq_oracle.c) built with -fsanitize=address,undefined and
  driven through every path the tests use (tests/sanitize/oracle_driver.c).
* The host side of libtq (kv_cache_vector_pi_amd/csrc/tq_host.cpp: seeded
  rotation, Lloyd-Max, argument validation of every entry point), built for
  the host only with the kernel launchers replaced by stand-ins that report
  an error (tests/sanitize/host_stubs.cpp), and driven by
  tests/sanitize/host_driver.cpp against a context described on the host.

GPU code is never built with a sanitizer here.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", "-fopenmp", "-ffp-contract=off", "-D_GNU_SOURCE"] + SAN +
         [os.path.join(ROOT, "oracle", "tq_oracle.c"),
          os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), "-lm", "-o", exe])
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1:abort_on_error=0")
    assert "oracle driver ok" in _run([exe], env=env)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_host_setup_and_validation_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "host_driver")
    inc = ["-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include"]
    srcs = [os.path.join(ROOT, "kv_cache_vector_pi_amd", "csrc", "tq_host.cpp"),
            os.path.join(ROOT, "tests", "sanitize", "host_stubs.cpp"),
            os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp")]
    _run(["g++"] + inc + SAN + srcs + ["-L/opt/rocm/lib", "-lamdhip64",
                                       "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    # the HIP runtime's own allocations are not this code's: leak checks off
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    assert "host driver ok" in _run([exe], env=env)
