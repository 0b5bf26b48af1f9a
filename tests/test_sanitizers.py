"""AddressSanitizer and UndefinedBehaviorSanitizer runs on the CPU (no GPU involved):

- the oracle (oracle/mq_oracle.c) with tests/oracle_asan_driver.c, which calls every exported
  oracle function on ragged tensors and convolutions in exactly sized buffers;
- the C ABI's host-side validation (csrc/mq_api.cpp) with tests/host_asan_driver.cpp, which
  calls every entry point with null, negative, huge, misaligned and mismatched arguments (the
  kernel launchers are stubs there).

Both are built with gcc / g++ (host code only) and must finish without a sanitizer report."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-O1", "-g"]


def _run(cmd, exe):
    subprocess.check_call(cmd)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
    return r.stdout


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    out = _run(["gcc", "-std=c11", "-fopenmp", "-ffp-contract=off", *SAN,
                os.path.join(HERE, "oracle_asan_driver.c"),
                os.path.join(ROOT, "oracle", "mq_oracle.c"), "-o", exe, "-lm"], exe)
    assert "ok" in out


@pytest.mark.skipif(not os.path.isdir("/opt/rocm/include"), reason="needs the HIP headers")
def test_host_validation_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_asan")
    out = _run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                "-D__syncthreads()=((void)0)", *SAN, os.path.join(HERE, "host_asan_driver.cpp"),
                os.path.join(ROOT, "microscaling_quantized_convolution_amd", "csrc", "mq_api.cpp"),
                "-o", exe], exe)
    assert "0 failures" in out
