"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two harnesses in tests/sanitize/ are compiled with gcc/g++ -fsanitize=address,undefined
(-fno-sanitize-recover: the first report fails the run) and executed:
  * oracle_harness.c: every oracle entry point (float64 and float32 forward, float64
    backward) on small and empty problems with every optional input present and absent and a
    padding mask, plus the prefix-sum worked example;
  * abi_harness.cpp: the C-ABI argument checks of scan_api.cpp and ssd_api.cpp, with the
    kernel launches and the one reachable HIP call stubbed (no device is touched), on valid
    problems, invalid arguments and sizes at the edges of int64.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = os.path.join(HERE, "sanitize")
CSRC = os.path.join(ROOT, "selective_state_space_fwd_amd", "csrc")
FLAGS = ["-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _run(cmd, exe, expect):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"build failed:\n{r.stderr[-3000:]}"
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout[-2000:], r.stderr[-4000:])
    assert r.returncode == 0 and expect in r.stdout, r.stderr[-4000:]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_harness")
    cmd = ["gcc", "-std=c11", *FLAGS, "-fopenmp", "-ffp-contract=off",
           "-I", os.path.join(ROOT, "oracle"), "-o", exe, os.path.join(SAN, "oracle_harness.c"),
           os.path.join(ROOT, "oracle", "ssm_ref.c"), os.path.join(ROOT, "oracle", "ssm_ref_bwd.c"),
           "-lm"]
    _run(cmd, exe, "oracle harness ok")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the ROCm headers not available")
def test_abi_checks_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_harness")
    cmd = ["g++", "-std=c++17", *FLAGS, "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", exe,
           os.path.join(SAN, "abi_harness.cpp"), os.path.join(CSRC, "scan_api.cpp"),
           os.path.join(CSRC, "ssd_api.cpp")]
    _run(cmd, exe, "abi harness ok")
