"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two drivers in tests/sanitize/ are built with gcc / g++ and
-fsanitize=address,undefined -fno-sanitize-recover=all and run:
  plan_harness.cpp  the decode library's host side (decode_attention_query_amd/
                    csrc/fa_plan.hpp: every entry point's argument checks, the
                    launch plan, the workspace layout) over random, extreme and
                    edge-case arguments, with the plan's invariants asserted;
  oracle_driver.c   the float64 oracle (oracle/decode_ref.c) on random small
                    problems with buffers of exactly the documented sizes.
Any out-of-bounds access, leak or undefined behaviour fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-g", "-O1"]
ROCM_INCLUDE = "/opt/rocm/include"  # hip_runtime_api.h, for hipStream_t in fa_decode.h


def _run(exe):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="2")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, f"{os.path.basename(exe)} failed:\n{r.stdout}\n{r.stderr[-4000:]}"
    return r.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_plan_and_checks_under_sanitizers(tmp_path):
    if not os.path.exists(os.path.join(ROCM_INCLUDE, "hip", "hip_runtime_api.h")):
        pytest.skip("needs the HIP runtime headers")
    exe = str(tmp_path / "plan_harness")
    subprocess.run(["g++", "-std=c++17", *SAN, f"-I{ROCM_INCLUDE}", "-D__HIP_PLATFORM_AMD__",
                    "-o", exe, os.path.join(HERE, "plan_harness.cpp")], check=True)
    assert "plan harness OK" in _run(exe)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    subprocess.run(["gcc", "-std=c11", *SAN, "-fopenmp", "-o", exe,
                    os.path.join(HERE, "oracle_driver.c"),
                    os.path.join(ROOT, "oracle", "decode_ref.c"), "-lm"], check=True)
    assert "oracle driver OK" in _run(exe)
