"""The library's host code (the pack: Gram matrix, multi-threaded Householder
tridiagonalization with a spin barrier, bisection, inverse iteration, quantization, the
refinement loop, the LoRA fold and the device layouts) built for the CPU under
AddressSanitizer + UndefinedBehaviorSanitizer and, separately, ThreadSanitizer, and run
through every host entry point by tests/sanitize/pack_driver.cpp with several threads.
No GPU is involved: only pack.cpp and status.cpp are compiled, with g++.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_diffusion_model_amd", "csrc")
SOURCES = [os.path.join(CSRC, "pack.cpp"), os.path.join(CSRC, "status.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "pack_driver.cpp")]


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
@pytest.mark.parametrize("san", ["address,undefined", "thread"])
def test_host_pack_under_sanitizer(san, tmp_path):
    exe = str(tmp_path / ("driver_" + san.split(",")[0]))
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-pthread", f"-fsanitize={san}",
           "-fno-sanitize-recover=all", "-I", CSRC, *SOURCES, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, SVDQ_NUM_THREADS="4", ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", TSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout + r.stderr)[-6000:]
    assert "ok (0 failures)" in r.stdout
