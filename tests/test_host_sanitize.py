"""The C ABI's host code under AddressSanitizer and UBSan (CPU only).

``rlk_api.cpp`` (argument validation, device binding, kernel parameters) is
compiled with g++ as host-only C++ and linked against a fake HIP runtime and
recording launchers (``tests/host_abi/stub_hip.cpp``) instead of the kernels.
``tests/host_abi/driver.cpp`` then calls every entry point: valid calls of
each head, dtype, cap form, layout and shard, the documented error cases of
the boundary (null pointers, V = 0, k outside [1, 4096], strides below V,
64-bit offset overflow, overlapping gradient rows, invalid caps and
directions, mixed devices, host memory, shard and combine bounds) and the
empty calls, checking statuses, the launch parameters and that every launch
stays inside the fake allocations.  Any out-of-bounds access, leak or
undefined operation in the host code fails the run (the input-validation
cases of "perf(logp): fused zero-workspace backward for the generic CUDA
fused logp", RL-Kernel pull request 495, Tests).  No GPU code is built.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_abi")
CSRC = os.path.join(ROOT, "vocab_log_softmax_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_host_abi_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_abi")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, "-I", HERE, os.path.join(CSRC, "rlk_api.cpp"),
           os.path.join(HERE, "stub_hip.cpp"), os.path.join(HERE, "driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "0 failed" in r.stdout, r.stdout
