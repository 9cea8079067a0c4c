"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/oracle_sanitize_driver.c calls every oracle function over special rows
(masked columns, all -inf rows, +1000 offsets, a single finite column, V = 1,
N = 0, ignored, out-of-range and duplicate targets, support mismatch, caps
off, 20 and 1e-7) with two OpenMP threads; built with gcc, host code only,
any out-of-bounds access, leak or undefined operation aborts the run.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _gcc_sanitizers_work(tmp):
    src = os.path.join(tmp, "probe.c")
    with open(src, "w") as f:
        f.write("int main(void) { return 0; }\n")
    r = subprocess.run(["gcc", *SAN, src, "-o", os.path.join(tmp, "probe")],
                       capture_output=True, text=True)
    return r.returncode == 0


def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    if shutil.which("gcc") is None or not _gcc_sanitizers_work(str(tmp_path)):
        pytest.skip("gcc with ASan/UBSan is not available")
    exe = str(tmp_path / "oracle_san")
    cmd = ["gcc", "-O1", "-g", "-std=c99", "-fopenmp", *SAN,
           os.path.join(ROOT, "oracle", "oracle.c"),
           os.path.join(ROOT, "tests", "oracle_sanitize_driver.c"), "-o", exe, "-lm"]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "status 0" in r.stdout
