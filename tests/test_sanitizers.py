"""The CPU oracle and the library's host packers under AddressSanitizer and
UndefinedBehaviorSanitizer (host code only): tests/sanitize/driver.cpp runs
every oracle step and the packers on small layers and checks the packers
against the oracle; any invalid access or undefined operation aborts it."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


@pytest.mark.skipif(not (os.path.exists(CLANG) and os.path.exists(CLANGXX)), reason="clang not installed")
def test_oracle_and_packers_under_sanitizers(tmp_path):
    csrc = os.path.join(ROOT, "w4ax_mixed_precision_amd", "csrc")
    oracle_o = str(tmp_path / "oracle.o")
    subprocess.run([CLANG, *SAN, "-std=c99", "-ffp-contract=off", "-c", os.path.join(ROOT, "oracle", "comet_oracle.c"),
                    "-o", oracle_o], check=True)
    exe = str(tmp_path / "driver")
    subprocess.run([CLANGXX, *SAN, "-std=c++17", "-ffp-contract=off", os.path.join(ROOT, "tests", "sanitize", "driver.cpp"),
                    os.path.join(csrc, "pack_weights.cpp"), oracle_o, "-o", exe, "-lpthread", "-lm"], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    print(r.stdout[-2000:], r.stderr[-4000:])
    assert r.returncode == 0, r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
    assert r.stdout.strip().endswith("(0 mismatches)")
