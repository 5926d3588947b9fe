"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two drivers under tests/host_sanitize/ are compiled with gcc / g++ and run:
the CPU oracle (oracle/oracle.c) on exact-size heap buffers over every dtype
and edge shapes, and the launch planning the C ABI and the kernel launchers
share (rmsnorm_bwd_amd/csrc/plan.h) over every accepted row length with the
invariants the kernels rely on (every column covered, whole wavefronts,
every dgamma partial inside the queried workspace). No GPU code is built
here.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_sanitize")
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _sanitizers_available(tmp_path):
    if not shutil.which("gcc") or not shutil.which("g++"):
        return False
    src = tmp_path / "probe.c"
    src.write_text("int main(void) { return 0; }\n")
    r = subprocess.run(["gcc", *SAN, str(src), "-o", str(tmp_path / "probe")], capture_output=True)
    return r.returncode == 0


def _run(cmd_build, exe):
    subprocess.run(cmd_build, check=True, capture_output=True, timeout=300)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report[-4000:]
    assert "runtime error" not in report and "ERROR: AddressSanitizer" not in report, report[-4000:]
    return report


def test_oracle_under_sanitizers(tmp_path):
    if not _sanitizers_available(tmp_path):
        pytest.skip("gcc sanitizer runtimes not available")
    exe = str(tmp_path / "oracle_driver")
    out = _run(["gcc", *SAN, "-std=c11", "-ffp-contract=off", os.path.join(ROOT, "oracle", "oracle.c"),
                os.path.join(HERE, "oracle_driver.c"), "-o", exe, "-lm"], exe)
    assert "0 failing cases" in out


def test_launch_planning_under_sanitizers(tmp_path):
    if not _sanitizers_available(tmp_path):
        pytest.skip("gcc sanitizer runtimes not available")
    exe = str(tmp_path / "plan_driver")
    out = _run(["g++", *SAN, "-std=c++17", "-I", os.path.join(ROOT, "rmsnorm_bwd_amd", "csrc"),
                os.path.join(HERE, "plan_driver.cpp"), "-o", exe], exe)
    assert "0 failed checks" in out
