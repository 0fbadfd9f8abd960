"""The planner and the plan entry points of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer: a host-only build (g++, no device code; the kernel launchers
and the few HIP runtime calls of the C ABI are link stubs that abort if reached) runs over
seeded random graphs under many option sets, the degenerate graphs and invalid CSR input
(tests/c/plan_sanitize.cpp). A sanitizer report or a failed check fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_graph_attention_02_amd", "csrc")


def test_planner_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    rocm_include = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")
    exe = str(tmp_path / "plan_sanitize")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-pthread",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__=1", "-I", rocm_include, "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, os.path.join(CSRC, "plan.cpp"), os.path.join(CSRC, "api.cpp"),
           os.path.join(ROOT, "tests", "c", "host_stubs.cpp"),
           os.path.join(ROOT, "tests", "c", "plan_sanitize.cpp"), "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert b.returncode == 0, b.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-6000:])
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr[-6000:]
    assert "failures 0" in r.stdout
