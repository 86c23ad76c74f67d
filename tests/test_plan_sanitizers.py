"""The QMoE contract validator and launch planner (csrc/qmoe_plan.cpp, pure
C++) built for the host with AddressSanitizer and UndefinedBehaviorSanitizer
and driven by tests/native/plan_check.cpp: a seeded fuzz of tensor
descriptors and attributes around the contract, checking the plan's
workspace and tiling invariants for every accepted case.  No GPU."""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT

CSRC = os.path.join(ROOT, "quantized_mixture_experts_router_amd", "csrc")


@pytest.mark.timeout(600)
def test_planner_under_asan_and_ubsan(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = tmp_path / "plan_check"
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "native", "plan_check.cpp"), os.path.join(CSRC, "qmoe_plan.cpp"),
           "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([str(exe), "200000"], capture_output=True, text=True, env=env, timeout=500)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert " 0 invariant failures" in r.stdout
