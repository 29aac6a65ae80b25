"""The host tile planner (csrc/plan.cpp) under AddressSanitizer and
UndefinedBehaviorSanitizer: tests/sanitize/plan_harness.cpp, built with g++
(host code only, no device code), walks about 27 000 valid plan descriptors
and a set of invalid ones and checks every plan's invariants (each tile once
per K range, inside the output, keys in order, chunk masks, landing order,
capacity and argument refusals).  The exact orders are checked against the
oracle in test_plan_lib.py; this test is about memory and arithmetic safety."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIP_INC = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(os.path.join(HIP_INC, "hip")),
                    reason="needs g++ and the HIP headers")
def test_planner_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "plan_san"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
           f"-I{HIP_INC}", f"-I{os.path.join(ROOT, 'include')}",
           f"-I{os.path.join(ROOT, 'tile_level_communication_amd', 'csrc')}",
           os.path.join(ROOT, "tile_level_communication_amd", "csrc", "plan.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "plan_harness.cpp"), "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=240)
    assert build.returncode == 0, build.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=240, env=env)
    assert run.returncode == 0, (run.stdout + run.stderr)[-3000:]
    assert "failures 0" in run.stdout, run.stdout
