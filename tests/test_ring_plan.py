"""Host check of the many-row coarse kernel's DMA ring schedule.

Compiles tests/ring_plan_check.cpp (g++) against the library's ring_plan.h,
the same constexpr code the kernel uses to address its DMA ops and choose its
wait counts, and runs it: every op of every stage in bounds for K up to 40960,
the LDS within 160 KB, and every wait count completing what the next stage
reads (counted op by op)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_ring_plan_bounds_and_waits(tmp_path):
    exe = tmp_path / "ring_plan_check"
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Werror", os.path.join(ROOT, "tests", "ring_plan_check.cpp"),
                    "-o", str(exe)], check=True, capture_output=True, text=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.strip().startswith("ok")
