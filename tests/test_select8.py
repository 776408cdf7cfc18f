"""Host check of the many-row coarse kernel's per-thread top-8 selection.

Compiles tests/select8_check.cpp (g++) against the library's select8.h, the
code the kernel runs for each (block, row) list of at most eight, and runs it:
300,000 rows (random, exact ties, near-ties whose keys agree above bit 5,
missing columns) against a sort by (score desc, column asc), and the sorting
network on every zero-one input."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_select8_matches_a_sort(tmp_path):
    exe = tmp_path / "select8_check"
    subprocess.run(["g++", "-std=c++17", "-O2", "-Wall", "-Wno-unknown-pragmas", "-Werror",
                    os.path.join(ROOT, "tests", "select8_check.cpp"), "-o", str(exe)],
                   check=True, capture_output=True, text=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.strip().startswith("ok")
