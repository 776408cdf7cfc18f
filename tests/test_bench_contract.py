"""bench.py's contract on the CPU: the one-GPU rule and the byte counts its
roofline divides by (no GPU needed)."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_module", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stdout + r.stderr


def test_algorithmic_bytes():
    b = _bench()
    assert b.WEIGHT_BYTES == 178_790_400                     # codes + scale pairs of one shard
    # + x read (10,240 B per row) + candidates written (124,160 B per row)
    assert b.coarse_alg_bytes(1) == 178_924_800
    assert b.coarse_alg_bytes(8) == 179_865_600
    assert b.coarse_alg_bytes(72) == 188_467_200


def test_coarse_kernel_names():
    b = _bench()
    assert b.coarse_kernel_name(1) == "coarse_resident_kernel<2, false>"
    assert b.coarse_kernel_name(2) == "coarse_resident_kernel<2, false>"
    assert b.coarse_kernel_name(3) == "coarse_resident_kernel<4, false>"
    assert b.coarse_kernel_name(8) == "coarse_resident_kernel<8, false>"
    assert b.coarse_kernel_name(16) == "coarse_mfma_kernel<1, false>"
    assert b.coarse_kernel_name(32) == "coarse_mfma_kernel<2, false>"
    assert b.coarse_kernel_name(33) == "coarse_h16_kernel<3>"
    assert b.coarse_kernel_name(72) == "coarse_h16_kernel<5>"
