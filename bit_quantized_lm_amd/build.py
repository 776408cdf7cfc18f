"""Build the draft-head shared library in-tree: bit_quantized_lm_amd/libdrafthead.so.

The host translation unit (quantiser, tiler, error state) is compiled with
g++ and -ffp-contract=off; the device translation unit (HIP kernels for
gfx950 and their entry points) with hipcc.  Usage: python -m bit_quantized_lm_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libdrafthead.so")
ARCH = os.environ.get("DRAFTHEAD_OFFLOAD_ARCH", "gfx950")


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in proc.stdout.splitlines()
                    if "packed-fp32-ops" not in line)   # harmless host-pass notice
    if proc.returncode != 0:
        raise RuntimeError(f"command failed ({proc.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    """Compile and link libdrafthead.so; returns its path."""
    hipcc = _hipcc()
    with tempfile.TemporaryDirectory() as tmp:
        host_o = os.path.join(tmp, "host.o")
        dev_o = os.path.join(tmp, "device.o")
        _run(["g++", "-O2", "-std=c++17", "-fPIC", "-ffp-contract=off", "-Wall", "-Wextra",
              "-c", os.path.join(CSRC, "host.cpp"), "-o", host_o])
        _run([hipcc, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
              # packed fp32 instructions are kept out of the device code
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-c", os.path.join(CSRC, "device.hip"), "-o", dev_o])
        tmp_lib = LIB + ".tmp"
        _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", host_o, dev_o,
              "-o", tmp_lib, "-lpthread"])
        os.replace(tmp_lib, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
