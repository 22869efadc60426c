"""Build the W4A16 shared library in-tree with hipcc for gfx950.

    python -m w4a16_gemm_amd.build          # writes w4a16_gemm_amd/libw4a16.so

The host (offline) part is compiled as plain C++ with -ffp-contract=off, the
device part as HIP for gfx950; both link into one shared library.  Packed-fp32
instructions are disabled for all device code.  The library is written to a
temporary name and renamed into place, so a reader never sees half a file.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libw4a16.so")
PEAKS_LIB = os.path.join(HERE, "libw4a16_peaks.so")   # achievable-peak probes (bench only)

ARCH = "gfx950"
DEVICE_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-ffp-contract=off"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"build step failed ({res.returncode}): {' '.join(cmd)}")
    return res


def build(verbose: bool = False) -> str:
    """Compile and link the library; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    inc = ["-I", INCLUDE, "-I", CSRC]
    host_o = os.path.join(BUILD_DIR, "host.o")
    dev_o = os.path.join(BUILD_DIR, "device.o")
    _run([hipcc, "-c", os.path.join(CSRC, "host.cpp"), *HOST_FLAGS, *inc, "-o", host_o], verbose)
    _run([hipcc, "-c", "-x", "hip", os.path.join(CSRC, "device.hip"), *DEVICE_FLAGS, *inc, "-o", dev_o], verbose)
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", host_o, dev_o, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    tmp = PEAKS_LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", "-x", "hip", os.path.join(CSRC, "peaks.hip"), *DEVICE_FLAGS, *inc, "-o", tmp],
         verbose)
    os.replace(tmp, PEAKS_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
