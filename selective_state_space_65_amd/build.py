"""Builds the HIP library libssm_scan.so in-tree for gfx950 with hipcc.

The library is the whole product path: C ABI + kernels in one shared object
(csrc/ssm_scan.hip, header include/ssm_scan.h).  Packed FP32 instructions are
disabled for every HIP compile (-packed-fp32-ops).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "ssm_scan.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libssm_scan.so")
# Instruction-rate probes for the roofline (bench.py only; not the scan path).
PROBE_SRC = os.path.join(HERE, "csrc", "rate_probe.hip")
PROBE_LIB = os.path.join(HERE, "librate_probe.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _compile(src, lib, verbose):
    tmp = lib + ".tmp"
    cmd = [hipcc()] + HIPCC_FLAGS + ["-I", INCLUDE, "-o", tmp, src]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        sys.stderr.write(proc.stdout + proc.stderr)
        raise RuntimeError("hipcc failed building %s" % lib)
    os.replace(tmp, lib)
    return lib


def build(verbose=False):
    """Compile csrc/ssm_scan.hip into libssm_scan.so and csrc/rate_probe.hip into
    librate_probe.so (always recompiles)."""
    _compile(PROBE_SRC, PROBE_LIB, verbose)
    return _compile(SRC, LIB, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
