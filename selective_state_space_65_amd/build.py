"""Builds the HIP library libssm_scan.so in-tree for gfx950 with hipcc.

The library is the whole product path: C ABI + kernels in one shared object
(csrc/ssm_scan.hip: the ABI and most kernels; csrc/scan_chunked.hip: the
chunked prefill scan; header include/ssm_scan.h).  The translation units are
compiled in parallel and linked.  Packed FP32 instructions are disabled for
every HIP compile (-packed-fp32-ops).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRCS = [os.path.join(HERE, "csrc", "ssm_scan.hip"), os.path.join(HERE, "csrc", "scan_chunked.hip")]
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
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _run(cmds, verbose):
    """Runs the hipcc command lines in parallel; raises if any fails."""
    procs = []
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    failed = []
    for cmd, proc in zip(cmds, procs):
        out, _ = proc.communicate()
        if proc.returncode != 0:
            sys.stderr.write(out)
            failed.append(cmd[-1])
    if failed:
        raise RuntimeError("hipcc failed on %s" % ", ".join(failed))


def _link(srcs, lib, verbose):
    """Compiles each source to an object (in parallel) and links them into lib."""
    objs = [lib + ".%d.o" % i for i in range(len(srcs))]
    _run([[hipcc()] + HIPCC_FLAGS + ["-I", INCLUDE, "-c", "-o", o, s] for s, o in zip(srcs, objs)], verbose)
    tmp = lib + ".tmp"
    _run([[hipcc()] + HIPCC_FLAGS + ["-shared", "-o", tmp] + objs], verbose)
    for o in objs:
        os.remove(o)
    os.replace(tmp, lib)
    return lib


def build(verbose=False):
    """Compile the library sources into libssm_scan.so and csrc/rate_probe.hip
    into librate_probe.so (always recompiles)."""
    _link([PROBE_SRC], PROBE_LIB, verbose)
    return _link(SRCS, LIB, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
