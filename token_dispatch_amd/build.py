"""Build the HIP libraries in-tree for gfx950 with hipcc.

libmoonep.so     the method: api.hip, plan.hip, move.hip, backward.hip
libmoonep_stream.so  the streaming kernels the benchmark measures ceilings with
                 (stream.hip, include/moonep_stream.h)

Every source is compiled for the device (gfx950 only) and linked next to this
file. Packed-FP32 instruction selection is switched off for all device code.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoonep.so")
SOURCES = ["api.hip", "plan.hip", "move.hip", "backward.hip"]
STREAM_LIB = os.path.join(HERE, "libmoonep_stream.so")
STREAM_SOURCES = ["stream.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def build(verbose: bool = False) -> str:
    os.makedirs(os.path.join(HERE, "_build"), exist_ok=True)
    procs = []
    objs = _compile(SOURCES, procs, verbose)
    stream_objs = _compile(STREAM_SOURCES, procs, verbose)
    for p, cmd in procs:
        if p.wait() != 0:
            raise RuntimeError("hipcc failed: " + " ".join(cmd))
    _link(objs, LIB, verbose)
    _link(stream_objs, STREAM_LIB, verbose)
    return LIB


def _compile(sources, procs, verbose):
    objs = []
    for src in sources:
        obj = os.path.join(HERE, "_build", src.replace(".hip", ".o"))
        cmd = [HIPCC] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd), cmd))
        objs.append(obj)
    return objs


def _link(objs, lib, verbose):
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, lib)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
