"""Build the HIP libraries in-tree for gfx950 with hipcc.

libmoonep.so     the method: api.hip, plan.hip, move.hip, backward.hip
libmoonep_stream.so  the streaming kernels the benchmark measures ceilings with
                 (stream.hip, include/moonep_stream.h)

Every source is compiled for the device (gfx950 only) and linked next to this
file. Packed-FP32 instruction selection is switched off for all device code.
No kernel is meant to need scratch memory: a launch of one that does pays for
setting up a private segment even when the frame is never touched, so the
build reads the compiler's resource-usage remarks and fails on any kernel with
a nonzero scratch size.
"""
import os
import re
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
    scratch = []
    for p, cmd in procs:
        out, _ = p.communicate()
        if p.returncode != 0:
            sys.stderr.write(out)
            raise RuntimeError("hipcc failed: " + " ".join(cmd))
        scratch += _scratch_kernels(out)
    if scratch:
        raise RuntimeError("kernels that need scratch memory: " + ", ".join(scratch))
    _link(objs, LIB, verbose)
    _link(stream_objs, STREAM_LIB, verbose)
    return LIB


def _compile(sources, procs, verbose):
    objs = []
    for src in sources:
        obj = os.path.join(HERE, "_build", src.replace(".hip", ".o"))
        cmd = [HIPCC] + FLAGS + ["-Rpass-analysis=kernel-resource-usage",
                                 "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                       text=True), cmd))
        objs.append(obj)
    return objs


def _scratch_kernels(remarks):
    """Kernels whose resource-usage remark gives a nonzero scratch size."""
    out, name = [], None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and int(m.group(1)) > 0:
            out.append(f"{name} ({m.group(1)} bytes/lane)")
    return out


def _link(objs, lib, verbose):
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, lib)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
