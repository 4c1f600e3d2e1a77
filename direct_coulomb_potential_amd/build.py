"""Build libcpmap.so (HIP for gfx950) in-tree.

Every HIP source under csrc/ is compiled by hipcc for gfx950 only and linked
into one shared library next to this file.  Packed-FP32 instruction selection
is switched off for all device code.
"""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libcpmap.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, jobs: int = 8) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    procs = []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
               "-fno-gpu-rdc", *DEVICE_FLAGS, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd), src))
        objs.append(obj)
        if len(procs) >= jobs:
            _wait(procs)
    _wait(procs)
    link = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", LIB + ".tmp", *objs]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def _wait(procs):
    failed = []
    for p, src in procs:
        if p.wait() != 0:
            failed.append(src)
    procs.clear()
    if failed:
        raise RuntimeError("hipcc failed on: " + ", ".join(failed))


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
