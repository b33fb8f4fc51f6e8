"""Compile librowreduce.so for gfx950 in-tree with hipcc.

Every HIP source is built with the packed-FP32 target feature switched off
(``-Xclang -target-feature -Xclang -packed-fp32-ops``) and with -O3.  The
library links only against the HIP runtime; it has no PyTorch dependency.

build_stress() compiles the same sources with RR_STRESS=1 into
librowreduce_stress.so: the race-stress build that only the tests load
(random per-wavefront delays around every LDS slot stage, poisoned slots
after their readers are done, grids capped so workgroups walk many rows).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "librowreduce.so")
LIB_STRESS = os.path.join(HERE, "librowreduce_stress.so")
SOURCES = ["rr_kernels.hip", "rr_api.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{CSRC}"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose: bool = False, extra_flags=(), out: str = LIB) -> str:
    objs = []
    tag = os.path.splitext(os.path.basename(out))[0]
    for src in SOURCES:
        obj = os.path.join(CSRC, f"{src}.{tag}.o")
        # an explicit compilation-unit id (otherwise derived from the command
        # line, object path included), so the device code a build embeds
        # depends only on the sources and flags
        cuid = "-cuid=" + (tag + "_" + src).replace(".", "_")
        _run([HIPCC, *COMMON, *extra_flags, cuid, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj],
             verbose)
        objs.append(obj)
    tmp = out + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp,
          "-Wl,-rpath,/opt/rocm/lib"], verbose)
    os.replace(tmp, out)
    for o in objs:
        os.remove(o)
    return out


def build_stress(verbose: bool = False) -> str:
    return build(verbose, extra_flags=("-DRR_STRESS=1",), out=LIB_STRESS)


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
