"""Compile the library for gfx950 in-tree with hipcc.

Three shared libraries, from the same sources:

* ``librowreduce.so`` -- the product: the kernels (rr_kernels.hip) and the
  C ABI of include/rowreduce.h (rr_api.cpp).
* ``librowreduce_diag.so`` -- the diagnostics build: the product's kernel
  object, linked unchanged, plus the entry points of include/rowreduce_diag.h
  (a forced kernel variant, the all-reduce self-test and the streaming copy;
  rr_api.cpp with RR_DIAG=1 and rr_diag.hip).  Tests that force a variant and
  the benchmark's copy reference use it; the product never carries them.
* ``librowreduce_stress.so`` -- the race-stress build that only the tests
  load: RR_STRESS=1 adds random per-wavefront delays around every LDS slot
  stage and poisons slots after their readers are done, and caps grids so
  workgroups walk many rows (it also carries the diagnostics entry points).

Every HIP source is built with the packed-FP32 target feature switched off
(``-Xclang -target-feature -Xclang -packed-fp32-ops``) and with -O3.  The
libraries link only against the HIP runtime; they have no PyTorch
dependency.  The compilations run in parallel.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "librowreduce.so")
LIB_DIAG = os.path.join(HERE, "librowreduce_diag.so")
LIB_STRESS = os.path.join(HERE, "librowreduce_stress.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{CSRC}"]

# object name -> (source, extra flags)
OBJECTS = {
    "kernels": ("rr_kernels.hip", ()),
    "api": ("rr_api.cpp", ()),
    "api_diag": ("rr_api.cpp", ("-DRR_DIAG=1",)),
    "diag": ("rr_diag.hip", ()),
    "kernels_stress": ("rr_kernels.hip", ("-DRR_STRESS=1",)),
    "api_stress": ("rr_api.cpp", ("-DRR_STRESS=1", "-DRR_DIAG=1")),
}
LIBRARIES = {
    LIB: ("kernels", "api"),
    LIB_DIAG: ("kernels", "api_diag", "diag"),
    LIB_STRESS: ("kernels_stress", "api_stress", "diag"),
}


def _obj_path(name):
    return os.path.join(CSRC, f"{name}.build.o")


def _compile_cmd(name):
    src, extra = OBJECTS[name]
    # an explicit compilation-unit id (otherwise derived from the command
    # line, object path included), so the device code a build embeds depends
    # only on the sources and flags
    cuid = "-cuid=" + (name + "_" + src).replace(".", "_")
    return [HIPCC, *COMMON, *extra, cuid, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", _obj_path(name)]


def _run_parallel(cmds, verbose):
    procs = []
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd)))
    failed = [cmd for cmd, p in procs if p.wait() != 0]
    if failed:
        raise subprocess.CalledProcessError(1, failed[0])


def build(verbose: bool = False, libraries=None) -> str:
    """Compile and link `libraries` (default: all three); returns the product path."""
    libraries = list(LIBRARIES) if libraries is None else list(libraries)
    names = sorted({o for lib in libraries for o in LIBRARIES[lib]})
    _run_parallel([_compile_cmd(n) for n in names], verbose)
    links = []
    for lib in libraries:
        objs = [_obj_path(o) for o in LIBRARIES[lib]]
        links.append([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", lib + ".tmp",
                      "-Wl,-rpath,/opt/rocm/lib"])
    _run_parallel(links, verbose)
    for lib in libraries:
        os.replace(lib + ".tmp", lib)
    for n in names:
        os.remove(_obj_path(n))
    return LIB


def build_stress(verbose: bool = False) -> str:
    build(verbose, libraries=[LIB_STRESS])
    return LIB_STRESS


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
