"""The built library's gfx950 code object, read from its own metadata (CPU only).

Every kernel that keeps a row in registers relies on the compiler not moving
those registers to scratch memory: a spill would silently turn one HBM read
into two.  This reads the kernel descriptors of the code object that the
build embedded in librowreduce.so (LLVM's offload bundler and readelf, on
code built here) and requires, for every kernel: no VGPR spills, no private
(scratch) segment, wave64, and a single gfx950 target in the bundle.
"""
import os
import re
import shutil
import subprocess

import pytest

import row_reduction_rmsnorm_amd as rr

LLVM = "/opt/rocm/llvm/bin"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"


def _tool(name):
    path = os.path.join(LLVM, name)
    if not os.path.exists(path):
        pytest.skip(f"{name} not available")
    return path


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    lib = rr.binding.LIB_PATH
    if not os.path.exists(lib):
        pytest.skip("library not built")
    tmp = tmp_path_factory.mktemp("codeobj")
    fatbin = tmp / "fatbin.bin"
    subprocess.run([_tool("llvm-objcopy"), f"--dump-section=.hip_fatbin={fatbin}", lib], check=True)
    listed = subprocess.run([_tool("clang-offload-bundler"), "--list", "--type=o", f"--input={fatbin}"],
                            check=True, capture_output=True, text=True).stdout.split()
    device = [t for t in listed if not t.startswith("host-")]
    assert device == [TARGET], listed
    co = tmp / "gfx950.co"
    subprocess.run([_tool("clang-offload-bundler"), "--unbundle", "--type=o", f"--input={fatbin}",
                    f"--targets={TARGET}", f"--output={co}"], check=True)
    notes = subprocess.run([_tool("llvm-readelf"), "--notes", str(co)], check=True, capture_output=True,
                           text=True).stdout
    found = {}
    cur = None
    for line in notes.splitlines():
        m = re.match(r"\s*\.(name|vgpr_spill_count|private_segment_fixed_size|wavefront_size|vgpr_count):\s+(\S+)",
                     line)
        if not m:
            continue
        key, val = m.groups()
        if key == "name":
            cur = val
            found[cur] = {}
        elif cur is not None:
            found[cur][key] = val
    shutil.rmtree(tmp, ignore_errors=True)
    return found


def test_every_kernel_is_present(kernels):
    names = " ".join(kernels)
    for family in ("norm_regs_kernel", "norm_loop_kernel", "norm_sub_kernel", "softmax_regs_kernel",
                   "softmax_sub_kernel", "softmax_packed_kernel", "softmax_loop_kernel",
                   "softmax_split_stats_kernel", "softmax_split_apply_kernel", "softmax_split_fused_kernel"):
        assert family in names, family
    # the diagnostic kernels live only in the diagnostics build
    assert "selftest_wave_kernel" not in names and "stream_copy_kernel" not in names


def test_no_spills_no_scratch_wave64(kernels):
    bad = [(n, k) for n, k in kernels.items()
           if k.get("vgpr_spill_count") != "0" or k.get("private_segment_fixed_size") != "0"
           or k.get("wavefront_size") != "64"]
    assert not bad, bad[:5]
