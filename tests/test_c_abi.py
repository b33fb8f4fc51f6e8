"""The boundary from plain C (CPU only): include/rowreduce.h compiles as C99
with warnings as errors, and a C program linked against librowreduce.so
calls the host-only entry points (plans, workspace sizes, argument checks,
status strings) and gets the same answers the Python binding gets.
"""
import os
import shutil
import subprocess

import pytest

import row_reduction_rmsnorm_amd as rr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

C_PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "rowreduce.h"

int main(void) {
  rr_plan p;
  if (rr_query_plan(RR_OP_SOFTMAX, 256, 152064, RR_BF16, RR_F32, 1, &p) != RR_OK) return 1;
  printf("vocab %d %d %lld %zu\n", p.variant, p.vecs_per_lane, (long long)p.chunks_per_row, p.workspace_bytes);
  if (rr_query_plan(RR_OP_RMSNORM, 8192, 4096, RR_BF16, RR_BF16, 1, &p) != RR_OK) return 2;
  printf("rms %d %d %d\n", p.variant, p.waves_per_row, p.vecs_per_lane);
  printf("ws %zu\n", rr_softmax_rows_workspace_bytes(256, 152064, RR_BF16, RR_F32));
  rr_softmax_opts o;
  memset(&o, 0, sizeof o);
  o.causal = 1;
  o.causal_period = 0;
  rr_status s = rr_softmax_rows_ex((void*)16, (const void*)4096, 4, 8, RR_F32, RR_F32, &o, NULL, 0, NULL);
  printf("bad %s %s\n", rr_status_string(s), strstr(rr_last_error_message(), "causal_period") ? "named" : "?");
  s = rr_rmsnorm(NULL, NULL, NULL, 0, 64, 1e-6f, RR_F32, NULL);
  printf("empty %s\n", rr_status_string(s));
  return 0;
}
"""


def _gcc():
    gcc = shutil.which("gcc")
    if not gcc:
        pytest.skip("gcc not available")
    return gcc


def test_header_is_c99():
    gcc = _gcc()
    subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-fsyntax-only",
                    "-x", "c", os.path.join(ROOT, "include", "rowreduce.h")], check=True)


def test_c_program_calls_the_host_entry_points(tmp_path):
    gcc = _gcc()
    lib = rr.binding.LIB_PATH
    if not os.path.exists(lib):
        pytest.skip("library not built")
    src = tmp_path / "demo.c"
    src.write_text(C_PROGRAM)
    exe = tmp_path / "demo"
    subprocess.run([gcc, "-std=c99", "-Wall", "-Werror", f"-I{os.path.join(ROOT, 'include')}", str(src),
                    "-o", str(exe), lib, f"-Wl,-rpath,{os.path.dirname(lib)}", "-Wl,-rpath,/opt/rocm/lib"],
                   check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.splitlines()
    p = rr.rr_query_plan(rr.RR_OP_SOFTMAX, 256, 152064, rr.RR_BF16, rr.RR_F32)
    assert out[0] == f"vocab {p['variant']} {p['vecs_per_lane']} {p['chunks_per_row']} {p['workspace_bytes']}"
    q = rr.rr_query_plan(rr.RR_OP_RMSNORM, 8192, 4096, rr.RR_BF16, rr.RR_BF16)
    assert out[1] == f"rms {q['variant']} {q['waves_per_row']} {q['vecs_per_lane']}"
    assert out[2] == f"ws {rr.rr_softmax_rows_workspace_bytes(256, 152064, rr.RR_BF16, rr.RR_F32)}"
    assert out[3] == "bad RR_ERR_INVALID_ARG named"
    assert out[4] == "empty RR_OK"
