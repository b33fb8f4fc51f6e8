"""Host-side tests of the C ABI (no GPU needed).

* the shared library loads and exports every function include/rowreduce.h
  declares;
* argument validation returns the documented status before any device work
  (every call here fails validation, so nothing is enqueued);
* the variant dispatch picks the documented kernel for the named workloads
  and across the row-length boundaries (integer logic, compared exactly).
"""
import ctypes
import os
import re

import pytest

import row_reduction_rmsnorm_amd as rr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rowreduce.h")
DIAG_HEADER = os.path.join(ROOT, "include", "rowreduce_diag.h")


def split_ws(M, S):
    """A split plan's workspace: M * S slots of 16 bytes, then one 4-byte
    epoch per row (the one-kernel form's tags), padded to 16 bytes."""
    return M * S * 16 + (M * 4 + 15) // 16 * 16


def _declared_functions(path=HEADER):
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(rr_[a-z0-9_]+)\s*\(", text)
    return sorted(set(names))


def _exported(path):
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True, check=True).stdout
    return sorted({l.split()[-1] for l in out.splitlines() if " T rr_" in l})


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert len(names) >= 9
    L = rr.lib()
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing
    assert sorted(rr.EXPORTS) == names


def test_library_exports_nothing_undeclared():
    assert _exported(rr.binding.LIB_PATH) == _declared_functions()


def test_diagnostics_build_exports_and_shares_the_kernel_object():
    """librowreduce_diag.so exports rowreduce.h plus rowreduce_diag.h (and
    the product none of the latter); its device code holds the product's
    code object byte for byte (the same compiled kernel object, linked
    unchanged) plus the diagnostic kernels."""
    diag = _declared_functions(DIAG_HEADER)
    assert sorted(rr.DIAG_EXPORTS) == diag
    assert _exported(rr.binding.DIAG_LIB_PATH) == sorted(set(_declared_functions()) | set(diag))
    assert not set(diag) & set(_exported(rr.binding.LIB_PATH))
    import bench
    prod = bench.fatbin_bytes(rr.binding.LIB_PATH)
    assert prod in bench.fatbin_bytes(rr.binding.DIAG_LIB_PATH)


def test_status_strings():
    assert rr.status_string(rr.RR_OK) == "RR_OK"
    assert rr.status_string(rr.RR_ERR_WORKSPACE) == "RR_ERR_WORKSPACE"
    assert rr.status_string(99) == "RR_UNKNOWN_STATUS"


# A fake "device" address: validation must reject the call before touching it.
P = 1 << 32


@pytest.mark.parametrize("args,status", [
    ((P, P, P, 4, 0, 1e-6, rr.RR_F32, None), rr.RR_ERR_INVALID_ARG),      # H < 1
    ((P, P, P, -1, 8, 1e-6, rr.RR_F32, None), rr.RR_ERR_INVALID_ARG),     # M < 0
    ((None, P, P, 4, 8, 1e-6, rr.RR_F32, None), rr.RR_ERR_INVALID_ARG),   # null y
    ((P, P, P, 4, 8, -1.0, rr.RR_F32, None), rr.RR_ERR_INVALID_ARG),      # eps < 0
    ((P, P, P, 4, 8, float("nan"), rr.RR_F32, None), rr.RR_ERR_INVALID_ARG),
    ((P, P, P, 4, 8, 1e-6, 7, None), rr.RR_ERR_INVALID_ARG),              # dtype
    ((P, P + 4, P << 4, 4, 8, 1e-6, rr.RR_F32, None), rr.RR_ERR_INVALID_ARG),  # y partly overlaps x
    ((P, P << 2, P + 8, 4, 8, 1e-6, rr.RR_F32, None), rr.RR_ERR_INVALID_ARG),  # gamma inside y
    ((P, P, P << 4, 4, (1 << 30) + 8, 1e-6, rr.RR_F32, None), rr.RR_ERR_UNSUPPORTED),
])
def test_rmsnorm_validation(args, status):
    assert rr.raw_rmsnorm(*args) == status
    assert rr.last_error_message()


def test_m_zero_is_a_noop_even_with_null_pointers():
    assert rr.raw_rmsnorm(None, None, None, 0, 8, 1e-6, rr.RR_F32, None) == rr.RR_OK
    assert rr.raw_softmax_rows(None, None, 0, 8, rr.RR_F32, rr.RR_F32, None, 0, None) == rr.RR_OK
    assert rr.raw_fused_add_rmsnorm(None, None, None, None, 0, 8, 1e-6, rr.RR_BF16, None) == rr.RR_OK


def test_stream_copy_validation():
    L = rr.diag_lib()
    assert L.rr_stream_copy(None, None, 0, None) == rr.RR_OK            # empty: no launch
    for dst, src, nb in ((P, P << 4, -16),          # negative size
                         (P, P << 4, 24),           # not a multiple of 16
                         (None, P << 4, 32),        # null destination
                         (P, None, 32),             # null source
                         (P + 8, P << 4, 32),       # misaligned destination
                         (P, (P << 4) + 4, 32),     # misaligned source
                         (P, P + 16, 64)):          # overlapping ranges
        assert L.rr_stream_copy(dst, src, nb, None) == rr.RR_ERR_INVALID_ARG, (dst, src, nb)
        assert L.rr_last_error_message().decode().startswith("rr_stream_copy")


def test_fused_validation():
    X, R, G, Y = P, P << 2, P << 4, P << 6
    ok = dict(y=Y, residual=R, x=X, gamma=G)
    call = lambda d, M=4, H=8, dt=rr.RR_BF16: rr.raw_fused_add_rmsnorm(
        d["y"], d["residual"], d["x"], d["gamma"], M, H, 1e-6, dt, None)
    assert call({**ok, "residual": None}) == rr.RR_ERR_INVALID_ARG
    assert call({**ok, "residual": X}) == rr.RR_ERR_INVALID_ARG          # residual == x
    assert call({**ok, "residual": Y + 2}) == rr.RR_ERR_INVALID_ARG      # residual overlaps y
    assert call({**ok, "y": X + 2}) == rr.RR_ERR_INVALID_ARG             # y partly overlaps x
    assert call({**ok, "gamma": R + 4}) == rr.RR_ERR_INVALID_ARG         # gamma inside residual


def test_layernorm_validation_and_plan():
    Y, X, G, Bt = P, P << 4, P << 8, P << 9
    f = rr.raw_layernorm
    assert f(Y, X, G, None, 0, 8, 1e-5, rr.RR_F32, None) == rr.RR_OK          # M = 0
    assert f(Y, X, G, Bt, 4, 0, 1e-5, rr.RR_F32, None) == rr.RR_ERR_INVALID_ARG
    assert f(Y, X, None, Bt, 4, 8, 1e-5, rr.RR_F32, None) == rr.RR_ERR_INVALID_ARG
    assert f(Y, X, G, Y + 4, 4, 8, 1e-5, rr.RR_F32, None) == rr.RR_ERR_INVALID_ARG  # beta in y
    p = rr.rr_query_plan(rr.RR_OP_LAYERNORM, 256, 5120, rr.RR_F32, rr.RR_F32)
    assert (p["variant_name"], p["waves_per_row"], p["vecs_per_lane"]) == ("block", 10, 2)
    assert rr.rr_query_plan(rr.RR_OP_LAYERNORM, 8, 64, rr.RR_F32, rr.RR_F32)["variant_name"] == "subwave"
    with pytest.raises(rr.RowReduceError):
        rr.rr_query_plan(rr.RR_OP_LAYERNORM, 8, 64, rr.RR_BF16, rr.RR_F32)


def test_softmax_validation():
    X, Y, W = P, P << 4, P << 8
    f = rr.raw_softmax_rows
    assert f(Y, X, 4, 0, rr.RR_F32, rr.RR_F32, None, 0, None) == rr.RR_ERR_INVALID_ARG
    assert f(Y, X, 4, 8, 3, rr.RR_F32, None, 0, None) == rr.RR_ERR_INVALID_ARG
    # in place with different dtypes
    assert f(X, X, 4, 8, rr.RR_BF16, rr.RR_F32, None, 0, None) == rr.RR_ERR_INVALID_ARG
    # long rows with few rows need the split workspace (from 56 rows up a
    # bf16 -> fp32 row is held by one workgroup and needs none)
    assert rr.rr_softmax_rows_workspace_bytes(256, 152064, rr.RR_BF16, rr.RR_F32) == 0
    need = rr.rr_softmax_rows_workspace_bytes(40, 152064, rr.RR_BF16, rr.RR_F32)
    assert need == split_ws(40, 19)
    assert f(Y, X, 40, 152064, rr.RR_BF16, rr.RR_F32, None, 0, None) == rr.RR_ERR_WORKSPACE
    assert f(Y, X, 40, 152064, rr.RR_BF16, rr.RR_F32, W, need - 8, None) == rr.RR_ERR_WORKSPACE
    assert f(Y, X, 40, 152064, rr.RR_BF16, rr.RR_F32, W + 8, need, None) == rr.RR_ERR_INVALID_ARG
    assert "workspace" in rr.last_error_message()


def test_noalloc_refuses_a_split_beyond_its_scratch():
    # 600 rows x 512 chunks x 16 bytes of (m, d) slots: more than the 4 MiB
    # static scratch; refused before any device work (the addresses are fake)
    M, N = 600, 1 << 21
    assert rr.rr_softmax_rows_ex_workspace_bytes(M, N, rr.RR_F32, rr.RR_F32) > 4 << 20
    f = rr.raw_softmax_rows_strided_noalloc
    assert f(P << 12, N, P, N, M, N, rr.RR_F32, rr.RR_F32, None, None) == rr.RR_ERR_WORKSPACE
    assert "scratch" in rr.last_error_message()
    # the ordinary argument checks still come first
    assert f(P << 12, N, P, N, M, 0, rr.RR_F32, rr.RR_F32, None, None) == rr.RR_ERR_INVALID_ARG
    assert f(None, N, P, N, M, N, rr.RR_F32, rr.RR_F32, None, None) == rr.RR_ERR_INVALID_ARG
    assert f(None, N, None, N, 0, N, rr.RR_F32, rr.RR_F32, None, None) == rr.RR_OK


def test_softmax_ex_validation():
    X, Y, W = P, P << 4, P << 8
    F, B = rr.RR_F32, rr.RR_BF16
    f = rr.raw_softmax_rows_ex
    o = rr.make_softmax_opts
    # flags outside {0, 1}
    bad = o()
    bad.log_output = 2
    assert f(Y, X, 4, 8, F, F, bad, None, 0, None) == rr.RR_ERR_INVALID_ARG
    assert "log_output" in rr.last_error_message()
    bad = o()
    bad.causal = -1
    assert f(Y, X, 4, 8, F, F, bad, None, 0, None) == rr.RR_ERR_INVALID_ARG
    # causal rule bounds
    assert f(Y, X, 4, 8, F, F, o(causal_period=0), None, 0, None) == rr.RR_ERR_INVALID_ARG
    assert "causal_period" in rr.last_error_message()
    assert f(Y, X, 4, 8, F, F, o(causal_period=4, causal_offset=-1), None, 0, None) == rr.RR_ERR_INVALID_ARG
    assert "causal_offset" in rr.last_error_message()
    # period and offset are ignored without the causal flag
    ign = o()
    ign.causal_period, ign.causal_offset = -5, -5
    assert f(Y, X, 0, 8, F, F, ign, None, 0, None) == rr.RR_OK
    # the plain checks still apply
    assert f(Y, X, 4, 0, F, F, None, None, 0, None) == rr.RR_ERR_INVALID_ARG
    assert f(X, X, 4, 8, B, F, o(log_output=True), None, 0, None) == rr.RR_ERR_INVALID_ARG
    # an empty batch succeeds before the options' pointers are needed
    assert f(None, None, 0, 8, F, F, o(causal_period=3), None, 0, None) == rr.RR_OK
    # log-softmax of few long rows splits like softmax and needs the workspace
    need = rr.rr_softmax_rows_ex_workspace_bytes(40, 152064, B, F, o(log_output=True))
    assert need == rr.rr_softmax_rows_workspace_bytes(40, 152064, B, F) == split_ws(40, 19)
    assert f(Y, X, 40, 152064, B, F, o(log_output=True), None, 0, None) == rr.RR_ERR_WORKSPACE
    # a causal call never splits, so it needs no workspace
    assert rr.rr_softmax_rows_ex_workspace_bytes(40, 152064, B, F, o(causal_period=40)) == 0
    assert rr.rr_softmax_rows_ex_workspace_bytes(40, 152064, B, F, None) == need
    assert rr.rr_softmax_rows_ex_workspace_bytes(4, 8, F, F, o(causal_period=0)) == 0


def test_softmax_causal_plans():
    S, C, F, B = rr.RR_OP_SOFTMAX, rr.RR_OP_SOFTMAX_CAUSAL, rr.RR_F32, rr.RR_BF16
    q = lambda op, M, N, a=F, b=F: rr.rr_query_plan(op, M, N, a, b)
    # rows that fit registers keep the softmax plan
    for M, N in ((28 * 4096, 4096), (16384, 1024), (10, 64), (1024, 40000)):
        assert q(C, M, N) == q(S, M, N)
    # where softmax would split (few long rows), the causal call holds the row
    # in one workgroup if it fits, else streams it
    assert q(S, 40, 152064, B, F)["variant_name"] == "split"
    p = q(C, 40, 152064, B, F)
    assert (p["variant_name"], p["block_threads"], p["workspace_bytes"]) == ("block", 1024, 0)
    p = q(C, 40, 200000, B, F)
    assert p["variant_name"] == "loop" and p["workspace_bytes"] == 0
    assert q(S, 40, 200000, B, F)["variant_name"] == "split"
    # from 56 rows up (bf16 -> fp32) softmax also holds such rows in one workgroup
    assert q(S, 64, 152064, B, F) == q(C, 64, 152064, B, F)
    assert q(S, 64, 152064, B, F)["variant_name"] == "block" and q(S, 63, 152064, B, F)["variant_name"] == "split"
    with rr.forced_variant(rr.RR_VARIANT_SPLIT):
        with pytest.raises(rr.RowReduceError):
            q(C, 10, 1024)
        assert q(S, 10, 1024)["variant_name"] == "split"
    with rr.forced_variant(rr.RR_VARIANT_LOOP):
        assert q(C, 10, 1024)["variant_name"] == "loop"


def test_strided_validation():
    """Stride bounds and the aliasing rules of the strided entry points (all
    rejected on the host before anything is enqueued)."""
    F, B, I = rr.RR_F32, rr.RR_BF16, rr.RR_ERR_INVALID_ARG
    X, Y, R, G = P, P << 4, P << 8, P << 12
    H = 64
    rms = rr.raw_rmsnorm_strided
    # strides below the row width, or absurdly large
    assert rms(Y, H, X, H - 1, G, 4, H, 1e-6, F, None) == I and "ldx" in rr.last_error_message()
    assert rms(Y, 0, X, H, G, 4, H, 1e-6, F, None) == I and "ldy" in rr.last_error_message()
    assert rms(Y, 1 << 41, X, H, G, 4, H, 1e-6, F, None) == I
    # y inside x's rows (same stride, overlapping column windows)
    assert rms(X + 4, 2 * H, X, 2 * H, G, 4, H, 1e-6, F, None) == I
    assert "overlaps" in rr.last_error_message()
    # in place needs the same stride
    assert rms(X, 2 * H, X, H, G, 4, H, 1e-6, F, None) == I
    # different strides with intersecting spans count as overlapping
    assert rms(X + 4 * H, 3 * H, X, 2 * H, G, 4, H, 1e-6, F, None) == I
    # gamma inside y's span
    assert rms(Y, 2 * H, X, H, Y + 4 * H, 4, H, 1e-6, F, None) == I
    # fused: the residual's window overlaps x's
    fz = rr.raw_fused_add_rmsnorm_strided
    assert fz(Y, H, X + 8, 2 * H, X, 2 * H, G, 4, H, 1e-6, B, None) == I
    assert "residual" in rr.last_error_message()
    assert fz(Y, H, R, H - 8, X, H, G, 4, H, 1e-6, B, None) == I and "ldr" in rr.last_error_message()
    # layernorm: beta inside y's span
    ln = rr.raw_layernorm_strided
    assert ln(Y, 2 * H, X, H, G, Y + 4, 4, H, 1e-5, F, None) == I
    # softmax: in place needs equal pointers, strides and dtypes
    sm = rr.raw_softmax_rows_strided
    assert sm(X, 2 * H, X, H, 4, H, F, F, None, None, 0, None) == I
    assert sm(X, H, X, H, 4, H, B, F, None, None, 0, None) == I
    assert sm(Y, H, X, H - 1, 4, H, F, F, None, None, 0, None) == I
    # options are still checked
    assert sm(Y, H, X, H, 4, H, F, F, rr.make_softmax_opts(causal_period=0), None, 0, None) == I
    # M == 0 is a no-op whatever the pointers
    assert rms(None, H, None, H, None, 0, H, 1e-6, F, None) == rr.RR_OK
    assert sm(None, H, None, H, 0, H, F, F, None, None, 0, None) == rr.RR_OK


# ----------------------------------------------------------------------------
# dispatch (the variant choice by row length)
# ----------------------------------------------------------------------------

WORKLOAD_PLANS = [
    # op, M, N, in, out -> variant, waves_per_row, vecs_per_lane, vec_elems, chunks
    # (workgroup-per-row plans keep two 16-byte loads in flight per lane)
    ((rr.RR_OP_RMSNORM, 64, 3584, rr.RR_F32, rr.RR_F32), ("block", 7, 2, 4, 1)),
    ((rr.RR_OP_FUSED_ADD_RMSNORM, 8192, 4096, rr.RR_BF16, rr.RR_BF16), ("block", 8, 1, 8, 1)),
    ((rr.RR_OP_RMSNORM, 8192, 4096, rr.RR_BF16, rr.RR_BF16), ("block", 4, 2, 8, 1)),
    ((rr.RR_OP_SOFTMAX, 16384, 1024, rr.RR_F32, rr.RR_F32), ("wave", 1, 4, 4, 1)),
    # bf16 read 4 elements (8 bytes) at a time when written as fp32
    ((rr.RR_OP_SOFTMAX, 256, 152064, rr.RR_BF16, rr.RR_F32), ("block", 16, 38, 4, 1)),
    ((rr.RR_OP_SOFTMAX, 55, 152064, rr.RR_BF16, rr.RR_F32), ("split", 4, 8, 4, 19)),
    ((rr.RR_OP_SOFTMAX, 4096, 32000, rr.RR_BF16, rr.RR_F32), ("block", 16, 8, 4, 1)),
    ((rr.RR_OP_SOFTMAX, 4096, 32000, rr.RR_BF16, rr.RR_BF16), ("block", 16, 4, 8, 1)),
    ((rr.RR_OP_SOFTMAX, 2048, 131072, rr.RR_BF16, rr.RR_F32), ("block", 16, 32, 4, 1)),
    ((rr.RR_OP_SOFTMAX, 28 * 4096, 4096, rr.RR_F32, rr.RR_F32), ("block", 8, 2, 4, 1)),
]


@pytest.mark.parametrize("args,expect", WORKLOAD_PLANS)
def test_dispatch_named_workloads(args, expect):
    p = rr.rr_query_plan(*args)
    got = (p["variant_name"], p["waves_per_row"], p["vecs_per_lane"], p["vec_elems"],
           p["chunks_per_row"])
    assert got == expect


def test_dispatch_boundaries():
    S, F, B = rr.RR_OP_SOFTMAX, rr.RR_F32, rr.RR_BF16
    v = lambda op, M, N, a=F, b=F, al=True: rr.rr_query_plan(op, M, N, a, b, al)["variant_name"]
    # softmax: a wavefront per row up to 2048 elements (32 fp32 per lane)
    assert v(S, 100, 2048) == "wave"
    assert v(S, 100, 2052) == "block"
    assert v(S, 100, 2048, B, B) == "wave"
    # norms keep 16 values per lane: a wavefront up to 1024, then a block
    assert v(rr.RR_OP_RMSNORM, 100, 1024) == "wave"
    assert v(rr.RR_OP_RMSNORM, 100, 1028) == "block"
    # block capacity: 16 wavefronts x 64 lanes x 16 (norm) or 32 (softmax) values
    assert v(rr.RR_OP_RMSNORM, 100, 16384) == "block"
    # longer norm rows are held packed by 1024 lanes up to 64K elements
    q = lambda op, N, a=F: rr.rr_query_plan(op, 3, N, a, a)
    assert q(rr.RR_OP_RMSNORM, 16388)["vecs_per_lane"] == 8 and q(rr.RR_OP_RMSNORM, 16388)["block_threads"] == 1024
    assert q(rr.RR_OP_LAYERNORM, 40000)["vecs_per_lane"] == 12
    assert q(rr.RR_OP_RMSNORM, 65536)["vecs_per_lane"] == 16
    assert q(rr.RR_OP_RMSNORM, 65540)["variant_name"] == "loop"
    assert q(rr.RR_OP_FUSED_ADD_RMSNORM, 32768)["vecs_per_lane"] == 8
    assert q(rr.RR_OP_FUSED_ADD_RMSNORM, 32772)["variant_name"] == "loop"     # fp32 fused: x and residual
    assert q(rr.RR_OP_FUSED_ADD_RMSNORM, 65536, B)["vecs_per_lane"] == 8
    assert q(rr.RR_OP_RMSNORM, 20480, B)["vecs_per_lane"] == 4
    assert q(rr.RR_OP_RMSNORM, 65544, B)["variant_name"] == "loop"
    assert v(S, 100, 32768) == "block"
    # longer softmax rows: split when rows are few; from 40 (fp32 in), 56
    # (bf16 -> fp32) or 80 (bf16 -> bf16) rows up the row is held packed (1024
    # lanes x up to 20 16-byte vectors); rows longer than that split below
    # 1024 rows and stream from 1024 rows up
    assert v(S, 47, 32772) == "split"
    assert v(S, 48, 32772) == "block"
    assert v(S, 63, 32772, F, B) == "split" and v(S, 64, 32772, F, B) == "block"
    assert v(S, 63, 65536, B, F) == "split" and v(S, 64, 65536, B, F) == "block"
    assert v(S, 79, 65536, B, B) == "split" and v(S, 80, 65536, B, B) == "block"
    assert rr.rr_query_plan(S, 64, 32772, F, F)["vecs_per_lane"] == 12
    assert v(S, 64, 81920) == "block"
    assert v(S, 64, 81924) == "split"
    assert v(S, 1023, 81924) == "split"
    assert v(S, 1024, 81924) == "loop"
    assert v(S, 1024, 163840, B, F) == "block"
    assert v(S, 1024, 163840, B, B) == "block"
    assert v(S, 1024, 163848, B, F) == "loop"
    assert v(S, 1023, 163848, B, F) == "split"
    # many rows written as fp32: workgroups of 2-vector lanes instead of a
    # wavefront holding 8 vectors (from 16384 rows) or 4 (from 65536 rows)
    assert v(S, 16383, 2048) == "wave" and v(S, 16384, 2048) == "block"
    assert rr.rr_query_plan(S, 16384, 2048, F, F)["vecs_per_lane"] == 2
    assert v(S, 65535, 1024, B, F) == "wave" and v(S, 65536, 1024, B, F) == "block"
    assert v(S, 16384, 1024) == "wave" and v(S, 131072, 2048, B, B) == "wave"
    # short rows: several rows per wavefront, L lanes per row
    assert v(S, 10, 128) == "subwave" and rr.rr_query_plan(S, 10, 128, F, F)["waves_per_row"] == 32
    assert v(S, 10, 132) == "wave"
    assert rr.rr_query_plan(S, 10, 8, F, F)["waves_per_row"] == 2
    assert rr.rr_query_plan(S, 10, 1, F, F)["waves_per_row"] == 1
    assert v(rr.RR_OP_FUSED_ADD_RMSNORM, 10, 256, B, B) == "subwave"
    assert v(S, 10, 7) == "subwave" and rr.rr_query_plan(S, 10, 7, F, F)["vec_elems"] == 1
    # softmax rows that are not whole aligned vectors (a ragged width, or rows
    # starting at a common offset within a vector) are cut at aligned
    # addresses and held like aligned rows (row_shift); up to 32 elements they
    # keep the scalar short-row path
    sh = lambda M, N, a=F, b=F, al=2, op=S: rr.rr_query_plan(op, M, N, a, b, al)
    assert v(S, 10, 20, al=2) == "subwave" and sh(10, 20)["vec_elems"] == 1 and sh(10, 20)["row_shift"] == 0
    # (vectors per lane with aligned starts and a ragged width, lead 0; with
    # starts at a common offset, room for a lead of up to vec - 1 elements)
    for M, N, a, b, name, nv1, nv2 in ((10, 33, F, F, "wave", 1, 1), (10, 1023, F, F, "wave", 4, 8),
                                       (16384, 1025, F, F, "wave", 8, 8), (8192, 4097, F, F, "block", 2, 2),
                                       (256, 50257, B, F, "block", 24, 24), (104, 50257, B, B, "block", 12, 12),
                                       (88, 50257, F, B, "block", 16, 16)):
        for al, nv in ((True, nv1), (2, nv2)):
            p = sh(M, N, a, b, al)
            assert (p["variant_name"], p["vecs_per_lane"], p["row_shift"]) == (name, nv, 1), (M, N, al, p)
            assert p["vec_elems"] == (4 if (a, b) != (B, B) else 8) and p["workspace_bytes"] == 0, p
    assert sh(64, 4097, op=rr.RR_OP_SOFTMAX_CAUSAL)["row_shift"] == 1
    # beyond a workgroup's registers with few rows (below 72 / 88 / 88 / 104
    # cut rows by dtype pair), or beyond the packed workgroup below 1024 rows: the split, its chunks sized for a row
    # at any offset (so that the workspace query, which sees no addresses,
    # covers every call); a causal call never splits
    for M, N, a, b, vec, nv, chunks in ((3, 50257, B, B, 8, 4, 7), (2, 50257, F, B, 4, 4, 13),
                                        (1, 50257, B, F, 4, 8, 7), (4, 152065, F, F, 4, 4, 38),
                                        (1023, 81925, F, F, 4, 4, 21), (4, 65536, F, F, 4, 4, 17)):
        for al in (True, 2):
            if al is True and N % vec == 0:
                continue
            p = sh(M, N, a, b, al)
            assert (p["variant_name"], p["row_shift"], p["vec_elems"], p["vecs_per_lane"]) == ("split", 1, vec, nv), p
            assert p["chunks_per_row"] == chunks and p["workspace_bytes"] == split_ws(M, chunks), p
            assert rr.rr_softmax_rows_workspace_bytes(M, N, a, b) == split_ws(M, chunks)
    assert rr.rr_query_plan(S, 4, 65536, F, F)["chunks_per_row"] == 16   # aligned rows: one chunk fewer
    assert sh(4, 50257, op=rr.RR_OP_SOFTMAX_CAUSAL)["variant_name"] == "block"
    # cut rows hand over to the packed kernel 24 rows later than aligned ones
    assert sh(87, 50257, B, F)["variant_name"] == "split" and sh(88, 50257, B, F)["variant_name"] == "block"
    assert sh(71, 50257)["variant_name"] == "split" and sh(72, 50257)["variant_name"] == "block"
    assert v(S, 63, 50256, B, F) == "split" and v(S, 64, 50256, B, F) == "block"
    # too long to hold with 1024 rows or more (or a causal call): the
    # streaming kernel, cut the same way; element access requested: scalar
    p = sh(1024, 81925)
    assert (p["variant_name"], p["vec_elems"], p["row_shift"], p["waves_per_row"]) == ("loop", 4, 1, 16), p
    p = sh(4, 200003, B, F, op=rr.RR_OP_SOFTMAX_CAUSAL)
    assert (p["variant_name"], p["vec_elems"], p["row_shift"], p["workspace_bytes"]) == ("loop", 4, 1, 0), p
    assert v(S, 10, 1024, al=False) == "loop" and sh(10, 1024, al=False)["row_shift"] == 0
    # norm rows that are not whole aligned vectors: cut at aligned addresses
    # in the register kernels (gamma read in each row's frame); longer ones
    # stream element by element
    for op in (rr.RR_OP_RMSNORM, rr.RR_OP_FUSED_ADD_RMSNORM, rr.RR_OP_LAYERNORM):
        for al in (True, 2):
            p = sh(10, 4100, B, B, al, op)                 # 4100 % 8 != 0
            assert (p["variant_name"], p["row_shift"], p["vec_elems"]) == ("block", 1, 8), p
        p = sh(4096, 1021, F, F, 2, op)
        # (an fp32 LayerNorm keeps to 2 vectors per lane on cut rows)
        want = "block" if op == rr.RR_OP_LAYERNORM else "wave"
        assert (p["variant_name"], p["row_shift"], p["vec_elems"]) == (want, 1, 4), p
        assert op != rr.RR_OP_LAYERNORM or p["vecs_per_lane"] <= 2, p
        p = sh(10, 20001, F, F, 2, op)                      # past the register budget
        assert (p["variant_name"], p["row_shift"], p["vec_elems"]) == ("loop", 0, 1), p
    assert v(rr.RR_OP_RMSNORM, 10, 4100, B, B, al=False) == "loop"


def test_forced_variants():
    S, F = rr.RR_OP_SOFTMAX, rr.RR_F32
    with rr.forced_variant(rr.RR_VARIANT_LOOP):
        assert rr.rr_query_plan(S, 10, 1024, F, F)["variant_name"] == "loop"
    with rr.forced_variant(rr.RR_VARIANT_SPLIT):
        p = rr.rr_query_plan(S, 10, 1024, F, F)
        assert p["variant_name"] == "split" and p["workspace_bytes"] == split_ws(10, 1)
        assert rr.rr_softmax_rows_workspace_bytes(10, 1024, F, F) == split_ws(10, 1)
        p = rr.rr_query_plan(S, 10, 1023, F, F, 2)      # a row cut at aligned addresses
        assert (p["variant_name"], p["row_shift"], p["vec_elems"]) == ("split", 1, 4)
    with rr.forced_variant(rr.RR_VARIANT_SPLIT_ONE_KERNEL):
        p = rr.rr_query_plan(S, 10, 5000, F, F)
        assert p["variant_name"] == "split1" and p["chunks_per_row"] == 2
        # the workspace query covers the aligned call even though cut rows are refused
        assert rr.rr_softmax_rows_workspace_bytes(10, 5000, F, F) == split_ws(10, 2)
        assert rr.rr_softmax_rows_workspace_bytes(1, 8, F, F) == split_ws(1, 1)
        with pytest.raises(rr.RowReduceError):
            rr.rr_query_plan(S, 10, 5001, F, F)               # the one-kernel form takes aligned rows
        with pytest.raises(rr.RowReduceError):
            rr.rr_query_plan(rr.RR_OP_RMSNORM, 10, 1024, F, F)   # no split RMSNorm
    with rr.forced_variant(rr.RR_VARIANT_WAVE):
        with pytest.raises(rr.RowReduceError):
            rr.rr_query_plan(S, 10, 4096, F, F)                  # row too long for a wave
    with pytest.raises(rr.RowReduceError):
        with rr.forced_variant(9):
            pass
    assert rr.rr_query_plan(S, 10, 1024, F, F)["variant_name"] == "wave"   # automatic again
    # the product library has no override at all; the diagnostics build, back
    # at automatic choice, plans exactly as the product does
    assert not hasattr(rr.binding.lib(), "rr_set_variant_override")
    D = rr.diag_lib()
    for shape in [(S, 10, 5000, F, F), (S, 256, 152064, rr.RR_BF16, F), (rr.RR_OP_RMSNORM, 8192, 4096, 1, 1)]:
        p = rr.binding.rr_plan()
        assert D.rr_query_plan(*shape, 1, ctypes.byref(p)) == rr.RR_OK
        assert p.as_dict() == rr.rr_query_plan(*shape), shape


def test_every_plan_covers_its_row():
    """For thousands of seeded (op, M, N, dtypes, alignment) cases, and every
    forced variant, the plan either is refused or holds the whole row: the
    register-resident kernels only ever touch lanes x vectors they were
    planned with, so a plan that did not cover N would silently drop the
    row's tail.  Also: thread counts within a workgroup's limit, workspace
    sizes for split plans, and work items that cover every row."""
    import numpy as np
    rng = np.random.default_rng(42)
    ops = [rr.RR_OP_RMSNORM, rr.RR_OP_FUSED_ADD_RMSNORM, rr.RR_OP_LAYERNORM, rr.RR_OP_SOFTMAX,
           rr.RR_OP_SOFTMAX_CAUSAL]
    variants = [rr.RR_VARIANT_AUTO, rr.RR_VARIANT_WAVE, rr.RR_VARIANT_BLOCK, rr.RR_VARIANT_SPLIT,
                rr.RR_VARIANT_LOOP, rr.RR_VARIANT_SPLIT_ONE_KERNEL, rr.RR_VARIANT_SUBWAVE,
                rr.RR_VARIANT_SPLIT_TWO_KERNELS]
    widths = np.concatenate([rng.integers(1, 300, 300), rng.integers(300, 70000, 400),
                             rng.integers(70000, 1 << 22, 100), [1 << 30, (1 << 30) - 8]])
    checked = 0
    for v in variants:
        with rr.forced_variant(v):
            for N in widths:
                N = int(N)
                op = ops[int(rng.integers(0, len(ops)))]
                M = int(rng.choice([0, 1, 7, 255, 256, 1023, 1024, 5000, 100000]))
                din = int(rng.integers(0, 2))
                dout = int(rng.integers(0, 2)) if op in (rr.RR_OP_SOFTMAX, rr.RR_OP_SOFTMAX_CAUSAL) else din
                aligned = [0, 1, 1, 2][int(rng.integers(0, 4))]   # element access, aligned, common offset
                try:
                    p = rr.rr_query_plan(op, M, N, din, dout, aligned)
                except rr.RowReduceError as e:
                    assert e.status == rr.RR_ERR_UNSUPPORTED and v != rr.RR_VARIANT_AUTO, (op, M, N, v)
                    continue
                checked += 1
                vec, nv, name = p["vec_elems"], p["vecs_per_lane"], p["variant_name"]
                width = 8 if din == rr.RR_BF16 else 4
                if op in (rr.RR_OP_SOFTMAX, rr.RR_OP_SOFTMAX_CAUSAL) and (din, dout) == (rr.RR_BF16, rr.RR_F32):
                    width = 4
                shift = p["row_shift"]
                if shift:
                    # rows cut at aligned addresses, room for the worst lead
                    # (vec - 1); the norms only in the register kernels
                    assert vec == width, p
                    assert aligned == 2 or (aligned == 1 and N % width != 0), p
                    assert name in ("wave", "block", "split", "split2", "loop"), p
                    if op not in (rr.RR_OP_SOFTMAX, rr.RR_OP_SOFTMAX_CAUSAL):
                        # (a workgroup's cut row may hold 3 bf16 vectors per lane)
                        assert name in ("wave", "block") and nv * vec <= (24 if nv == 3 else 16), p
                        assert nv != 3 or name == "block", p
                        if op == rr.RR_OP_LAYERNORM:
                            # an fp32 wavefront holds 2 vectors at most; a
                            # workgroup stages gamma and beta (at any lead) in LDS
                            assert not (name == "wave" and vec == 4 and nv > 2), p
                            lds = (N + 19) * 8 if vec == 4 else 2 * ((N + 2 * vec - 2) // vec) * 16
                            assert name == "wave" or lds <= 61440, p
                    if name == "loop":
                        pass                                  # streams any length
                    elif name in ("split", "split2"):
                        cap = p["chunks_per_row"] * 256 * nv * vec
                        assert cap >= N + vec - 1, p          # any lead, also with aligned starts
                    else:
                        cap = (64 if name == "wave" else p["block_threads"]) * nv * vec
                        assert cap >= (N if aligned == 1 else N + vec - 1), p
                else:
                    assert vec in (1, width) and (vec == 1 or (aligned == 1 and N % width == 0)), p
                assert 1 <= p["block_threads"] <= 1024 and p["block_threads"] % 64 == 0, p
                if name == "subwave":
                    assert p["waves_per_row"] * vec >= N and p["rows_per_group"] * p["waves_per_row"] == 256, p
                elif name == "wave":
                    assert 64 * nv * vec >= N and p["rows_per_group"] * 64 == p["block_threads"], p
                elif name == "block":
                    assert p["block_threads"] * nv * vec >= N and p["rows_per_group"] == 1, p
                elif name in ("split", "split1", "split2"):
                    assert op == rr.RR_OP_SOFTMAX and vec > 1, p
                    if v == rr.RR_VARIANT_AUTO:
                        assert rr.rr_softmax_rows_workspace_bytes(M, N, din, dout) >= p["workspace_bytes"], p
                    assert p["chunks_per_row"] * 256 * nv * vec >= N, p
                    assert p["workspace_bytes"] == split_ws(M, p["chunks_per_row"]), p
                    assert p["work_items"] == M * p["chunks_per_row"], p
                    continue
                else:
                    assert name == "loop", p
                assert p["workspace_bytes"] == 0, p
                assert p["work_items"] * p["rows_per_group"] >= M, p
    assert checked > 1500
