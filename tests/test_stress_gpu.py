"""Race stress of the LDS slot stages (GPU).

librowreduce_stress.so is the same source built with RR_STRESS=1: every LDS
slot stage pauses each wavefront for a random 0-7 x 512 cycles before its slot
write and before its slot reads, poisons the other slot set with NaN right
after each barrier, and every grid is capped at 37 workgroups so that each
workgroup walks many rows and reuses its two slot sets over and over.  None of
that changes any arithmetic, so a stage whose barriers order every write
before every read, and every read before the next write of the same slot,
gives the stress build the same bits as the normal one.  Each case below runs
a kernel family that has an LDS stage through both builds (the stress build
twice, its pauses differing) and requires bitwise-equal outputs.  The normal
build's results are checked against the oracle by the parity tests.
"""
import os

import numpy as np
import pytest

import row_reduction_rmsnorm_amd as rr
from row_reduction_rmsnorm_amd import build as rr_build

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

F32, BF16 = rr.RR_F32, rr.RR_BF16


@pytest.fixture(scope="module")
def libs():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert os.path.exists(rr_build.LIB_STRESS), "the race-stress build is missing (run build())"
    # the normal build: the diagnostics library, which links the product's
    # kernel object unchanged and can force the two-kernel split below
    normal = rr.diag_lib()
    stress = rr.load_library(rr_build.LIB_STRESS)
    for L in (normal, stress):
        L.rr_set_variant_override(rr.RR_VARIANT_AUTO)
    yield normal, stress
    for L in (normal, stress):
        L.rr_set_variant_override(rr.RR_VARIANT_AUTO)


def _say(*a):
    print(*a, flush=True)


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _dev(a, dt):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return (t if dt == F32 else t.to(torch.bfloat16)).cuda()


def _bits(t):
    return t.view(torch.int32 if t.dtype == torch.float32 else torch.int16).cpu()


def _plan(op, M, N, din, dout=None):
    return rr.rr_query_plan(op, M, N, din, din if dout is None else dout)["variant_name"]


def _same_three_ways(run):
    """run(L) -> output tensor; normal build once, stress build twice."""
    normal, stress = LIBS
    ref = _bits(run(normal))
    for k in range(2):
        got = _bits(run(stress))
        assert torch.equal(ref, got), f"stress build run {k} differs from the normal build"


LIBS = None


@pytest.fixture(autouse=True)
def _set_libs(libs):
    global LIBS
    LIBS = libs
    yield


def _norm_rows(M, N, seed, far_every=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, N)).astype(np.float32)
    if far_every:
        x[::far_every, 0] = 1.0e3           # first element far from the row mean
    g = rng.uniform(0.5, 1.5, N).astype(np.float32)
    b = rng.uniform(-1.0, 1.0, N).astype(np.float32)
    return x, g, b


NORM_CASES = [
    # (op, dtype, M, N, expected plan)
    ("rms", BF16, 257, 4096, "block"),
    ("rms", F32, 100, 20480, "block"),      # packed (more than 16 values per lane)
    ("rms", F32, 64, 70001, "loop"),
    ("fused", BF16, 257, 4096, "block"),
    ("fused", BF16, 100, 20480, "block"),
    ("layer", F32, 257, 5120, "block"),
    ("layer", BF16, 100, 20480, "block"),
    ("layer", BF16, 64, 70000, "loop"),
    ("rms", BF16, 257, 4097, "block"),      # rows cut at aligned addresses (every lead)
    ("fused", BF16, 100, 4097, "block"),
    ("layer", F32, 100, 5121, "block"),     # gamma and beta staged in LDS (fp32 entries)
    ("layer", BF16, 100, 4097, "block"),    # (bf16 blocks)
]


@pytest.mark.parametrize("op,dt,M,N,plan", NORM_CASES)
def test_norm_lds_stages_under_stress(op, dt, M, N, plan):
    _say(f"stress {op} dt={dt} {M}x{N}")
    code = {"rms": rr.RR_OP_RMSNORM, "fused": rr.RR_OP_FUSED_ADD_RMSNORM, "layer": rr.RR_OP_LAYERNORM}[op]
    assert _plan(code, M, N, dt) == plan
    x, g, b = _norm_rows(M, N, seed=M + N, far_every=5 if op == "layer" else 0)
    xd, gd, bd = _dev(x, dt), _dev(g, dt), _dev(b, dt)
    r0 = _dev(np.random.default_rng(1).standard_normal((M, N)), dt)

    def run(L):
        y = torch.empty_like(xd)
        if op == "rms":
            st = L.rr_rmsnorm(y.data_ptr(), xd.data_ptr(), gd.data_ptr(), M, N, 1e-6, dt, _stream())
        elif op == "layer":
            st = L.rr_layernorm(y.data_ptr(), xd.data_ptr(), gd.data_ptr(), bd.data_ptr(), M, N, 1e-5, dt,
                                _stream())
        else:
            res = r0.clone()
            st = L.rr_fused_add_rmsnorm(y.data_ptr(), res.data_ptr(), xd.data_ptr(), gd.data_ptr(), M, N,
                                        1e-6, dt, _stream())
        assert st == 0, st
        torch.cuda.synchronize()
        return torch.cat([y, res]) if op == "fused" else y
    _same_three_ways(run)


def _softmax_rows(M, N, seed):
    rng = np.random.default_rng(seed)
    x = (8.0 * rng.standard_normal((M, N))).astype(np.float32)
    x[1::3] += 1000.0
    x[::2, N // 3:] = -np.inf              # masked tails on even rows (the head stays finite)
    return x


SOFTMAX_CASES = [
    # (in dtype, out dtype, M, N, expected plan, log output)
    (F32, F32, 300, 4096, "block", 0),
    (F32, F32, 300, 4097, "block", 0),      # a ragged width: rows cut at aligned addresses
    (BF16, F32, 96, 50257, "block", 1),     # the same, packed, log output
    (F32, F32, 1024, 81924, "loop", 0),     # too long to hold with this many rows: streams
    (BF16, F32, 80, 152064, "block", 0),    # packed
    (BF16, F32, 80, 152064, "block", 1),
    (F32, F32, 4, 152064, "split", 0),
    (BF16, F32, 4, 152064, "split", 1),
    (F32, F32, 40, 1 << 19, "split", 0),    # more than 64 chunks: the merge kernel runs
    (BF16, F32, 4, 50257, "split", 1),      # split rows cut at aligned addresses
    (F32, F32, 40, (1 << 19) + 3, "split", 0),
]


@pytest.mark.parametrize("din,dout,M,N,plan,log", SOFTMAX_CASES)
def test_softmax_lds_stages_under_stress(din, dout, M, N, plan, log):
    _say(f"stress softmax {din}->{dout} {M}x{N} log={log}")
    assert _plan(rr.RR_OP_SOFTMAX, M, N, din, dout) == plan
    xd = _dev(_softmax_rows(M, N, seed=N + M), din)
    opts = rr.make_softmax_opts(log_output=bool(log))

    def run(L):
        y = torch.empty((M, N), dtype=torch.float32 if dout == F32 else torch.bfloat16, device="cuda")
        nb = L.rr_softmax_rows_ex_workspace_bytes(M, N, din, dout, opts)
        ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
        st = L.rr_softmax_rows_ex(y.data_ptr(), xd.data_ptr(), M, N, din, dout, opts, ws.data_ptr(), nb,
                                  _stream())
        assert st == 0, st
        torch.cuda.synchronize()
        return y
    _same_three_ways(run)


def test_causal_rule_and_two_kernel_split_under_stress():
    """The causal rule's workgroup-per-row stage (one row per workgroup, and
    two rows of a period per workgroup with one shared barrier), and the
    split row forced to its two-kernel form (the default split plans above
    run the one-kernel form, whose grid is one workgroup per chunk)."""
    M, N = 300, 4096
    xd = _dev(_softmax_rows(M, N, seed=3), F32)
    for P, O in ((128, N - 128), (128, 0), (97, 0)):
        _say(f"stress causal rule {M}x{N} P={P} O={O}")
        causal = rr.make_softmax_opts(causal_period=P, causal_offset=O)

        def run_causal(L):
            y = torch.empty((M, N), dtype=torch.float32, device="cuda")
            st = L.rr_softmax_rows_ex(y.data_ptr(), xd.data_ptr(), M, N, F32, F32, causal, None, 0, _stream())
            assert st == 0, st
            torch.cuda.synchronize()
            return y
        _same_three_ways(run_causal)

    M, N = 4, 152064
    _say(f"stress two-kernel split {M}x{N}")
    xs = _dev(_softmax_rows(M, N, seed=4), F32)
    normal, stress = LIBS

    def run_split(L):
        y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        nb = L.rr_softmax_rows_workspace_bytes(M, N, F32, F32)
        ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
        assert L.rr_set_variant_override(rr.RR_VARIANT_SPLIT_TWO_KERNELS) == 0
        try:
            st = L.rr_softmax_rows(y.data_ptr(), xs.data_ptr(), M, N, F32, F32, ws.data_ptr(), nb, _stream())
        finally:
            L.rr_set_variant_override(rr.RR_VARIANT_AUTO)
        assert st == 0, st
        torch.cuda.synchronize()
        return y
    _same_three_ways(run_split)
