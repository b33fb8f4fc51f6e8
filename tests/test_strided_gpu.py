"""GPU parity of the strided entry points: rows that are column slices of
wider matrices (a row stride larger than the width), against the fp64
oracle on the same rows gathered contiguously.

Checked as well: the elements between the slices are never written, the
strided calls with stride equal to the width give the bits of the
contiguous calls, outputs into another column slice of the input's own
buffer, the fused op writing its output back into its strided input, and
unaligned strides (the scalar path).
"""
import numpy as np
import pytest

import oracle
import workloads
from tests import compare
from tests.test_parity_gpu import (DTYPES, _as, _bits, _rr, _say, _tdt, check_fused, check_norm,
                                   softmax_input)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SENTINEL = 7.25   # exact in fp32 and bf16


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rr = _rr()
    rr.lib()
    yield


def embed(rows_cpu, ld, col0, fill=SENTINEL):
    """A [M, ld] device buffer holding rows_cpu in columns col0 .. col0+N-1
    and `fill` elsewhere; returns (buffer, view of the rows)."""
    M, N = rows_cpu.shape
    buf = torch.full((M, ld), fill, dtype=rows_cpu.dtype, device="cuda")
    buf[:, col0:col0 + N] = rows_cpu.cuda()
    return buf, buf[:, col0:col0 + N]


def untouched(buf, col0, N, what):
    """Every element outside columns col0 .. col0+N-1 still holds SENTINEL."""
    b = buf.float().cpu()
    mask = torch.ones(b.shape, dtype=torch.bool)
    mask[:, col0:col0 + N] = False
    assert bool((b[mask] == SENTINEL).all()), f"{what}: wrote outside the slice"


# (M, N, ld_x, col_x, ld_y, col_y): aligned strides on each path (short rows,
# a wavefront per row, a workgroup per row, streaming), and unaligned strides
# or column offsets (the scalar path)
NORM_CASES = [
    (100, 24, 64, 8, 40, 16),
    (33, 1024, 3072, 1024, 1536, 512),
    (9, 4096, 12288, 4096, 8192, 0),
    (7, 20000, 20480, 0, 24576, 4096),
    (17, 1000, 1003, 3, 1001, 1),
    (5, 3584, 3592, 8, 3584, 0),
]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("case", NORM_CASES, ids=lambda c: "x".join(map(str, c)))
def test_rmsnorm_and_layernorm_strided(case, dt):
    rr = _rr()
    M, N, ldx, cx, ldy, cy = case
    _say(f"strided norms {dt} {case}")
    x_cpu = _as(workloads.random_rows(M, N, seed=M + N), dt)
    g_cpu = _as(workloads.gamma_vector(N, seed=N), dt)
    b_cpu = _as(workloads.gamma_vector(N, seed=N + 1) - 1.0, dt)
    xbuf, xv = embed(x_cpu, ldx, cx)
    ybuf, yv = embed(torch.zeros(M, N, dtype=_tdt(dt)), ldy, cy)
    rr.rr_rmsnorm_strided(yv, xv, g_cpu.cuda(), 1e-6)
    torch.cuda.synchronize()
    check_norm(x_cpu, g_cpu, 1e-6, dt, yv.cpu(), f"rms strided {dt} {case}")
    untouched(ybuf, cy, N, "rms y")
    untouched(xbuf, cx, N, "rms x")
    rr.rr_layernorm_strided(yv, xv, g_cpu.cuda(), b_cpu.cuda(), 1e-5)
    torch.cuda.synchronize()
    ref = oracle.layernorm(compare.to_f64(x_cpu), compare.to_f64(g_cpu), compare.to_f64(b_cpu), 1e-5)
    compare.check_layernorm(yv.cpu(), ref, compare.to_f64(g_cpu), compare.to_f64(b_cpu),
                            f"layernorm strided {dt} {case}")
    untouched(ybuf, cy, N, "layernorm y")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("case", NORM_CASES, ids=lambda c: "x".join(map(str, c)))
def test_fused_strided_output_into_input(case, dt):
    """vLLM's layout: x is a strided slice, the residual is its own
    (here also strided) matrix, and y is written back over x."""
    rr = _rr()
    M, N, ldx, cx, ldr, cr = case
    _say(f"strided fused {dt} {case}")
    x_cpu = _as(workloads.random_rows(M, N, seed=2 * M + N), dt)
    r_cpu = _as(workloads.random_rows(M, N, seed=3 * M + N), dt)
    g_cpu = _as(workloads.gamma_vector(N, seed=N + 2), dt)
    xbuf, xv = embed(x_cpu, ldx, cx)
    rbuf, rv = embed(r_cpu, ldr, cr)
    rr.rr_fused_add_rmsnorm_strided(xv, rv, xv, g_cpu.cuda(), 1e-6)
    torch.cuda.synchronize()
    check_fused(x_cpu, r_cpu, g_cpu, 1e-6, dt, xv.cpu(), rv.cpu(), f"fused strided {dt} {case}")
    untouched(xbuf, cx, N, "fused x/y")
    untouched(rbuf, cr, N, "fused residual")


STRIDED_SOFTMAX = [
    # M, N, ld_x, col_x, ld_y, col_y
    (300, 16, 48, 16, 16, 0),
    (64, 1024, 4096, 2048, 1024, 0),
    (20, 4096, 8192, 4096, 4104, 8),
    (9, 40000, 40008, 8, 40000, 0),
    (3, 152064, 152080, 16, 152072, 8),
    (11, 999, 1000, 1, 1003, 2),
]


@pytest.mark.parametrize("log_output", [False, True])
@pytest.mark.parametrize("din,dout", DTYPES)
@pytest.mark.parametrize("case", STRIDED_SOFTMAX, ids=lambda c: "x".join(map(str, c)))
def test_softmax_strided(case, din, dout, log_output):
    rr = _rr()
    M, N, ldx, cx, ldy, cy = case
    _say(f"strided softmax {din}->{dout} log={log_output} {case}")
    x_cpu = softmax_input(M, N, seed=M * 7 + N, dt=din)
    xbuf, xv = embed(x_cpu, ldx, cx)
    ybuf, yv = embed(torch.zeros(M, N, dtype=_tdt(dout)), ldy, cy)
    opts = rr.make_softmax_opts(log_output=log_output)
    n = rr.rr_softmax_rows_ex_workspace_bytes(M, N, rr.dtype_code(xv), rr.dtype_code(yv), opts)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda") if n else None
    rr.rr_softmax_rows_strided(yv, xv, opts, ws)
    torch.cuda.synchronize()
    xf = compare.to_f64(x_cpu)
    if log_output:
        compare.check_log_softmax(yv.cpu(), xf, oracle.log_softmax(xf), f"log strided {case}")
    else:
        compare.check_softmax(yv.cpu(), xf, oracle.softmax(xf), f"softmax strided {case}")
    untouched(ybuf, cy, N, "softmax y")


def test_softmax_strided_causal_into_own_buffer():
    """Scores as column slices of one buffer, probabilities written into the
    buffer's other half: disjoint column windows with one stride are not an
    overlap.  The causal rule reads only kept keys."""
    rr = _rr()
    M, N = 64, 1024
    x_cpu = softmax_input(M, N, seed=77, dt="f32")
    buf = torch.full((M, 2 * N), SENTINEL, device="cuda")
    buf[:, :N] = x_cpu.cuda()
    xv, yv = buf[:, :N], buf[:, N:]
    rr.rr_softmax_rows_strided(yv, xv, rr.make_softmax_opts(causal_period=M, causal_offset=N - M))
    torch.cuda.synchronize()
    xf = compare.to_f64(x_cpu)
    keys = np.minimum(N, np.arange(M) % M + (N - M) + 1)
    xf[np.arange(N)[None, :] >= keys[:, None]] = -np.inf
    compare.check_softmax(yv.cpu(), xf, oracle.softmax(xf), "causal strided own buffer")
    assert torch.equal(buf[:, :N].cpu(), x_cpu), "input half changed"


def test_stride_equal_to_width_is_the_contiguous_call_bitwise():
    rr = _rr()
    for dt in ("f32", "bf16"):
        M, N = 64, 4096
        x = _as(workloads.random_rows(M, N, seed=5), dt).cuda()
        g = _as(workloads.gamma_vector(N, seed=6), dt).cuda()
        a, b = torch.empty_like(x), torch.empty_like(x)
        rr.rr_rmsnorm(a, x, g, 1e-6)
        rr.rr_rmsnorm_strided(b, x, g, 1e-6)
        torch.cuda.synchronize()
        assert torch.equal(_bits(a), _bits(b))
        s = softmax_input(M, N, seed=9, dt=dt).cuda()
        a = torch.empty(M, N, device="cuda")
        b = torch.empty_like(a)
        rr.rr_softmax_rows(a, s, None)
        rr.rr_softmax_rows_strided(b, s)
        torch.cuda.synchronize()
        assert torch.equal(_bits(a), _bits(b))


def test_bf16_to_f32_softmax_on_8_byte_aligned_rows_is_the_aligned_call_bitwise():
    """A bf16 softmax written as fp32 reads 8 bytes per vector, so rows that
    start 8 (not 16) bytes into a line take the same vector kernel: the same
    bits as the same rows stored 16-byte aligned, and the oracle's values."""
    rr = _rr()
    for (M, N) in [(33, 100), (40, 1028), (9, 32004), (3, 152068), (1100, 4)]:
        x_cpu = softmax_input(M, N, seed=N, dt="bf16")
        _say(f"bf16->f32 softmax, 8-byte aligned rows, {M}x{N}")
        ws_n = rr.rr_softmax_rows_workspace_bytes(M, N, rr.RR_BF16, rr.RR_F32)
        ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda") if ws_n else None
        ref = torch.empty(M, N, device="cuda")
        xa = x_cpu.cuda()
        if N % 8:
            # a 16-byte aligned copy of the rows (row stride a multiple of 8)
            _, xa = embed(x_cpu, N + (8 - N % 8), 0)
        rr.rr_softmax_rows_strided(ref, xa, None, ws)
        # the same rows 4 elements (8 bytes) into a wider buffer whose stride
        # is 8 bytes past a multiple of 16
        ld = N + 4 + (12 if (N + 4) % 8 == 0 else 8)
        assert (ld * 2) % 16 == 8 and ld >= N + 4
        buf, xv = embed(x_cpu, ld, 4)
        y = torch.empty(M, N, device="cuda")
        rr.rr_softmax_rows_strided(y, xv, None, ws)
        torch.cuda.synchronize()
        assert torch.equal(_bits(ref), _bits(y)), f"{M}x{N}"
        xf = compare.to_f64(x_cpu)
        compare.check_softmax(y.cpu(), xf, oracle.softmax(xf), f"8-byte rows {M}x{N}")
        untouched(buf, 4, N, "input")


# (M, N, ld, col, gamma_col): rows cut at aligned addresses.  x, y and the
# residual each sit in an [M, ld] buffer at column `col` (one offset within a
# vector for all three); gamma (beta) is aligned (gamma_col None) or a slice
# at gamma_col of a longer vector whose other elements are NaN: a cut row
# reads gamma's first and last aligned blocks whole, and those NaNs must not
# reach any output
CUT_NORM_CASES = [
    (66, 33, 33, 0, None),          # contiguous rows of an odd width: every lead
    (66, 33, 33, 0, 3),
    (7, 1021, 1021, 0, None),
    (66, 4097, 4097, 0, None),
    (66, 4097, 4097, 0, 5),
    (9, 4096, 4101, 3, None),       # a column slice: lead 3 on every row
    (9, 4096, 4101, 3, 3),          # gamma at the rows' offset
    (5, 16377, 16377, 0, None),     # the longest rows a workgroup holds at any lead
    (5, 16377, 16377, 0, 7),
    (3, 7661, 7661, 0, 5),          # the longest fp32 LayerNorm rows held (gamma and beta in LDS)
    (3, 7662, 7662, 0, None),
    (3, 15353, 15353, 0, 3),        # the longest bf16 LayerNorm rows held
    (2, 15354, 15354, 0, None),
    (3, 20001, 20001, 0, None),     # longer: bf16 RMSNorm rows held as 3 vectors per lane, else element by element
    (3, 24569, 24569, 0, 3),        # the longest bf16 RMSNorm rows held at any lead
    (2, 24577, 24577, 0, None),     # beyond every workgroup: element by element
]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("case", CUT_NORM_CASES, ids=lambda c: "x".join(map(str, c)))
def test_norm_rows_cut_at_aligned_addresses(case, dt):
    rr = _rr()
    M, N, ld, col, gcol = case
    code = rr.RR_F32 if dt == "f32" else rr.RR_BF16
    _say(f"cut norm rows {dt} {case}")
    for op in (rr.RR_OP_RMSNORM, rr.RR_OP_FUSED_ADD_RMSNORM, rr.RR_OP_LAYERNORM):
        p = rr.rr_query_plan(op, M, N, code, code, 2)
        # rows a workgroup holds at any lead: 16 wavefronts of up to 16
        # values per lane (24 for bf16: 3 vectors); a LayerNorm row while
        # its staged gamma and beta fit the LDS budget (60 KiB: bf16, 1920
        # aligned 16-byte blocks of each for a row at any lead; fp32, an
        # 8-byte entry per element plus 19 of padding)
        limit = 24569 if dt == "bf16" else 16377
        if op == rr.RR_OP_LAYERNORM:
            limit = 15353 if dt == "bf16" else 7661
        want = 32 < N <= limit
        assert p["row_shift"] == (1 if want else 0), (op, p)
    x_np = workloads.random_rows(M, N, seed=M + N + col)
    x_np[::3, 0] = 1.0e3                       # LayerNorm rows whose first element is far from the mean
    x_cpu = _as(x_np, dt)
    r_cpu = _as(workloads.random_rows(M, N, seed=2 * M + N), dt)
    g_cpu = _as(workloads.gamma_vector(N, seed=N), dt)
    b_cpu = _as(workloads.gamma_vector(N, seed=N + 1) - 1.0, dt)
    if gcol is None:
        gd, bd = g_cpu.cuda(), b_cpu.cuda()
    else:
        G = torch.full((N + gcol + 16,), float("nan"), dtype=_tdt(dt), device="cuda")
        Bt = torch.full((N + gcol + 16,), float("nan"), dtype=_tdt(dt), device="cuda")
        G[gcol:gcol + N] = g_cpu.cuda()
        Bt[gcol:gcol + N] = b_cpu.cuda()
        gd, bd = G[gcol:gcol + N], Bt[gcol:gcol + N]
    xbuf, xv = embed(x_cpu, ld, col)
    ybuf, yv = embed(torch.zeros(M, N, dtype=_tdt(dt)), ld, col)
    rr.rr_rmsnorm_strided(yv, xv, gd, 1e-6)
    torch.cuda.synchronize()
    check_norm(x_cpu, g_cpu, 1e-6, dt, yv.cpu(), f"cut rms {dt} {case}")
    untouched(ybuf, col, N, "cut rms y")
    for beta in (bd, None):
        rr.rr_layernorm_strided(yv, xv, gd, beta, 1e-5)
        torch.cuda.synchronize()
        bref = compare.to_f64(b_cpu) if beta is not None else np.zeros(N)
        ref = oracle.layernorm(compare.to_f64(x_cpu), compare.to_f64(g_cpu), bref, 1e-5)
        compare.check_layernorm(yv.cpu(), ref, compare.to_f64(g_cpu), bref,
                                f"cut layernorm {dt} {case} beta={beta is not None}")
        untouched(ybuf, col, N, "cut layernorm y")
    rbuf, rv = embed(r_cpu, ld, col)
    ybuf2, yv2 = embed(torch.zeros(M, N, dtype=_tdt(dt)), ld, col)
    rr.rr_fused_add_rmsnorm_strided(yv2, rv, xv, gd, 1e-6)
    torch.cuda.synchronize()
    check_fused(x_cpu, r_cpu, g_cpu, 1e-6, dt, yv2.cpu(), rv.cpu(), f"cut fused {dt} {case}")
    untouched(rbuf, col, N, "cut fused residual")
    untouched(ybuf2, col, N, "cut fused y")
    untouched(xbuf, col, N, "cut x")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_cut_rows_different_strides_and_in_place(dt):
    """Rows cut at aligned addresses with x and y in buffers of different
    strides (equal modulo the vector width, same column), and in place (y is
    x): the norms, the fused op writing y over x, and the softmax."""
    rr = _rr()
    code = rr.RR_F32 if dt == "f32" else rr.RR_BF16
    M, N, col = 9, 4093, 3
    ldx, ldy = N + 8, N + 24                      # both equal to N mod 8
    _say(f"cut rows, strides {ldx}/{ldy}, in place, {dt}")
    x_cpu = _as(workloads.random_rows(M, N, seed=N + 11), dt)
    r_cpu = _as(workloads.random_rows(M, N, seed=N + 12), dt)
    g_cpu = _as(workloads.gamma_vector(N, seed=N + 13), dt)
    assert rr.rr_query_plan(rr.RR_OP_RMSNORM, M, N, code, code, 2)["row_shift"] == 1
    xbuf, xv = embed(x_cpu, ldx, col)
    ybuf, yv = embed(torch.zeros(M, N, dtype=_tdt(dt)), ldy, col)
    rr.rr_rmsnorm_strided(yv, xv, g_cpu.cuda(), 1e-6)
    torch.cuda.synchronize()
    check_norm(x_cpu, g_cpu, 1e-6, dt, yv.cpu(), f"cut rms strides {dt}")
    untouched(ybuf, col, N, "cut rms y (other stride)")
    # in place: y is x
    ibuf, iv = embed(x_cpu, ldx, col)
    rr.rr_rmsnorm_strided(iv, iv, g_cpu.cuda(), 1e-6)
    torch.cuda.synchronize()
    check_norm(x_cpu, g_cpu, 1e-6, dt, iv.cpu(), f"cut rms in place {dt}")
    untouched(ibuf, col, N, "cut rms in place")
    # fused, y written over x, residual at a third stride
    fbuf, fv = embed(x_cpu, ldx, col)
    rbuf, rv = embed(r_cpu, N + 16, col)
    rr.rr_fused_add_rmsnorm_strided(fv, rv, fv, g_cpu.cuda(), 1e-6)
    torch.cuda.synchronize()
    check_fused(x_cpu, r_cpu, g_cpu, 1e-6, dt, fv.cpu(), rv.cpu(), f"cut fused in place {dt}")
    untouched(fbuf, col, N, "cut fused y/x")
    untouched(rbuf, col, N, "cut fused residual")
    # softmax in place on contiguous rows of an odd width
    s_cpu = softmax_input(M, N, seed=N + 14, dt=dt)
    sd = s_cpu.cuda()
    rr.rr_softmax_rows(sd, sd, None)
    torch.cuda.synchronize()
    xf = compare.to_f64(s_cpu)
    compare.check_softmax(sd.cpu(), xf, oracle.softmax(xf), f"cut softmax in place {dt}")


@pytest.mark.parametrize("dt,M,N", [("bf16", 6000, 4097), ("f32", 4095, 4097), ("bf16", 5000, 1025)])
def test_cut_layernorm_rows_walked_by_resident_workgroups(dt, M, N):
    """A workgroup's cut LayerNorm rows read gamma and beta staged in LDS once
    per workgroup, with no more workgroups than the device holds, each walking
    rows grid-stride: enough contiguous rows of an odd width (every row at its
    own lead) that each workgroup walks several, every third row's first
    element far from its mean, every row against the oracle."""
    rr = _rr()
    code = rr.RR_F32 if dt == "f32" else rr.RR_BF16
    p = rr.rr_query_plan(rr.RR_OP_LAYERNORM, M, N, code, code, 2)
    assert (p["variant_name"], p["row_shift"]) == ("block", 1), p
    _say(f"cut layernorm {dt} {M}x{N}, resident workgroups")
    x_np = workloads.random_rows(M, N, seed=M + N + 7)
    x_np[::3, 0] = 1.0e3
    x = _as(x_np, dt)
    g = _as(workloads.gamma_vector(N, seed=N + 5), dt)
    b = _as(workloads.gamma_vector(N, seed=N + 6) - 1.0, dt)
    y = torch.empty((M, N), dtype=_tdt(dt), device="cuda")
    rr.rr_layernorm(y, x.cuda(), g.cuda(), b.cuda(), 1e-5)
    torch.cuda.synchronize()
    gf, bf = compare.to_f64(g), compare.to_f64(b)
    ref = oracle.layernorm(compare.to_f64(x), gf, bf, 1e-5)
    compare.check_layernorm(y.cpu(), ref, gf, bf, f"cut layernorm {dt} {M}x{N}")
