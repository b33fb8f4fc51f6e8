"""Seeded random sweep on the GPU: shapes, dtypes, alignment, strides and
options drawn at random (fixed seed), every operation against the fp64
oracle.  It complements the hand-picked grids with cases nobody chose: odd
widths near every dispatch boundary, column offsets that break alignment, and
random option mixes.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests import compare
from tests.test_parity_gpu import _as, _rr, _say, _tdt, check_fused, check_norm, softmax_input

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

CASES = 48


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rr = _rr()
    rr.lib()
    yield


def _width(rng):
    # widths near the dispatch boundaries, and anywhere
    edges = [32, 64, 256, 1024, 2048, 4096, 16384, 32768, 65536, 81920, 163840]
    if rng.random() < 0.6:
        e = int(rng.choice(edges))
        return max(1, e + int(rng.integers(-9, 10)))
    return int(rng.integers(1, 200000))


def _rows(rng, N):
    budget = 1_500_000 // max(N, 1)
    return int(rng.integers(1, max(2, min(budget, 3000))))


def _slice(x_cpu, rng, pad_max=9):
    """x on the GPU as a column slice of a wider buffer (random left pad and
    row stride), or contiguous."""
    M, N = x_cpu.shape
    if rng.random() < 0.5:
        return x_cpu.cuda()
    pad = int(rng.integers(0, pad_max))
    ld = N + pad + int(rng.integers(0, pad_max))
    buf = torch.zeros((M, ld), dtype=x_cpu.dtype, device="cuda")
    buf[:, pad:pad + N] = x_cpu.cuda()
    return buf[:, pad:pad + N]


def _empty_like_slice(M, N, dt, rng):
    return _slice(torch.zeros((M, N), dtype=dt), rng)


@pytest.mark.parametrize("case", range(CASES))
def test_random_case(case):
    rr = _rr()
    rng = np.random.default_rng(1000 + case)
    N = _width(rng)
    M = _rows(rng, N)
    kind = ["rms", "fused", "layer", "softmax"][case % 4]
    dt = "bf16" if rng.random() < 0.5 else "f32"
    _say(f"random case {case}: {kind} {dt} {M}x{N}")
    if kind in ("rms", "fused", "layer"):
        x = _as(workloads.random_rows(M, N, seed=case, offset_every=5, offset=50.0), dt)
        g = _as(workloads.gamma_vector(N, seed=case), dt)
        xs = _slice(x, rng)
        ys = _empty_like_slice(M, N, _tdt(dt), rng)
        if kind == "rms":
            rr.rr_rmsnorm_strided(ys, xs, g.cuda(), 1e-6)
            torch.cuda.synchronize()
            check_norm(x, g, 1e-6, dt, ys.cpu(), f"random rms {case}")
        elif kind == "fused":
            r = _as(workloads.random_rows(M, N, seed=case + 1), dt)
            rs = _slice(r, rng)
            rr.rr_fused_add_rmsnorm_strided(ys, rs, xs, g.cuda(), 1e-6)
            torch.cuda.synchronize()
            check_fused(x, r, g, 1e-6, dt, ys.cpu(), rs.cpu(), f"random fused {case}")
        else:
            b = _as(workloads.gamma_vector(N, seed=case + 2) - 1.0, dt)
            rr.rr_layernorm_strided(ys, xs, g.cuda(), b.cuda(), 1e-5)
            torch.cuda.synchronize()
            gf, bf = compare.to_f64(g), compare.to_f64(b)
            ref = oracle.layernorm(compare.to_f64(x), gf, bf, 1e-5)
            compare.check_layernorm(ys.cpu(), ref, gf, bf, f"random ln {case}")
        return
    dout = "bf16" if rng.random() < 0.3 else "f32"
    x = softmax_input(M, N, seed=case, dt=dt)
    log_output = bool(rng.random() < 0.4)
    causal = bool(rng.random() < 0.4)
    xf = compare.to_f64(x)
    period = offset = None
    if causal:
        period = int(rng.integers(1, M + 1))
        offset = int(rng.integers(0, N + 2))
        keys = np.minimum(N, np.arange(M) % period + offset + 1)
        masked = np.arange(N)[None, :] >= keys[:, None]
        xf[masked] = -np.inf
        x = _as(np.where(masked, np.float32(np.nan), compare.to_f64(x)).astype(np.float32), dt)
    xs = _slice(x, rng)
    ys = _empty_like_slice(M, N, _tdt(dout), rng)
    opts = rr.make_softmax_opts(log_output=log_output, causal_period=period,
                                causal_offset=offset if causal else 0)
    n = rr.rr_softmax_rows_ex_workspace_bytes(M, N, rr.dtype_code(xs), rr.dtype_code(ys), opts)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda") if n else None
    rr.rr_softmax_rows_strided(ys, xs, opts, ws)
    torch.cuda.synchronize()
    what = f"random softmax {case} {dt}->{dout} log={log_output} causal={causal}"
    if log_output:
        compare.check_log_softmax(ys.cpu(), xf, oracle.log_softmax(xf), what)
    else:
        compare.check_softmax(ys.cpu(), xf, oracle.softmax(xf), what)


CUT_CASES = 40


@pytest.mark.parametrize("case", range(CUT_CASES))
def test_random_softmax_rows_cut_at_aligned_addresses(case):
    """Softmax calls whose rows are not whole aligned vectors but whose input
    and output rows share their offset within a vector: contiguous rows of a
    width off the vector grid (each row at a different offset), or column
    slices with the same left pad and the same stride (one offset), drawn at
    random with dtypes, log output and the causal rule.  Such rows are cut at
    aligned addresses (row_shift) whenever a held plan can hold them."""
    rr = _rr()
    rng = np.random.default_rng(5000 + case)
    N = _width(rng) | 1                  # odd: never a whole number of vectors
    M = _rows(rng, N)
    din = "bf16" if rng.random() < 0.5 else "f32"
    dout = "bf16" if rng.random() < 0.3 else "f32"
    log_output = bool(rng.random() < 0.4)
    causal = bool(rng.random() < 0.4)
    x = softmax_input(M, N, seed=case + 77, dt=din)
    xf = compare.to_f64(x)
    period = offset = None
    if causal:
        period = int(rng.integers(1, M + 1))
        offset = int(rng.integers(0, N + 2))
        keys = np.minimum(N, np.arange(M) % period + offset + 1)
        masked = np.arange(N)[None, :] >= keys[:, None]
        xf[masked] = -np.inf
        x = _as(np.where(masked, np.float32(np.nan), compare.to_f64(x)).astype(np.float32), din)
    if rng.random() < 0.5:
        xs = x.cuda()
        ys = torch.empty((M, N), dtype=_tdt(dout), device="cuda")
    else:
        pad = int(rng.integers(1, 9))
        ld = N + pad + int(rng.integers(0, 9))
        X = torch.zeros((M, ld), dtype=x.dtype, device="cuda")
        X[:, pad:pad + N] = x.cuda()
        Y = torch.zeros((M, ld), dtype=_tdt(dout), device="cuda")
        xs, ys = X[:, pad:pad + N], Y[:, pad:pad + N]
    op = rr.RR_OP_SOFTMAX_CAUSAL if causal else rr.RR_OP_SOFTMAX
    plan = rr.rr_query_plan(op, M, N, rr.dtype_code(xs), rr.dtype_code(ys), 2)
    _say(f"random cut-row softmax {case}: {din}->{dout} {M}x{N} log={log_output} causal={causal} "
         f"plan={plan['variant_name']} shift={plan['row_shift']}")
    if plan["variant_name"] in ("wave", "block", "split"):
        assert plan["row_shift"] == 1, plan
    opts = rr.make_softmax_opts(log_output=log_output, causal_period=period,
                                causal_offset=offset if causal else 0)
    n = rr.rr_softmax_rows_ex_workspace_bytes(M, N, rr.dtype_code(xs), rr.dtype_code(ys), opts)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda") if n else None
    rr.rr_softmax_rows_strided(ys, xs, opts, ws)
    torch.cuda.synchronize()
    what = f"random cut-row softmax {case} {din}->{dout} log={log_output} causal={causal}"
    if log_output:
        compare.check_log_softmax(ys.cpu(), xf, oracle.log_softmax(xf), what)
    else:
        compare.check_softmax(ys.cpu(), xf, oracle.softmax(xf), what)


NORM_CUT_CASES = 36


@pytest.mark.parametrize("case", range(NORM_CUT_CASES))
def test_random_norm_rows_cut_at_aligned_addresses(case):
    """RMSNorm, fused add + RMSNorm and LayerNorm (with and without beta) on
    rows cut at aligned addresses, drawn at random: widths off the vector
    grid up to past the register kernels' reach, contiguous rows (every row
    at its own offset) or column slices of one offset, gamma (beta) aligned or
    a slice at any offset of a longer vector whose other elements are NaN,
    and rows whose first element lies far from their mean."""
    rr = _rr()
    rng = np.random.default_rng(7000 + case)
    N = int(rng.integers(33, 20000)) | 1
    M = _rows(rng, N)
    dt = "bf16" if rng.random() < 0.5 else "f32"
    kind = ["rms", "fused", "layer", "layer_nobeta"][case % 4]
    x = workloads.random_rows(M, N, seed=case + 11, offset_every=4, offset=30.0)
    if kind.startswith("layer"):
        x[::3, 0] = 1.0e3                 # first element far from the row's mean
    x = _as(x, dt)
    g = _as(workloads.gamma_vector(N, seed=case + 12), dt)
    b = _as(workloads.gamma_vector(N, seed=case + 13) - 1.0, dt)

    def param(v):
        if rng.random() < 0.5:
            return v.cuda()
        off = int(rng.integers(1, 16))
        buf = torch.full((N + off + 16,), float("nan"), dtype=v.dtype, device="cuda")
        buf[off:off + N] = v.cuda()
        return buf[off:off + N]

    contiguous = rng.random() < 0.5
    pad = 0 if contiguous else int(rng.integers(1, 9))
    ld = N if contiguous else N + pad + 8 * int(rng.integers(0, 3))

    def embed(t):
        if contiguous:
            return t.cuda(), None
        buf = torch.zeros((M, ld), dtype=t.dtype, device="cuda")
        buf[:, pad:pad + N] = t.cuda()
        return buf[:, pad:pad + N], buf

    op = {"rms": rr.RR_OP_RMSNORM, "fused": rr.RR_OP_FUSED_ADD_RMSNORM}.get(kind, rr.RR_OP_LAYERNORM)
    code = rr.RR_F32 if dt == "f32" else rr.RR_BF16
    plan = rr.rr_query_plan(op, M, N, code, code, 2)
    _say(f"random cut-row norm {case}: {kind} {dt} {M}x{N} contiguous={contiguous} pad={pad} "
         f"plan={plan['variant_name']} shift={plan['row_shift']} nv={plan['vecs_per_lane']}")
    xs, _ = embed(x)
    ys, ybuf = embed(torch.zeros((M, N), dtype=_tdt(dt)))
    gd = param(g)
    what = f"random cut-row norm {case} {kind} {dt} {M}x{N}"
    if kind == "rms":
        rr.rr_rmsnorm_strided(ys, xs, gd, 1e-6)
        torch.cuda.synchronize()
        check_norm(x, g, 1e-6, dt, ys.cpu(), what)
    elif kind == "fused":
        r = _as(workloads.random_rows(M, N, seed=case + 14), dt)
        rs, _ = embed(r)
        rr.rr_fused_add_rmsnorm_strided(ys, rs, xs, gd, 1e-6)
        torch.cuda.synchronize()
        check_fused(x, r, g, 1e-6, dt, ys.cpu(), rs.cpu(), what)
    else:
        with_beta = kind == "layer"
        bd = param(b) if with_beta else None
        rr.rr_layernorm_strided(ys, xs, gd, bd, 1e-5)
        torch.cuda.synchronize()
        gf = compare.to_f64(g)
        bf = compare.to_f64(b) if with_beta else np.zeros(N)
        ref = oracle.layernorm(compare.to_f64(x), gf, bf, 1e-5)
        compare.check_layernorm(ys.cpu(), ref, gf, bf, what)
    if ybuf is not None:
        # nothing outside the slice is written
        outside = torch.cat([ybuf[:, :pad], ybuf[:, pad + N:]], dim=1)
        assert not outside.any(), f"{what}: writes outside the slice"
