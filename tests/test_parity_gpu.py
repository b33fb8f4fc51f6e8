"""GPU parity: the HIP kernels (through the C ABI) against the fp64 oracle.

Inputs come from ``workloads`` (seeded, shared by both sides); expected values
come only from ``oracle``.  Bars are in tests/compare.py.  Shapes straddle
every dispatch boundary (a wavefront per row up to 1024/2048 elements, a
workgroup per row up to 16384/32768, split and streaming beyond), with ragged
tails, partial workgroups (M = 7), unaligned rows, masked and fully masked
rows, +1000 offsets and spikes, each variant forced on shapes it supports,
the named workloads at full size, and run-to-run bitwise determinism.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests import compare

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import row_reduction_rmsnorm_amd as rr
    rr.lib()
    yield


def _rr():
    import row_reduction_rmsnorm_amd as rr
    return rr


def _say(*a):
    print(*a, flush=True)


def _tdt(name):
    return torch.float32 if name == "f32" else torch.bfloat16


def _as(x32: np.ndarray, dt: str):
    return workloads.to_dtype(x32, dt)


# ----------------------------------------------------------------------------
# runners
# ----------------------------------------------------------------------------

def run_rmsnorm(x_cpu, g_cpu, eps, inplace=False):
    rr = _rr()
    x = x_cpu.cuda()
    g = g_cpu.cuda()
    y = x if inplace else torch.empty_like(x)
    rr.rr_rmsnorm(y, x, g, eps)
    torch.cuda.synchronize()
    return y.cpu()


def run_fused(x_cpu, r_cpu, g_cpu, eps, y_is_x=False):
    rr = _rr()
    x = x_cpu.cuda()
    r = r_cpu.cuda()
    g = g_cpu.cuda()
    y = x if y_is_x else torch.empty_like(x)
    rr.rr_fused_add_rmsnorm(y, r, x, g, eps)
    torch.cuda.synchronize()
    return y.cpu(), r.cpu()


def run_softmax(x_cpu, out_dt, inplace=False):
    rr = _rr()
    x = x_cpu.cuda()
    y = x if inplace else torch.empty(x.shape, dtype=out_dt, device=x.device)
    ws = rr.softmax_workspace(x, out_dt)
    rr.rr_softmax_rows(y, x, ws)
    torch.cuda.synchronize()
    return y.cpu()


def check_norm(x_cpu, g_cpu, eps, dt, y_cpu, what):
    ref = oracle.rmsnorm(compare.to_f64(x_cpu), compare.to_f64(g_cpu), eps)
    if dt == "bf16":
        return compare.check_bf16(y_cpu, ref, what)
    return compare.check_rms_f32(y_cpu, ref, what)


def check_fused(x_cpu, r_cpu, g_cpu, eps, dt, y_cpu, r_out_cpu, what):
    h_ref, y_ref = oracle.fused_add_rmsnorm(compare.to_f64(x_cpu), compare.to_f64(r_cpu),
                                            compare.to_f64(g_cpu), eps, dt)
    # the new residual is the correctly rounded sum: bit-exact
    if dt == "bf16":
        compare.check_bf16_exact(r_out_cpu, h_ref, what + " residual")
        return compare.check_bf16(y_cpu, y_ref, what + " y")
    assert np.array_equal(compare.to_f64(r_out_cpu), h_ref), what + " residual"
    return compare.check_rms_f32(y_cpu, y_ref, what + " y")


def check_softmax(x_cpu, y_cpu, what):
    xf = compare.to_f64(x_cpu)
    ref = oracle.softmax(xf)
    return compare.check_softmax(y_cpu, xf.reshape(ref.shape), ref, what)


def softmax_input(M, N, seed, dt):
    """N(0, 8) rows; every third row +1000; rows with 30% masked entries;
    row 2 fully masked (when it exists) and one spike per row."""
    x = workloads.random_rows(M, N, seed, scale=8.0, offset_every=3, offset=1000.0)
    rng = np.random.default_rng(seed + 1)
    if M > 1 and N > 1:
        mask = rng.random((M, N)) < 0.3
        mask[:, 0] = False
        mask[::2] = False
        x[mask] = -np.inf
    if N > 4:
        cols = rng.integers(0, N, M)
        x[np.arange(M), cols] = rng.uniform(20, 30, M).astype(np.float32)
    if M > 2:
        x[2, :] = -np.inf
    return _as(x, dt)


# ----------------------------------------------------------------------------
# the wave64 all-reduce primitive
# ----------------------------------------------------------------------------

def test_wave_allreduce_lane_ids_spikes_and_bitwise_equal_lanes():
    rr = _rr()
    groups = []
    groups.append(np.arange(64, dtype=np.float32))                 # lane ids
    for k in range(64):                                            # a spike in each lane
        g = np.zeros(64, np.float32)
        g[k] = 1.0
        groups.append(g)
    groups.append(np.ones(64, np.float32))                         # 64 lanes x 1 -> 64
    rng = np.random.default_rng(5)
    for _ in range(32):
        groups.append(rng.standard_normal(64).astype(np.float32) * 100)
    inp = torch.from_numpy(np.concatenate(groups)).cuda()
    out = torch.empty_like(inp)
    rr.rr_selftest_wave_allreduce(out, inp, 0)
    s = out.cpu().numpy().reshape(-1, 64)
    assert np.all(s == s[:, :1]), "lanes differ after the sum all-reduce"
    ref = np.array([np.sum(g.astype(np.float64)) for g in groups])
    assert s[0, 0] == 2016.0 and np.all(s[1:65, 0] == 1.0) and s[65, 0] == 64.0
    assert np.allclose(s[:, 0], ref, rtol=1e-5, atol=1e-2)
    rr.rr_selftest_wave_allreduce(out, inp, 1)
    mx = out.cpu().numpy().reshape(-1, 64)
    assert np.all(mx == mx[:, :1])
    assert np.array_equal(mx[:, 0], np.array([g.max() for g in groups]))


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (64 << 20) + 16, (1 << 30) + 32])
def test_stream_copy_bytes(nbytes):
    """The measurement copy moves every byte (both launch shapes: 1024-lane
    groups below 1 GiB, 256-lane groups from 1 GiB) and nothing past the end."""
    rr = _rr()
    _say("stream copy", nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda")
    dst = torch.full((nbytes + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    rr.rr_stream_copy(dst[:nbytes], src)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert bool((dst[nbytes:] == 0xA5).all())


def test_wave_allreduce_md_pairs():
    from oracle import online_ref
    rr = _rr()
    rng = np.random.default_rng(6)
    cases = []
    for _ in range(40):
        m = (rng.standard_normal(64) * 10).astype(np.float32)
        d = rng.uniform(1, 3, 64).astype(np.float32)
        cases.append((m, d))
    m = np.full(64, -np.inf, np.float32)
    cases.append((m, np.zeros(64, np.float32)))                    # all identity
    m = (rng.standard_normal(64) * 5).astype(np.float32)
    d = np.ones(64, np.float32)
    m[::3] = -np.inf
    d[::3] = 0.0
    cases.append((m, d))                                           # mixed identity
    for k in (0, 17, 63):                                          # one finite lane
        m = np.full(64, -np.inf, np.float32)
        d = np.zeros(64, np.float32)
        m[k], d[k] = 1000.0, 2.0
        cases.append((m, d))
    inp = torch.from_numpy(np.concatenate([np.concatenate(c) for c in cases])).cuda()
    out = torch.empty_like(inp)
    rr.rr_selftest_wave_allreduce(out, inp, 2)
    res = out.cpu().numpy().reshape(-1, 2, 64)
    for i, (m, d) in enumerate(cases):
        gm, gd = res[i, 0], res[i, 1]
        assert np.all(gm == gm[0]) and np.all(gd == gd[0]), f"case {i}: lanes differ"
        acc = online_ref.IDENTITY
        for a, b in zip(m.astype(float), d.astype(float)):
            acc = online_ref.merge(acc, (a, b))
        assert gm[0] == np.float32(acc[0])
        if acc[0] == -np.inf:
            assert gd[0] == 0.0
        else:
            assert abs(gd[0] - acc[1]) <= 1e-5 * acc[1], (i, gd[0], acc)


# ----------------------------------------------------------------------------
# RMSNorm and fused add + RMSNorm over the shape grid
# ----------------------------------------------------------------------------

NORM_N = [1, 7, 64, 65, 1000, 1024, 1028, 2048, 3584, 4096, 8191, 16384, 16392]
NORM_M = [1, 7, 64]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("N", NORM_N)
def test_rmsnorm_grid(dt, N):
    for M in NORM_M:
        _say(f"rmsnorm {dt} M={M} N={N}")
        x = _as(workloads.random_rows(M, N, seed=N + M, scale=2.0), dt)
        g = _as(workloads.gamma_vector(N, seed=N), dt)
        y = run_rmsnorm(x, g, 1e-6)
        check_norm(x, g, 1e-6, dt, y, f"rmsnorm {dt} {M}x{N}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("N", NORM_N)
def test_fused_grid(dt, N):
    for M in NORM_M:
        _say(f"fused {dt} M={M} N={N}")
        x = _as(workloads.random_rows(M, N, seed=N + M), dt)
        r = _as(workloads.random_rows(M, N, seed=N + M + 100, scale=3.0), dt)
        g = _as(workloads.gamma_vector(N, seed=N + 1), dt)
        y, r_out = run_fused(x, r, g, 1e-6)
        check_fused(x, r, g, 1e-6, dt, y, r_out, f"fused {dt} {M}x{N}")


def test_norm_edge_cases():
    rr = _rr()
    # zero rows, constant rows, huge and tiny magnitudes, eps = 0
    for dt in ("f32", "bf16"):
        M, N = 6, 4096
        x = workloads.random_rows(M, N, seed=1)
        x[0] = 0.0                       # all-zero row with eps > 0 -> y = 0
        x[1] = 3.0                       # constant row
        x[2] *= 1e15                     # large magnitudes (sum of squares ~4e33, inside fp32)
        x[3] *= 1e-15                    # small magnitudes (squares well above fp32 subnormals)
        xt, g = _as(x, dt), _as(workloads.gamma_vector(N, 2), dt)
        check_norm(xt, g, 1e-6, dt, run_rmsnorm(xt, g, 1e-6), f"edge {dt}")
        x[0] = 1.0
        xt = _as(x, dt)
        check_norm(xt, g, 0.0, dt, run_rmsnorm(xt, g, 0.0), f"edge eps0 {dt}")
    # M = 0 leaves the output untouched
    y = torch.full((0, 64), 7.0, device="cuda")
    rr.rr_rmsnorm(y, torch.empty((0, 64), device="cuda"), torch.ones(64, device="cuda"), 1e-6)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_norm_in_place_and_unaligned(dt):
    rr = _rr()
    M, N = 9, 4096
    x = _as(workloads.random_rows(M, N, seed=3), dt)
    g = _as(workloads.gamma_vector(N, 4), dt)
    check_norm(x, g, 1e-6, dt, run_rmsnorm(x, g, 1e-6, inplace=True), "in place")
    r = _as(workloads.random_rows(M, N, seed=5), dt)
    y, r_out = run_fused(x, r, g, 1e-6, y_is_x=True)
    check_fused(x, r, g, 1e-6, dt, y, r_out, "fused y is x")
    # unaligned rows: views one element into a buffer
    base = torch.empty(M * N + 1, dtype=_tdt(dt), device="cuda")
    xv = base[1:].view(M, N)
    xv.copy_(x.cuda())
    y = torch.empty(M * N + 1, dtype=_tdt(dt), device="cuda")[1:].view(M, N)
    plan = rr.rr_query_plan(rr.RR_OP_RMSNORM, M, N, rr.dtype_code(xv), rr.dtype_code(xv), False)
    assert plan["variant_name"] == "loop" and plan["vec_elems"] == 1
    rr.rr_rmsnorm(y, xv, g.cuda(), 1e-6)
    torch.cuda.synchronize()
    check_norm(x, g, 1e-6, dt, y.cpu(), "unaligned")


@pytest.mark.parametrize("variant", ["wave", "block", "loop", "subwave"])
def test_norm_forced_variants(variant):
    rr = _rr()
    code = {"wave": rr.RR_VARIANT_WAVE, "block": rr.RR_VARIANT_BLOCK, "loop": rr.RR_VARIANT_LOOP,
            "subwave": rr.RR_VARIANT_SUBWAVE}[variant]
    shapes = {"wave": [8, 64, 520, 1024], "block": [8, 1024, 3584, 4096, 16384],
              "loop": [8, 1024, 4096, 20000, 65536], "subwave": [8, 16, 24, 64, 128]}[variant]
    with rr.forced_variant(code):
        for dt in ("f32", "bf16"):
            for N in shapes:
                for M in (1, 7, 130):
                    _say(f"norm forced {variant} {dt} M={M} N={N}")
                    x = _as(workloads.random_rows(M, N, seed=M * 7 + N), dt)
                    g = _as(workloads.gamma_vector(N, seed=N), dt)
                    check_norm(x, g, 1e-6, dt, run_rmsnorm(x, g, 1e-6), f"{variant} {dt} {M}x{N}")
                    r = _as(workloads.random_rows(M, N, seed=M + N), dt)
                    y, r_out = run_fused(x, r, g, 1e-6)
                    check_fused(x, r, g, 1e-6, dt, y, r_out, f"{variant} fused {dt} {M}x{N}")


# ----------------------------------------------------------------------------
# LayerNorm (f3)
# ----------------------------------------------------------------------------

def run_layernorm(x_cpu, g_cpu, b_cpu, eps, inplace=False):
    rr = _rr()
    x = x_cpu.cuda()
    y = x if inplace else torch.empty_like(x)
    rr.rr_layernorm(y, x, g_cpu.cuda(), None if b_cpu is None else b_cpu.cuda(), eps)
    torch.cuda.synchronize()
    return y.cpu()


def check_ln(x_cpu, g_cpu, b_cpu, eps, y_cpu, what):
    gf = compare.to_f64(g_cpu)
    bf = None if b_cpu is None else compare.to_f64(b_cpu)
    ref = oracle.layernorm(compare.to_f64(x_cpu), gf, bf, eps)
    return compare.check_layernorm(y_cpu, ref, gf, bf, what)


def ln_input(M, N, seed, dt, offset=0.0, spread=1.0):
    rng = np.random.default_rng(seed)
    x = (offset + spread * rng.standard_normal((M, N))).astype(np.float32)
    g = rng.uniform(0.5, 1.5, N).astype(np.float32)
    b = rng.uniform(-1.0, 1.0, N).astype(np.float32)
    return _as(x, dt), _as(g, dt), _as(b, dt)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("N", [1, 2, 7, 64, 65, 1000, 1024, 1028, 3584, 5120, 8191, 16384, 16392, 40000])
def test_layernorm_grid(dt, N):
    for M in (1, 7, 64):
        for (offset, spread) in ((0.0, 1.0), (101.0, 0.6)):
            _say(f"layernorm {dt} M={M} N={N} offset={offset}")
            x, g, b = ln_input(M, N, seed=N + M, dt=dt, offset=offset, spread=spread)
            check_ln(x, g, b, 1e-5, run_layernorm(x, g, b, 1e-5), f"ln {dt} {M}x{N} +{offset}")
        x, g, _ = ln_input(M, N, seed=N + M + 1, dt=dt)
        check_ln(x, g, None, 1e-5, run_layernorm(x, g, None, 1e-5), f"ln no beta {dt} {M}x{N}")


PACKED_NORM_N = {"f32": [16388, 20480, 32768, 40000, 65536, 65540],
                 "bf16": [16392, 20480, 32768, 40000, 65536, 65544]}


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_norms_packed_long_rows(dt):
    """Rows past the register budget of the workgroup-per-row norm kernel,
    held packed by 1024 lanes up to 64K elements (the last width of each list
    streams instead): RMSNorm, fused add + RMSNorm (including the fp32 fused
    limit at 32K) and LayerNorm with a large offset, including in place."""
    rr = _rr()
    code = rr.RR_F32 if dt == "f32" else rr.RR_BF16
    for N in PACKED_NORM_N[dt]:
        for M in (1, 7, 33):
            plans = {op: rr.rr_query_plan(op, M, N, code, code)
                     for op in (rr.RR_OP_RMSNORM, rr.RR_OP_FUSED_ADD_RMSNORM, rr.RR_OP_LAYERNORM)}
            _say(f"packed norms {dt} M={M} N={N} " +
                 " ".join(f"{p['variant_name']}/{p['vecs_per_lane']}" for p in plans.values()))
            x = _as(workloads.random_rows(M, N, seed=N + M), dt)
            g = _as(workloads.gamma_vector(N, seed=N), dt)
            check_norm(x, g, 1e-6, dt, run_rmsnorm(x, g, 1e-6, inplace=(M == 7)), f"rms {dt} {M}x{N}")
            r = _as(workloads.random_rows(M, N, seed=N + M + 1), dt)
            yf, rf = run_fused(x, r, g, 1e-6, y_is_x=(M == 7))
            check_fused(x, r, g, 1e-6, dt, yf, rf, f"fused {dt} {M}x{N}")
            xl, gl, bl = ln_input(M, N, seed=N + 2 * M, dt=dt, offset=101.0, spread=0.6)
            check_ln(xl, gl, bl, 1e-5, run_layernorm(xl, gl, bl, 1e-5), f"ln {dt} {M}x{N}")
            check_ln(xl, gl, None, 1e-5, run_layernorm(xl, gl, None, 1e-5, inplace=True), f"ln nb {dt} {M}x{N}")


@pytest.mark.parametrize("variant", ["wave", "block", "loop", "subwave"])
def test_layernorm_forced_variants(variant):
    rr = _rr()
    code = {"wave": rr.RR_VARIANT_WAVE, "block": rr.RR_VARIANT_BLOCK, "loop": rr.RR_VARIANT_LOOP,
            "subwave": rr.RR_VARIANT_SUBWAVE}[variant]
    shapes = {"wave": [8, 64, 520, 1024], "block": [8, 1024, 5120, 16384],
              "loop": [8, 1024, 5120, 20000], "subwave": [8, 24, 64, 128]}[variant]
    with rr.forced_variant(code):
        for dt in ("f32", "bf16"):
            for N in shapes:
                for M in (1, 7, 130):
                    x, g, b = ln_input(M, N, seed=3 * N + M, dt=dt, offset=50.0, spread=2.0)
                    check_ln(x, g, b, 1e-5, run_layernorm(x, g, b, 1e-5), f"{variant} ln {dt} {M}x{N}")


def test_layernorm_edge_cases():
    # constant rows give beta (x - mean = 0 exactly when the sum is about the first element)
    x = np.full((5, 4096), 101.25, np.float32)
    g = workloads.gamma_vector(4096, 1)
    b = np.linspace(-1, 1, 4096).astype(np.float32)
    y = run_layernorm(_as(x, "f32"), _as(g, "f32"), _as(b, "f32"), 1e-5)
    assert np.array_equal(y.numpy(), np.broadcast_to(b, (5, 4096)))
    # in place, and unaligned rows
    xt, gt, bt = ln_input(9, 4096, seed=8, dt="f32", offset=3.0)
    check_ln(xt, gt, bt, 1e-5, run_layernorm(xt, gt, bt, 1e-5, inplace=True), "ln in place")
    rr = _rr()
    base = torch.empty(9 * 4096 + 1, device="cuda")
    xv = base[1:].view(9, 4096)
    xv.copy_(xt.cuda())
    yv = torch.empty(9 * 4096 + 1, device="cuda")[1:].view(9, 4096)
    rr.rr_layernorm(yv, xv, gt.cuda(), bt.cuda(), 1e-5)
    torch.cuda.synchronize()
    check_ln(xt, gt, bt, 1e-5, yv.cpu(), "ln unaligned")



@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("N", [96, 1024, 4096, 20480, 70000])
def test_layernorm_first_element_far_from_the_mean(dt, N):
    """LayerNorm sums about a row's first element.  When that element lies far
    from the row's mean, the one-reduction variance would cancel and every
    x - K would be rounded at the scale of the distance, so the kernels sum
    again about the mean.  Rows here put the first element at various
    distances (some rows take that second sum, some do not), on the
    short-row, wavefront, workgroup, packed and streaming paths."""
    _say(f"layernorm far first element {dt} N={N}")
    rng = np.random.default_rng(N)
    x = rng.standard_normal((8, N)).astype(np.float32)
    x[:, 0] = np.array([50.0, -300.0, 1.0e4, 7.0, -7.0, 0.5, 2.5, -3.0], np.float32)
    x[7, 1:] += 1.0e3                      # mean far from zero as well
    g = rng.uniform(0.5, 1.5, N).astype(np.float32)
    b = rng.uniform(-1.0, 1.0, N).astype(np.float32)
    xt, gt, bt = _as(x, dt), _as(g, dt), _as(b, dt)
    check_ln(xt, gt, bt, 1e-5, run_layernorm(xt, gt, bt, 1e-5), f"ln far first {dt} N={N}")


def test_workload_layernorm_full():
    """The LayerNorm exercise's shape: 256 x 5120, x ~ U(100, 102)."""
    w = workloads.make("layernorm")
    _say(w.description)
    y = run_layernorm(w.arrays["x"], w.arrays["gamma"], w.arrays["beta"], w.eps)
    _say(check_ln(w.arrays["x"], w.arrays["gamma"], w.arrays["beta"], w.eps, y, w.name))


# ----------------------------------------------------------------------------
# softmax over the shape grid
# ----------------------------------------------------------------------------

SOFTMAX_N = [1, 7, 63, 64, 65, 1000, 1023, 1024, 1025, 2047, 2048, 2049, 2056, 3584, 4096,
             8191, 16384, 16385, 32768, 50000, 152064]
DTYPES = [("f32", "f32"), ("bf16", "f32"), ("f32", "bf16"), ("bf16", "bf16")]


@pytest.mark.parametrize("din,dout", DTYPES)
@pytest.mark.parametrize("N", SOFTMAX_N)
def test_softmax_grid(din, dout, N):
    for M in ([1, 7, 64] if N < 50000 else [1, 7, 40]):
        _say(f"softmax {din}->{dout} M={M} N={N}")
        x = softmax_input(M, N, seed=N + 3 * M, dt=din)
        y = run_softmax(x, _tdt(dout))
        check_softmax(x, y, f"softmax {din}->{dout} {M}x{N}")


def test_short_rows_unaligned_and_partial_groups():
    """Short rows (several per wavefront), including unaligned widths (scalar
    lanes), row counts that leave a partial group, and fully masked rows."""
    for N in (1, 2, 3, 5, 7, 17, 31, 32):
        for M in (1, 3, 255, 257, 1000):
            for dt in ("f32", "bf16"):
                x = softmax_input(M, N, seed=N * 1000 + M, dt=dt)
                check_softmax(x, run_softmax(x, _tdt(dt)), f"short softmax {dt} {M}x{N}")
                xn = _as(workloads.random_rows(M, N, seed=N + M), dt)
                g = _as(workloads.gamma_vector(N, seed=N), dt)
                check_norm(xn, g, 1e-6, dt, run_rmsnorm(xn, g, 1e-6), f"short rms {dt} {M}x{N}")
                r = _as(workloads.random_rows(M, N, seed=N + M + 1), dt)
                yf, rf = run_fused(xn, r, g, 1e-6)
                check_fused(xn, r, g, 1e-6, dt, yf, rf, f"short fused {dt} {M}x{N}")


def test_softmax_many_rows_and_partial_groups():
    for (M, N) in [(257, 1024), (1023, 33000), (1024, 33000), (4097, 64)]:
        _say(f"softmax rows M={M} N={N}")
        x = softmax_input(M, N, seed=M, dt="f32")
        check_softmax(x, run_softmax(x, torch.float32), f"{M}x{N}")


@pytest.mark.parametrize("variant", ["wave", "block", "split", "split1", "split2", "loop", "subwave"])
def test_softmax_forced_variants(variant):
    rr = _rr()
    code = {"wave": rr.RR_VARIANT_WAVE, "block": rr.RR_VARIANT_BLOCK,
            "split": rr.RR_VARIANT_SPLIT, "split1": rr.RR_VARIANT_SPLIT_ONE_KERNEL,
            "split2": rr.RR_VARIANT_SPLIT_TWO_KERNELS,
            "loop": rr.RR_VARIANT_LOOP, "subwave": rr.RR_VARIANT_SUBWAVE}[variant]
    shapes = {"wave": [8, 64, 1024, 2048], "block": [8, 1024, 4096, 16384, 32768, 65536],
              "split": [8, 1024, 4096, 4104, 65536], "split1": [8, 4104, 65536], "split2": [8, 4104, 65536],
              "loop": [8, 1024, 4096, 100000], "subwave": [8, 16, 40, 64, 128]}[variant]
    with rr.forced_variant(code):
        for din, dout in DTYPES:
            for N in shapes:
                if variant == "wave" and din == "bf16" and N > 2048:
                    continue
                for M in (1, 7, 33):
                    _say(f"softmax forced {variant} {din}->{dout} M={M} N={N}")
                    x = softmax_input(M, N, seed=M + N, dt=din)
                    y = run_softmax(x, _tdt(dout))
                    check_softmax(x, y, f"{variant} {din}->{dout} {M}x{N}")


def test_split_one_kernel_equals_two_kernels_bitwise():
    """The one-kernel split and the two-kernel split use the same chunks and
    merge order: identical bits, on the vocabulary workload's first rows and
    on shapes whose chunks the device cannot hold at once (there the request
    runs the two kernels)."""
    rr = _rr()
    cases = [workloads.make("sm_vocab", rows=64).arrays["x"],
             softmax_input(1023, 33000, seed=4, dt="f32"),
             softmax_input(700, 131072, seed=5, dt="bf16")]
    for x in cases:
        outs = []
        for code in (rr.RR_VARIANT_SPLIT_ONE_KERNEL, rr.RR_VARIANT_SPLIT_TWO_KERNELS, rr.RR_VARIANT_SPLIT):
            with rr.forced_variant(code):
                outs.append(run_softmax(x, torch.float32))
        assert torch.equal(_bits(outs[0]), _bits(outs[1])), tuple(x.shape)
        assert torch.equal(_bits(outs[2]), _bits(outs[1])), tuple(x.shape)
        check_softmax(x, outs[0], f"split {tuple(x.shape)}")


def test_split_one_kernel_on_a_reused_workspace():
    """The one-kernel split takes only slots its own call wrote: one workspace
    serves call after call of both forms on different inputs, each input's
    first call being a one-kernel call that finds the slots of the previous
    input's one-kernel call (other values, the previous epoch's tag), and
    every one-kernel call must equal the two-kernel call on the same input
    bit for bit."""
    rr = _rr()
    M, N = 48, 152064
    for din, dout in (("bf16", "bf16"), ("bf16", "f32"), ("f32", "f32")):
        odt = _tdt(dout)
        nb = rr.rr_softmax_rows_workspace_bytes(M, N, rr.RR_F32 if din == "f32" else rr.RR_BF16,
                                                rr.RR_F32 if dout == "f32" else rr.RR_BF16)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        for k in range(4):
            _say(f"reused workspace {din}->{dout} call {k}")
            x = softmax_input(M, N, seed=200 + k, dt=din).cuda()
            outs = []
            for code in (rr.RR_VARIANT_SPLIT_ONE_KERNEL, rr.RR_VARIANT_SPLIT_TWO_KERNELS, rr.RR_VARIANT_SPLIT):
                with rr.forced_variant(code):
                    y = torch.full((M, N), 3.0, dtype=odt, device="cuda")
                    rr.rr_softmax_rows(y, x, ws)
                    torch.cuda.synchronize()
                    outs.append(y)
            assert torch.equal(_bits(outs[1]), _bits(outs[0])), (din, dout, k)
            assert torch.equal(_bits(outs[1]), _bits(outs[2])), (din, dout, k)
            if k == 0:
                check_softmax(x.cpu(), outs[0].cpu(), f"one-kernel split {din}->{dout} {M}x{N}")


def test_split_one_kernel_on_zeroed_and_filled_workspaces():
    """The one-kernel split's tags come from per-row epochs kept in the
    workspace: a workspace of zeros (epoch 0, every slot word 0) or of 0xff
    bytes must not look like published pairs, and twelve calls in a row on
    one workspace, the input changing every time, must each equal the
    two-kernel split on the same input bit for bit."""
    rr = _rr()
    M, N = 16, 152064
    nb = rr.rr_softmax_rows_workspace_bytes(M, N, rr.RR_BF16, rr.RR_F32)
    for fill in (0x00, 0xff):
        ws = torch.full((nb,), fill, dtype=torch.uint8, device="cuda")
        x = softmax_input(M, N, seed=300 + fill, dt="bf16").cuda()
        outs = []
        for code in (rr.RR_VARIANT_SPLIT_ONE_KERNEL, rr.RR_VARIANT_SPLIT_TWO_KERNELS):
            with rr.forced_variant(code):
                y = torch.full((M, N), 3.0, dtype=torch.float32, device="cuda")
                rr.rr_softmax_rows(y, x, ws)
                torch.cuda.synchronize()
                outs.append(y)
        assert torch.equal(_bits(outs[0]), _bits(outs[1])), f"workspace filled with {fill:#x}"
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    ws2 = torch.empty(nb, dtype=torch.uint8, device="cuda")
    for k in range(12):
        _say(f"one-kernel split, call {k} on one workspace")
        x = softmax_input(M, N, seed=400 + k, dt="bf16").cuda()
        got = torch.empty((M, N), dtype=torch.float32, device="cuda")
        want = torch.empty_like(got)
        with rr.forced_variant(rr.RR_VARIANT_SPLIT_ONE_KERNEL):
            rr.rr_softmax_rows(got, x, ws)
        with rr.forced_variant(rr.RR_VARIANT_SPLIT_TWO_KERNELS):
            rr.rr_softmax_rows(want, x, ws2)
        torch.cuda.synchronize()
        assert torch.equal(_bits(got), _bits(want)), f"call {k}"


def test_split_one_kernel_wait_that_expires_is_counted_and_recomputed():
    """The one-kernel split's bounded wait: with the diagnostics build's wait
    at its default, every chunk's summary arrives in time (the fallback
    counter stays at 0); with the wait at 0 ticks workgroups give up on
    summaries not yet written, count them, and summarise those chunks from x
    themselves -- the output must still equal the two-kernel form's bit for
    bit."""
    rr = _rr()
    M, N = 40, 152064
    x = softmax_input(M, N, seed=321, dt="bf16").cuda()
    ws = rr.softmax_workspace(x, torch.float32)
    assert rr.rr_query_plan(rr.RR_OP_SOFTMAX, M, N, rr.RR_BF16, rr.RR_F32)["variant_name"] == "split"
    with rr.forced_variant(rr.RR_VARIANT_SPLIT_TWO_KERNELS):
        ref = torch.empty((M, N), dtype=torch.float32, device="cuda")
        rr.rr_softmax_rows(ref, x, ws)
        torch.cuda.synchronize()
    rr.split_fallbacks(reset=True)
    for ticks, what in ((rr.SPLIT_WAIT_TICKS_DEFAULT, "default wait"), (0, "no wait")):
        _say(f"one-kernel split {M}x{N}, {what}")
        with rr.split_wait(ticks):
            outs = []
            for k in range(3):
                y = torch.full((M, N), 3.0, dtype=torch.float32, device="cuda")
                rr.rr_softmax_rows(y, x, ws)
                torch.cuda.synchronize()
                outs.append(y)
        n = rr.split_fallbacks(reset=True)
        _say(f"  chunks summarised again: {n} of {3 * M * 19 * 18}")
        for y in outs:
            assert torch.equal(_bits(ref), _bits(y)), what
        if ticks:
            assert n == 0, f"{n} summaries missed a {ticks}-tick wait"
        else:
            assert n > 0, "a zero wait never gave up"


def test_split_row_longer_than_the_resident_grid():
    """One row of 2^25 fp32 values: more chunks than workgroups the GPU holds
    at once, so the one-kernel form falls back to the two kernels; both the
    default and the forced one-kernel request must match the oracle."""
    rr = _rr()
    x = softmax_input(1, 1 << 25, seed=6, dt="f32")
    check_softmax(x, run_softmax(x, torch.float32), "1 x 2^25")
    with rr.forced_variant(rr.RR_VARIANT_SPLIT_ONE_KERNEL):
        check_softmax(x, run_softmax(x, torch.float32), "1 x 2^25 one-kernel request")


def test_split_rows_with_many_chunks_are_merged_first():
    """Rows of more than 64 chunks take the merge kernel (each row's chunk
    summaries folded into one pair before pass B): a few rows just past the
    threshold and well past it, fp32 and bf16, plain and log output."""
    rr = _rr()
    for (M, N, dt) in [(2, 1 << 19, "f32"), (3, 65536 * 8 + 8, "bf16"), (5, 300000, "f32")]:
        p = rr.rr_query_plan(rr.RR_OP_SOFTMAX, M, N, rr.RR_F32 if dt == "f32" else rr.RR_BF16, rr.RR_F32)
        assert p["variant_name"] == "split" and p["chunks_per_row"] > 64, p
        _say(f"split with merge {dt} {M} x {N} ({p['chunks_per_row']} chunks)")
        x = softmax_input(M, N, seed=N + M, dt=dt)
        check_softmax(x, run_softmax(x, torch.float32), f"merged split {M}x{N}")
        y = run_ex_log(x)
        xf = compare.to_f64(x)
        compare.check_log_softmax(y, xf, oracle.log_softmax(xf), f"merged split log {M}x{N}")


def run_ex_log(x_cpu):
    rr = _rr()
    x = x_cpu.cuda()
    y = rr.softmax_rows_ex(x, out_dtype=torch.float32, log_output=True)
    torch.cuda.synchronize()
    return y.cpu()


def test_longest_row_closed_form():
    """One row of 2^30 fp32 values (the longest row the library accepts; 2^18
    chunks): the row is an 8-value pattern p repeated 2^27 times, so its
    softmax is softmax(p) / 2^27 at every position, with softmax(p) from the
    oracle.  Checked on the GPU in fp64: masked keys exactly 0, every other
    value within 1e-4 relative of the closed form (the chunk merge sums 2^18
    pairs in fp32), and the row sums to 1 within 1e-5."""
    rr = _rr()
    N = 1 << 30
    pattern = np.array([0.0, 1.0, 2.0, 3.0, -np.inf, 0.5, -2.0, 4.0], dtype=np.float32)
    ref = oracle.softmax(pattern[None, :].astype(np.float64))[0] / float(N // 8)
    x = torch.from_numpy(pattern).cuda().repeat(N // 8)
    y = torch.empty_like(x)
    _say(f"softmax 1 x 2^30 f32 ({rr.rr_query_plan(rr.RR_OP_SOFTMAX, 1, N, rr.RR_F32, rr.RR_F32)['chunks_per_row']} chunks)")
    ws = rr.softmax_workspace(x.view(1, N), torch.float32)
    rr.rr_softmax_rows(y.view(1, N), x.view(1, N), ws)
    torch.cuda.synchronize()
    del x
    y8 = y.view(-1, 8)
    refd = torch.from_numpy(ref).cuda()
    worst = 0.0
    total = 0.0
    step = 1 << 24
    for a in range(0, y8.shape[0], step):
        blk = y8[a:a + step].double()
        assert bool((blk[:, 4] == 0).all()), "masked key not 0"
        keep = [0, 1, 2, 3, 5, 6, 7]
        rel = ((blk[:, keep] - refd[keep]).abs() / refd[keep]).max().item()
        worst = max(worst, rel)
        total += blk.sum().item()
    _say(f"max rel err {worst:.3e}, row sum - 1 = {total - 1:.3e}")
    assert worst <= 1e-4
    assert abs(total - 1.0) <= 1e-5
    del y, y8
    torch.cuda.empty_cache()


def test_grid_capped_when_rows_outnumber_one_dispatch():
    """2^32 + 3 rows of 8 bf16 values: one workgroup per 256 rows would need
    more work-items than a dispatch counts (32 bits), so the grid is capped
    and the kernel walks the remaining rows grid-stride.  In place; zero rows
    give exactly 1/8 everywhere; the first, middle and last rows carry a
    pattern checked against the oracle."""
    rr = _rr()
    M, N = (1 << 32) + 3, 8
    p = rr.rr_query_plan(rr.RR_OP_SOFTMAX, M, N, rr.RR_BF16, rr.RR_BF16)
    assert p["work_items"] * p["block_threads"] > 0xFFFFFFFF, p
    pattern = torch.tensor([[0.0, -np.inf, 1.0, 2.0, -np.inf, 3.0, 0.5, -1.0]], dtype=torch.bfloat16)
    x = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    special = (0, M // 2, M - 1)
    for r in special:
        x[r] = pattern[0].cuda()
    _say(f"softmax in place {M} x {N} bf16 (plan {p['variant_name']}, {p['work_items']} workgroups)")
    rr.rr_softmax_rows(x, x, None)
    torch.cuda.synchronize()
    xf = compare.to_f64(pattern)
    ref = oracle.softmax(xf)
    for r in special:
        compare.check_softmax(x[r:r + 1].cpu(), xf, ref, f"row {r}")
        x[r] = 0.125
    step = 1 << 28
    bad = 0
    for a in range(0, M, step):
        bad += int((x[a:a + step] != 0.125).sum())
    assert bad == 0, f"{bad} values differ from 1/8"
    del x
    torch.cuda.empty_cache()


def test_packed_long_rows_many_rows():
    """Rows beyond 32 widened values per lane held packed in registers
    (1024-lane workgroups, 12-20 vectors per lane), with many rows."""
    rr = _rr()
    for (M, N, dt) in [(1024, 100000, "bf16"), (1100, 152064, "bf16"), (1024, 81920, "f32"),
                       (1030, 40000, "f32")]:
        p = rr.rr_query_plan(rr.RR_OP_SOFTMAX, M, N, rr.RR_BF16 if dt == "bf16" else rr.RR_F32,
                             rr.RR_F32)
        assert p["variant_name"] == "block" and p["vecs_per_lane"] >= 12, p
        _say(f"packed softmax {dt} M={M} N={N} nv={p['vecs_per_lane']}")
        x = softmax_input(M, N, seed=M + N, dt=dt)
        check_softmax(x, run_softmax(x, torch.float32), f"packed {M}x{N}")
    # the packed kernel's edges for bf16 -> fp32 (8-byte vectors: 24 to 40 per
    # lane), on few rows with the variant forced
    with rr.forced_variant(rr.RR_VARIANT_BLOCK):
        for (N, nv) in [(98304, 24), (98308, 32), (163836, 40), (163840, 40)]:
            p = rr.rr_query_plan(rr.RR_OP_SOFTMAX, 5, N, rr.RR_BF16, rr.RR_F32)
            assert p["vec_elems"] == 4 and p["vecs_per_lane"] == nv and p["block_threads"] == 1024, p
            _say(f"packed softmax bf16->f32 M=5 N={N} nv={nv}")
            x = softmax_input(5, N, seed=N, dt="bf16")
            check_softmax(x, run_softmax(x, torch.float32), f"packed forced 5x{N}")



SHIFT_WIDTHS = [33, 63, 65, 1023, 1025, 2049, 4097, 8191, 16385, 32767, 50257]
SHIFT_DTYPES = [("f32", "f32"), ("bf16", "f32"), ("bf16", "bf16"), ("f32", "bf16")]


@pytest.mark.parametrize("din,dout", SHIFT_DTYPES)
@pytest.mark.parametrize("N", SHIFT_WIDTHS)
def test_softmax_rows_cut_at_aligned_addresses(din, dout, N):
    """Softmax rows that are not whole aligned vectors are cut into vectors at
    aligned addresses (row_shift plans): contiguous rows of a width that is not
    a whole number of vectors (row r starts at offset r * N within a vector),
    and column slices at an odd column of wider matrices with equal strides
    (one common offset), whose surrounding columns must stay untouched."""
    rr = _rr()
    code = {"f32": rr.RR_F32, "bf16": rr.RR_BF16}
    for M in (1, 7, 66):
        plan = rr.rr_query_plan(rr.RR_OP_SOFTMAX, M, N, code[din], code[dout], 2)
        _say(f"cut rows {din}->{dout} M={M} N={N} plan={plan['variant_name']} shift={plan['row_shift']}")
        if N > 32 and N <= 32768:
            assert plan["row_shift"] == 1, plan
        x = softmax_input(M, N, seed=N + M, dt=din)
        check_softmax(x, run_softmax(x, _tdt(dout)), f"cut rows {din}->{dout} {M}x{N}")
    M, c0, ld = 9, 3, N + 5
    x = softmax_input(M, N, seed=N + 1000, dt=din)
    X = torch.full((M, ld), float("nan"), dtype=_tdt(din), device="cuda")
    X[:, c0:c0 + N] = x.cuda()
    Y = torch.full((M, ld), 7.0, dtype=_tdt(dout), device="cuda")
    nb = rr.rr_softmax_rows_workspace_bytes(M, N, code[din], code[dout])
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda") if nb else None
    rr.rr_softmax_rows_strided(Y[:, c0:c0 + N], X[:, c0:c0 + N], None, ws)
    torch.cuda.synchronize()
    Yc = Y.cpu()
    check_softmax(x, Yc[:, c0:c0 + N].contiguous(), f"cut column slice {din}->{dout} N={N}")
    assert bool((Yc[:, :c0] == 7.0).all()) and bool((Yc[:, c0 + N:] == 7.0).all()), "columns outside the slice changed"


# (M, N, in dtype, out dtype, log output): few rows too long for one
# workgroup's registers, so the row is split over workgroups with its chunks
# cut at aligned addresses; the last case has more than 64 chunks per row
# (the merge kernel runs)
SPLIT_CUT_CASES = [
    (1, 50257, "bf16", "f32", False), (4, 50257, "bf16", "f32", True), (39, 50257, "f32", "f32", False),
    (2, 152065, "bf16", "bf16", False), (5, 152065, "f32", "bf16", True), (7, 32769, "f32", "f32", False),
    (100, 163841, "bf16", "f32", False), (3, (1 << 19) + 3, "f32", "f32", False),
]


@pytest.mark.parametrize("M,N,din,dout,log", SPLIT_CUT_CASES)
def test_softmax_split_rows_cut_at_aligned_addresses(M, N, din, dout, log):
    """The split with rows cut at aligned addresses: contiguous rows of an odd
    width (each row at its own offset within a vector) and the same rows as a
    column slice at an odd column, against the oracle; the slice's
    neighbouring columns must stay untouched."""
    rr = _rr()
    code = {"f32": rr.RR_F32, "bf16": rr.RR_BF16}
    opts = rr.make_softmax_opts(log_output=log)
    x = softmax_input(M, N, seed=N + 7 * M, dt=din)
    xf = compare.to_f64(x)
    ref = oracle.log_softmax(xf) if log else oracle.softmax(xf)
    nb = rr.rr_softmax_rows_ex_workspace_bytes(M, N, code[din], code[dout], opts)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    for al, c0 in ((True, None), (2, 3)):
        plan = rr.rr_query_plan(rr.RR_OP_SOFTMAX, M, N, code[din], code[dout], al)
        _say(f"split cut rows {din}->{dout} {M}x{N} log={log} slice={c0} chunks={plan['chunks_per_row']}")
        assert (plan["variant_name"], plan["row_shift"]) == ("split", 1), plan
        assert nb >= plan["workspace_bytes"]
        if c0 is None:
            xs = x.cuda()
            Y = ys = torch.empty((M, N), dtype=_tdt(dout), device="cuda")
        else:
            ld = N + 6
            X = torch.full((M, ld), float("nan"), dtype=_tdt(din), device="cuda")
            X[:, c0:c0 + N] = x.cuda()
            Y = torch.full((M, ld), 7.0, dtype=_tdt(dout), device="cuda")
            xs, ys = X[:, c0:c0 + N], Y[:, c0:c0 + N]
        rr.rr_softmax_rows_strided(ys, xs, opts, ws)
        torch.cuda.synchronize()
        got = ys.cpu().contiguous()
        what = f"split cut rows {din}->{dout} {M}x{N} log={log} slice={c0}"
        if log:
            compare.check_log_softmax(got, xf, ref, what)
        else:
            compare.check_softmax(got, xf, ref, what)
        if c0 is not None:
            Yc = Y.cpu()
            assert bool((Yc[:, :c0] == 7.0).all()) and bool((Yc[:, c0 + N:] == 7.0).all()), what

# (M, N, in dtype, out dtype, log output, causal (period, offset) or None,
# column offset or None): rows cut at aligned addresses that no workgroup can
# hold (1024 rows or more, or a causal call), streamed twice
LOOP_CUT_CASES = [
    (1024, 81925, "f32", "f32", False, None, None),
    (8, 200003, "bf16", "f32", True, (8, 150000), None),
    (4, 300001, "f32", "bf16", False, (4, 290000), 3),
    (3, 163845, "bf16", "bf16", False, (3, 163844), 5),
]


@pytest.mark.parametrize("M,N,din,dout,log,causal,c0", LOOP_CUT_CASES)
def test_softmax_streamed_rows_cut_at_aligned_addresses(M, N, din, dout, log, causal, c0):
    """The streaming kernel with rows cut at aligned addresses, against the
    oracle (masked keys as -inf in the oracle's input, NaN in the kernel's,
    which must never read them); a column slice's neighbours stay untouched."""
    rr = _rr()
    code = {"f32": rr.RR_F32, "bf16": rr.RR_BF16}
    x = softmax_input(M, N, seed=N + 3 * M, dt=din)
    xf = compare.to_f64(x)
    period, offset = causal if causal else (None, 0)
    if causal:
        keys = np.minimum(N, np.arange(M) % period + offset + 1)
        masked = np.arange(N)[None, :] >= keys[:, None]
        xf[masked] = -np.inf
        x = torch.from_numpy(np.where(masked, np.float32(np.nan), compare.to_f64(x)).astype(np.float32)).to(_tdt(din))
    opts = rr.make_softmax_opts(log_output=log, causal_period=period, causal_offset=offset)
    op = rr.RR_OP_SOFTMAX_CAUSAL if causal else rr.RR_OP_SOFTMAX
    plan = rr.rr_query_plan(op, M, N, code[din], code[dout], 2)
    _say(f"streamed cut rows {din}->{dout} {M}x{N} log={log} causal={causal} slice={c0} plan={plan['variant_name']}")
    assert (plan["variant_name"], plan["row_shift"]) == ("loop", 1), plan
    if c0 is None:
        xs = x.cuda()
        Y = ys = torch.empty((M, N), dtype=_tdt(dout), device="cuda")
    else:
        ld = N + 7
        X = torch.full((M, ld), float("nan"), dtype=_tdt(din), device="cuda")
        X[:, c0:c0 + N] = x.cuda()
        Y = torch.full((M, ld), 7.0, dtype=_tdt(dout), device="cuda")
        xs, ys = X[:, c0:c0 + N], Y[:, c0:c0 + N]
    rr.rr_softmax_rows_strided(ys, xs, opts, None)
    torch.cuda.synchronize()
    got = ys.cpu().contiguous()
    what = f"streamed cut rows {din}->{dout} {M}x{N} log={log} causal={causal}"
    if log:
        compare.check_log_softmax(got, xf, oracle.log_softmax(xf), what)
    else:
        compare.check_softmax(got, xf, oracle.softmax(xf), what)
    if c0 is not None:
        Yc = Y.cpu()
        assert bool((Yc[:, :c0] == 7.0).all()) and bool((Yc[:, c0 + N:] == 7.0).all()), what
    del xs, ys, Y
    torch.cuda.empty_cache()


def test_softmax_in_place_unaligned_and_tiny():
    rr = _rr()
    for dt in ("f32", "bf16"):
        x = softmax_input(9, 4096, seed=11, dt=dt)
        check_softmax(x, run_softmax(x, _tdt(dt), inplace=True), f"in place {dt}")
    # unaligned input pointer
    M, N = 5, 3000
    x = softmax_input(M, N, seed=12, dt="f32")
    base = torch.empty(M * N + 1, device="cuda")
    xv = base[1:].view(M, N)
    xv.copy_(x.cuda())
    y = torch.empty(M, N, device="cuda")
    rr.rr_softmax_rows(y, xv, None)
    torch.cuda.synchronize()
    check_softmax(x, y.cpu(), "unaligned")
    # the pages' worked examples, through the kernels
    # ... and a row whose fifth entry is 90, where exp without the max
    # subtracted overflows fp32 (the pages' overflow test)
    for row in ([1000.0, 1001.0], [1.0, 3.0, 2.0], [2.0, 4.0, 1.0], [1.0, 2.0, 5.0, 3.0],
                [0.0, 0.1, 0.2, 0.3, 0.4, 90.0, 0.6, 0.7]):
        x = torch.tensor([row], dtype=torch.float32)
        y = run_softmax(x, torch.float32)
        check_softmax(x, y, f"example {row}")
    # M = 0: a successful no-op that touches nothing
    y0 = torch.full((0, 64), 7.0, device="cuda")
    rr.rr_softmax_rows(y0, torch.empty((0, 64), device="cuda"), None)
    # N = 1: probability 1, or NaN for a masked entry
    x = torch.tensor([[5.0], [-np.inf], [0.0]], dtype=torch.float32)
    y = run_softmax(x, torch.float32).numpy()
    assert y[0, 0] == 1.0 and np.isnan(y[1, 0]) and y[2, 0] == 1.0


# Rows whose entries lie 87-92 below the row maximum: exp(x - m) is then a
# float below 2^-126 that rounds to a bf16 subnormal (bf16's subnormals reach
# down to 2^-133), so a kernel that flushed such exponentials to zero would
# be up to 128 bf16 ulps off.  One case per kernel family the planner picks
# for bf16 outputs: short rows, a wavefront per row, a workgroup per row,
# the packed workgroup, the split row, rows cut at aligned addresses.
SUBNORMAL_CASES = [
    (64, 24, "f32"), (64, 1024, "bf16"), (16, 8192, "f32"), (80, 65536, "bf16"),
    (4, 65536, "bf16"), (3, 152064, "f32"), (64, 1021, "bf16"),
]


@pytest.mark.parametrize("M,N,din", SUBNORMAL_CASES)
def test_softmax_bf16_output_subnormal_probabilities(M, N, din):
    rr = _rr()
    rng = np.random.default_rng(M * 7 + N)
    x = rng.uniform(-92.0, -87.0, (M, N)).astype(np.float32)
    # a quarter of the entries whose exponentials are normal but small (so
    # that d stays near 1), and the maximum 0
    sel = rng.random((M, N)) < 0.25
    x[sel] = rng.uniform(-40.0, -20.0, int(sel.sum())).astype(np.float32)
    x[:, rng.integers(0, N)] = 0.0
    x_cpu = _as(x, din)
    plan = rr.rr_query_plan(rr.RR_OP_SOFTMAX, M, N, rr.RR_F32 if din == "f32" else rr.RR_BF16, rr.RR_BF16,
                            aligned16=1 if (N * (4 if din == "f32" else 2)) % 16 == 0 else 2)
    _say(f"[subnormal] M={M} N={N} {din}->bf16 plan={plan['variant_name']}")
    y = run_softmax(x_cpu, torch.bfloat16)
    info = check_softmax(x_cpu, y, f"subnormal outputs {M}x{N} {din}->bf16")
    # the case must reach the subnormal range: most outputs are nonzero subnormals
    yb = compare.bf16_bits_of_tensor(y)
    sub = ((yb & 0x7F80) == 0) & ((yb & 0x7F) != 0)
    assert sub.mean() > 0.3, f"only {sub.mean():.2f} of the outputs are subnormal"
    _say(f"  {info}")


def test_softmax_shift_invariance_bitwise():
    # adding an exact constant to every entry of a dyadic row changes no
    # x - m and so no output bit (same kernel, same order)
    M, N = 64, 4096
    x = workloads.random_rows(M, N, seed=21)
    x = np.round(x * 64) / 64
    y1 = run_softmax(_as(x, "f32"), torch.float32)
    y2 = run_softmax(_as(x + np.float32(512.0), "f32"), torch.float32)
    assert torch.equal(_bits(y1), _bits(y2))


def _bits(t):
    return t.contiguous().view(torch.int32 if t.element_size() == 4 else torch.int16)


def test_determinism_run_to_run():
    """Same inputs, same launch: the same bits (NaN rows included)."""
    rr = _rr()
    for name in ("fused", "sm_wave"):
        w = workloads.make(name, rows=1024)
        outs = []
        for _ in range(3):
            if w.op == "fused_add_rmsnorm":
                y, r = run_fused(w.arrays["x"], w.arrays["residual"], w.arrays["gamma"], w.eps)
                outs.append(torch.cat([y.view(-1).float(), r.view(-1).float()]))
            else:
                outs.append(run_softmax(w.arrays["x"], torch.float32))
        assert all(torch.equal(_bits(outs[0]), _bits(o)) for o in outs[1:]), name
    x = softmax_input(8, 152064, seed=2, dt="bf16")
    a = run_softmax(x, torch.float32)
    b = run_softmax(x, torch.float32)
    assert torch.equal(_bits(a), _bits(b))


# ----------------------------------------------------------------------------
# the named workloads at full size, in the launch configuration the benchmark
# times (automatic dispatch, default grid)
# ----------------------------------------------------------------------------

def test_workload_rms_f32_full():
    w = workloads.make("rms_f32")
    _say(w.description)
    y = run_rmsnorm(w.arrays["x"], w.arrays["gamma"], w.eps)
    info = check_norm(w.arrays["x"], w.arrays["gamma"], w.eps, "f32", y, w.name)
    _say(info)


def test_workload_fused_full():
    w = workloads.make("fused")
    _say(w.description)
    y, r_out = run_fused(w.arrays["x"], w.arrays["residual"], w.arrays["gamma"], w.eps)
    info = check_fused(w.arrays["x"], w.arrays["residual"], w.arrays["gamma"], w.eps, "bf16",
                       y, r_out, w.name)
    _say(info)


def test_workload_rmsnorm_bf16_8192x4096_full():
    w = workloads.make("fused")
    _say("rmsnorm bf16 8192x4096 (the fused workload's x and gamma)")
    y = run_rmsnorm(w.arrays["x"], w.arrays["gamma"], w.eps)
    _say(check_norm(w.arrays["x"], w.arrays["gamma"], w.eps, "bf16", y, "rmsnorm bf16"))


def test_workload_sm_wave_full():
    w = workloads.make("sm_wave")
    _say(w.description)
    y = run_softmax(w.arrays["x"], torch.float32)
    _say(check_softmax(w.arrays["x"], y, w.name))


def test_workload_sm_vocab_full():
    """The vocabulary workload as planned (one packed workgroup per row), and
    all of its rows through the split-row (m, d) combine the workload is
    named for (the two-kernel form: 256 rows of 19 chunks are more than the
    device holds at once for the one-kernel form)."""
    rr = _rr()
    w = workloads.make("sm_vocab")
    _say(w.description)
    y = run_softmax(w.arrays["x"], torch.float32)
    _say(check_softmax(w.arrays["x"], y, w.name))
    with rr.forced_variant(rr.RR_VARIANT_SPLIT):
        assert rr.rr_query_plan(rr.RR_OP_SOFTMAX, 256, 152064, rr.RR_BF16, rr.RR_F32)["chunks_per_row"] == 19
        ys = run_softmax(w.arrays["x"], torch.float32)
    _say(check_softmax(w.arrays["x"], ys, w.name + " (split)"))


def test_workload_sm_causal_full_sampled():
    """All 114688 rows run on the GPU; sampled rows against the oracle, and
    properties checked on every row (sum 1, masked keys exactly 0, finite,
    non-negative)."""
    w = workloads.make("sm_causal")
    _say(w.description)
    x = w.arrays["x"].cuda()
    y = torch.empty_like(x)
    _rr().rr_softmax_rows(y, x, None)
    torch.cuda.synchronize()
    M, N = x.shape
    rows = sorted({0, 1, 2, 63, 64, 1000, 2047, 2048, 4094, 4095, 4096, 4097, 8191,
                   M // 2, M - 4096, M - 2, M - 1} |
                  set(np.random.default_rng(7).integers(0, M, 48).tolist()))
    xs = w.arrays["x"][rows]
    ys = y[rows].cpu()
    _say(check_softmax(xs, ys, "sm_causal sampled"))
    # every row: sum to 1, masked entries exactly 0, finite and >= 0
    rs = y.double().sum(dim=1)
    assert float((rs - 1.0).abs().max()) <= compare.SOFTMAX_ROWSUM_ATOL
    masked = torch.isneginf(x)
    assert int((y[masked] != 0).sum()) == 0
    assert bool(torch.isfinite(y).all()) and bool((y >= 0).all())
    # the number of masked keys in row r is 4095 - (r mod 4096)
    nm = masked.sum(dim=1).cpu().numpy()
    assert np.array_equal(nm, 4095 - (np.arange(M) % 4096))
