"""GPU parity of rr_softmax_rows_ex: log-softmax and the causal rule whose
masked keys are never read, against the fp64 oracle.

The causal kernels are given inputs whose masked region holds NaN, +inf and
3e38: a kernel that read any masked key would produce a NaN or a wrong
normaliser.  The oracle gets the same rows with the masked keys set to
-inf, which is what the causal rule means.  Expected values come only from
``oracle``; bars are in tests/compare.py.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests import compare
from tests.test_parity_gpu import DTYPES, _as, _bits, _rr, _say, _tdt, softmax_input

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rr = _rr()
    rr.lib()
    yield


def run_ex(x_cpu, out_dt, log_output=False, period=None, offset=0, inplace=False):
    rr = _rr()
    x = x_cpu.cuda()
    y = x if inplace else torch.empty(x.shape, dtype=out_dt, device=x.device)
    rr.softmax_rows_ex(x, out=y, log_output=log_output, causal_period=period, causal_offset=offset)
    torch.cuda.synchronize()
    return y.cpu()


def kept_keys(M, N, period, offset):
    """Keys each row keeps under the causal rule: min(N, (i mod P) + O + 1)."""
    return np.minimum(N, np.arange(M) % period + offset + 1)


def causal_inputs(M, N, period, offset, seed, dt):
    """(x_given, x_meant): the softmax test rows; x_given has garbage in the
    masked region, x_meant has -inf there (as fp64)."""
    x = softmax_input(M, N, seed, dt)
    xf = compare.to_f64(x)
    keys = kept_keys(M, N, period, offset)
    cols = np.arange(N)[None, :]
    masked = cols >= keys[:, None]
    meant = xf.copy()
    meant[masked] = -np.inf
    garbage = np.array([np.nan, np.inf, 3e38], dtype=np.float64)
    given = xf.copy()
    given[masked] = garbage[(np.arange(M)[:, None] + cols) % 3][masked]
    return _as(given.astype(np.float32), dt), meant


def check_ex(y_cpu, x_meant, log_output, what):
    if log_output:
        ref = oracle.log_softmax(x_meant)
        return compare.check_log_softmax(y_cpu, x_meant, ref, what)
    ref = oracle.softmax(x_meant)
    return compare.check_softmax(y_cpu, x_meant, ref, what)


# ----------------------------------------------------------------------------
# log-softmax
# ----------------------------------------------------------------------------

LOG_N = [1, 7, 64, 65, 1000, 1024, 2048, 2056, 4096, 16385, 32768, 50000, 152064]


@pytest.mark.parametrize("din,dout", DTYPES)
@pytest.mark.parametrize("N", LOG_N)
def test_log_softmax_grid(din, dout, N):
    for M in ([1, 7, 33] if N < 50000 else [1, 7]):
        _say(f"log-softmax {din}->{dout} M={M} N={N}")
        x = softmax_input(M, N, seed=7 * N + M, dt=din)
        y = run_ex(x, _tdt(dout), log_output=True)
        check_ex(y, compare.to_f64(x), True, f"log-softmax {din}->{dout} {M}x{N}")


@pytest.mark.parametrize("variant", ["wave", "block", "split", "split1", "split2", "loop", "subwave"])
def test_log_softmax_forced_variants(variant):
    rr = _rr()
    code = {"wave": rr.RR_VARIANT_WAVE, "block": rr.RR_VARIANT_BLOCK,
            "split": rr.RR_VARIANT_SPLIT, "split1": rr.RR_VARIANT_SPLIT_ONE_KERNEL,
            "split2": rr.RR_VARIANT_SPLIT_TWO_KERNELS,
            "loop": rr.RR_VARIANT_LOOP, "subwave": rr.RR_VARIANT_SUBWAVE}[variant]
    shapes = {"wave": [8, 1024, 2048], "block": [8, 4096, 32768, 65536],
              "split": [8, 4104, 65536], "split1": [8, 65536], "split2": [8, 4104, 65536],
              "loop": [8, 4096, 100000], "subwave": [8, 40, 128]}[variant]
    with rr.forced_variant(code):
        for din, dout in DTYPES:
            for N in shapes:
                if variant == "wave" and din == "bf16" and N > 2048:
                    continue
                for M in (1, 7):
                    _say(f"log-softmax forced {variant} {din}->{dout} M={M} N={N}")
                    x = softmax_input(M, N, seed=M + 3 * N, dt=din)
                    y = run_ex(x, _tdt(dout), log_output=True)
                    check_ex(y, compare.to_f64(x), True, f"log {variant} {din}->{dout} {M}x{N}")


def test_log_softmax_exp_matches_softmax_and_examples():
    """exp(log-softmax) is the softmax; the pages' worked examples."""
    x = softmax_input(64, 4096, seed=31, dt="f32")
    lg = run_ex(x, torch.float32, log_output=True)
    sm = run_ex(x, torch.float32)
    ok = ~torch.isnan(sm)
    assert float((lg.double().exp() - sm.double())[ok].abs().max()) <= 4e-6
    for row in ([1000.0, 1001.0], [1.0, 3.0, 2.0], [2.0, 4.0, 1.0], [1.0, 2.0, 5.0, 3.0]):
        xr = torch.tensor([row], dtype=torch.float32)
        y = run_ex(xr, torch.float32, log_output=True)
        check_ex(y, compare.to_f64(xr), True, f"log example {row}")
    # N = 1: log 1 = 0, or NaN for a masked entry; in place
    x1 = torch.tensor([[5.0], [-np.inf], [0.0]], dtype=torch.float32)
    y1 = run_ex(x1, torch.float32, log_output=True, inplace=True).numpy()
    assert y1[0, 0] == 0.0 and np.isnan(y1[1, 0]) and y1[2, 0] == 0.0


# ----------------------------------------------------------------------------
# causal rule (masked keys never read)
# ----------------------------------------------------------------------------

CAUSAL_CASES = [
    # M, N, period, offset: square attention blocks, offsets (keys beyond the
    # queries), a period that does not divide M, offsets past N, unaligned N,
    # each dispatch path (subwave, wave, block, packed, loop)
    (40, 8, 8, 0),
    (100, 31, 7, 3),
    (64, 64, 64, 0),
    (300, 1024, 300, 0),
    (33, 2048, 33, 2015),
    (70, 1000, 64, 900),
    (65, 4096, 64, 0),
    (20, 4096, 20, 5000),
    (17, 16385, 17, 16000),
    (33, 32768, 33, 32735),
    (1030, 40000, 1030, 38970),
    (9, 152064, 9, 152055),
    (300, 1025, 300, 0),        # odd widths: rows cut at aligned addresses (wave, block, packed)
    (40, 4097, 40, 4057),
    (66, 50257, 66, 50191),
    # rows q and P - 1 - q of a period in one workgroup (aligned rows of the
    # workgroup plan with kept counts that vary along the period): an odd
    # period (its middle row alone), rows past the last whole period, an
    # offset, 16 wavefronts per row, four vectors per lane
    (129, 4096, 43, 0),
    (1000, 3072, 700, 100),
    (64, 8192, 64, 1800),
    (2048, 16384, 2048, 0),
]


@pytest.mark.parametrize("log_output", [False, True])
@pytest.mark.parametrize("din,dout", DTYPES)
@pytest.mark.parametrize("case", CAUSAL_CASES, ids=lambda c: "x".join(map(str, c)))
def test_causal_grid(case, din, dout, log_output):
    M, N, P, O = case
    rr = _rr()
    p = rr.rr_query_plan(rr.RR_OP_SOFTMAX_CAUSAL, M, N, rr.dtype_code(torch.empty(0, dtype=_tdt(din))),
                         rr.dtype_code(torch.empty(0, dtype=_tdt(dout))), True)
    _say(f"causal {din}->{dout} log={log_output} M={M} N={N} P={P} O={O} plan={p['variant_name']}")
    given, meant = causal_inputs(M, N, P, O, seed=M + N + P, dt=din)
    y = run_ex(given, _tdt(dout), log_output=log_output, period=P, offset=O)
    check_ex(y, meant, log_output, f"causal {din}->{dout} {M}x{N} P={P} O={O} log={log_output}")


@pytest.mark.parametrize("variant", ["wave", "block", "loop", "subwave"])
def test_causal_forced_variants(variant):
    rr = _rr()
    code = {"wave": rr.RR_VARIANT_WAVE, "block": rr.RR_VARIANT_BLOCK,
            "loop": rr.RR_VARIANT_LOOP, "subwave": rr.RR_VARIANT_SUBWAVE}[variant]
    shapes = {"wave": [8, 1024, 2048], "block": [8, 4096, 65536, 163840],
              "loop": [8, 4096, 100000], "subwave": [8, 40, 128]}[variant]
    with rr.forced_variant(code):
        for din, dout in DTYPES:
            for N in shapes:
                if variant == "wave" and din == "bf16" and N > 2048:
                    continue
                if variant == "block" and din == "f32" and N > 81920:
                    continue   # beyond a 1024-lane workgroup's registers for fp32
                for log_output in (False, True):
                    M = 37
                    O = max(0, N - M)
                    _say(f"causal forced {variant} {din}->{dout} N={N} log={log_output}")
                    given, meant = causal_inputs(M, N, M, O, seed=N + M, dt=din)
                    y = run_ex(given, _tdt(dout), log_output, period=M, offset=O)
                    check_ex(y, meant, log_output, f"causal {variant} {din}->{dout} {M}x{N}")


def test_causal_in_place_and_unaligned():
    rr = _rr()
    for dt in ("f32", "bf16"):
        given, meant = causal_inputs(50, 4096, 50, 4000, seed=3, dt=dt)
        y = run_ex(given, _tdt(dt), period=50, offset=4000, inplace=True)
        check_ex(y, meant, False, f"causal in place {dt}")
    # unaligned input pointer: the scalar streaming path
    M, N = 30, 3000
    given, meant = causal_inputs(M, N, M, N - M, seed=4, dt="f32")
    base = torch.empty(M * N + 1, device="cuda")
    xv = base[1:].view(M, N)
    xv.copy_(given.cuda())
    y = torch.empty(M, N, device="cuda")
    rr.softmax_rows_ex(xv, out=y, causal_period=M, causal_offset=N - M)
    torch.cuda.synchronize()
    check_ex(y.cpu(), meant, False, "causal unaligned")


def test_ex_without_options_is_rr_softmax_rows_bitwise():
    """No options, or all-zero options: the same kernels and bits as
    rr_softmax_rows (with the split path's workspace where it needs one)."""
    rr = _rr()
    for (M, N, din, dout) in [(64, 1024, "f32", "f32"), (9, 32768, "bf16", "f32"),
                              (40, 152064, "bf16", "f32"), (300, 24, "bf16", "bf16")]:
        x = softmax_input(M, N, seed=M * N, dt=din).cuda()
        ws = rr.softmax_workspace(x, _tdt(dout))
        a = torch.empty(x.shape, dtype=_tdt(dout), device="cuda")
        b = torch.empty_like(a)
        c = torch.empty_like(a)
        rr.rr_softmax_rows(a, x, ws)
        rr.rr_softmax_rows_ex(b, x, None, ws)
        rr.rr_softmax_rows_ex(c, x, rr.make_softmax_opts(), ws)
        torch.cuda.synchronize()
        assert torch.equal(_bits(a), _bits(b)) and torch.equal(_bits(a), _bits(c)), (M, N)


def test_causal_equals_plain_softmax_on_masked_input_bitwise():
    """The causal kernel on garbage-masked rows gives the same bits as the
    plain kernel on rows with -inf in the masked region: the masked keys
    enter the arithmetic as -inf either way, in the same order."""
    for (M, N, P, O) in [(64, 1024, 64, 960), (65, 4096, 64, 0), (1030, 40000, 1030, 38970),
                         (129, 4096, 43, 0), (1000, 3072, 700, 100), (300, 16384, 256, 0)]:
        given, meant = causal_inputs(M, N, P, O, seed=5, dt="f32")
        yc = run_ex(given, torch.float32, period=P, offset=O)
        yp = run_ex(torch.from_numpy(meant.astype(np.float32)), torch.float32)
        assert torch.equal(_bits(yc), _bits(yp)), (M, N, P, O)


def test_workload_sm_causal_aware_full():
    """The attention-score workload (28 heads x 4096 queries x 4096 keys)
    through the causal kernel with NaN in the masked half: bitwise equal to
    the plain kernel on the -inf-masked input (whose parity the sampled
    full-size test checks), on every row."""
    rr = _rr()
    w = workloads.make("sm_causal")
    _say(w.description)
    x = w.arrays["x"].cuda()
    y_plain = torch.empty_like(x)
    rr.rr_softmax_rows(y_plain, x, None)
    masked = torch.isneginf(x)
    x.masked_fill_(masked, float("nan"))
    y = torch.empty_like(x)
    rr.softmax_rows_ex(x, out=y, causal_period=4096, causal_offset=0)
    torch.cuda.synchronize()
    assert torch.equal(_bits(y), _bits(y_plain))
    assert int((y[masked] != 0).sum()) == 0
    # the log form on sampled rows against the oracle
    yl = torch.empty_like(x)
    rr.softmax_rows_ex(x, out=yl, log_output=True, causal_period=4096, causal_offset=0)
    torch.cuda.synchronize()
    M = x.shape[0]
    rows = sorted({0, 1, 4095, 4096, M // 2, M - 1} |
                  set(np.random.default_rng(8).integers(0, M, 24).tolist()))
    xs = compare.to_f64(w.arrays["x"][rows])
    _say(check_ex(yl[rows].cpu(), xs, True, "sm_causal log sampled"))
