"""Pins for the CPU oracle: checks that do not trust the oracle itself.

Each oracle function is checked against something other than its own formula:
the pages' printed worked examples (tests/golden/worked_examples.json),
closed forms, invariants, a different algorithm (the online recurrence and
every bracketing of the merge, brute force on tiny rows), and library
routines that compute the same definition (torch fp64 softmax / rms_norm,
torch's bf16 conversion).  The cases are chosen so that a dropped term, a
wrong sign, a misplaced eps, a wrong divisor, a transposed operand or a
double rounding fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import online_ref

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _golden():
    with open(GOLDEN, encoding="utf-8") as f:
        return json.load(f)


def _tol(decimals):
    return 0.5 * 10.0 ** (-decimals) + 1e-12


# ----------------------------------------------------------------------------
# worked examples printed on the pages
# ----------------------------------------------------------------------------

def test_rmsnorm_worked_example():
    for ex in _golden()["rmsnorm"]:
        x = np.array([ex["x"]])
        y = oracle.rmsnorm(x, np.array(ex["gamma"]), ex["eps"])[0]
        tol = _tol(ex["decimals"])
        assert np.all(np.abs(y - np.array(ex["y"])) <= tol), (ex["id"], y)
        # r itself: y_j = x_j * r with gamma = 1
        r = y[0] / ex["x"][0]
        assert abs(r - ex["r"]) <= tol
        assert abs(np.mean(y * y) - ex["mean_square_y"]) <= 1e-12


def test_softmax_worked_examples():
    for ex in _golden()["softmax"]:
        x = np.array([ex["x"]])
        tol = _tol(ex["decimals"])
        m, d = oracle.softmax_stats(x)
        if "d" in ex:
            assert abs(d[0] - ex["d"]) <= tol, (ex["id"], d)
        if "m" in ex:
            assert m[0] == ex["m"]
        if "y" in ex:
            y = oracle.softmax(x)[0]
            assert np.all(np.abs(y - np.array(ex["y"])) <= tol), (ex["id"], y)
        if "exps" in ex:
            e = np.exp(np.array(ex["x"]) - m[0])
            assert np.all(np.abs(e - np.array(ex["exps"])) <= tol)
        if "steps" in ex:
            # the intermediate online states printed on the page
            for k, (ms, ds) in enumerate(ex["steps"]):
                mk, dk = online_ref.online_stats(ex["x"][: k + 1])
                assert mk == ms and abs(dk - ds) <= tol, (ex["id"], k, mk, dk)
            mo, do = online_ref.online_stats(ex["x"])
            assert abs(do - d[0]) <= 1e-15 * d[0]


def test_merge_worked_examples():
    g = _golden()["merge"]
    ex = g[0]
    a = online_ref.online_stats(ex["A"])
    b = online_ref.online_stats(ex["B"])
    assert a == (3.0, 1.0 + math.exp(-2.0))
    assert b == (2.0, 1.0)
    mm = online_ref.merge(a, b)
    assert mm[0] == 3.0
    assert abs(mm[1] - (1.0 + math.exp(-2.0) + math.exp(-1.0))) <= 1e-15
    # equals the three-pass statistic of the union
    m, d = oracle.softmax_stats(np.array([ex["A"] + ex["B"]]))
    assert m[0] == mm[0] and abs(d[0] - mm[1]) <= 2e-16 * d[0]

    ex = g[1]
    m, d = oracle.softmax_stats(np.array([ex["x"]]))
    assert m[0] == ex["m"]
    assert abs(d[0] - ex["s"]) <= _tol(ex["s_decimals"])
    assert abs(d[0] * math.exp(m[0]) - ex["T"]) <= _tol(ex["T_decimals"])


# ----------------------------------------------------------------------------
# RMSNorm: closed forms, invariants, library routine
# ----------------------------------------------------------------------------

def test_rmsnorm_constant_row_closed_form():
    # x_j = c for all j: mean square c^2, so y_j = c / sqrt(c^2 + eps) * gamma_j.
    # With eps != 0 this separates "eps inside the root" from the other
    # placements, and H from H - 1.
    H, c, eps = 7, 0.25, 0.01
    gamma = np.arange(1, H + 1, dtype=np.float64)
    y = oracle.rmsnorm(np.full((1, H), c), gamma, eps)[0]
    expect = c / math.sqrt(c * c + eps) * gamma
    assert np.allclose(y, expect, rtol=1e-15, atol=0)


def test_rmsnorm_unit_mean_square_and_scale_invariance():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((5, 33))
    y = oracle.rmsnorm(x, np.ones(33), 0.0)
    assert np.allclose(np.mean(y * y, axis=1), 1.0, rtol=0, atol=1e-14)
    # eps = 0: multiplying a row by a power of two changes nothing, bitwise
    y2 = oracle.rmsnorm(x * 8.0, np.ones(33), 0.0)
    assert np.array_equal(y, y2)


def test_rmsnorm_matches_torch_fp64():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(12)
    for (M, H, eps) in [(3, 5, 1e-6), (4, 97, 1e-2), (2, 3584, 1e-6), (6, 1, 0.5)]:
        x = rng.standard_normal((M, H)) * 2.0
        g = rng.uniform(0.5, 1.5, H)
        y = oracle.rmsnorm(x, g, eps)
        ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (H,),
                                           weight=torch.from_numpy(g), eps=eps).numpy()
        assert np.allclose(y, ref, rtol=1e-13, atol=1e-15), (M, H)


def test_rmsnorm_rejects_empty_row():
    with pytest.raises(ValueError):
        oracle.rmsnorm(np.zeros((2, 0)), np.zeros(0), 1e-6)


# ----------------------------------------------------------------------------
# LayerNorm: closed forms, invariants, library routine
# ----------------------------------------------------------------------------

def test_layernorm_closed_forms():
    # x = (1, 2, 3, 4): mean 2.5, variance (2.25 + 0.25 + 0.25 + 2.25) / 4 = 1.25
    y = oracle.layernorm(np.array([[1.0, 2.0, 3.0, 4.0]]), np.ones(4), None, 0.0)[0]
    expect = (np.array([1.0, 2.0, 3.0, 4.0]) - 2.5) / math.sqrt(1.25)
    assert np.allclose(y, expect, rtol=1e-15, atol=1e-15)
    # a constant row has x - mean = 0, so y = beta exactly, whatever eps and gamma
    beta = np.linspace(-1, 1, 9)
    y = oracle.layernorm(np.full((2, 9), 101.25), np.arange(1.0, 10.0), beta, 1e-5)
    assert np.array_equal(y, np.stack([beta, beta]))
    # eps inside the root and the 1/H divisor: two values +-a give var = a^2
    a, eps = 0.5, 0.01
    y = oracle.layernorm(np.array([[a, -a]]), np.ones(2), np.zeros(2), eps)[0]
    assert np.allclose(y, [a / math.sqrt(a * a + eps), -a / math.sqrt(a * a + eps)], rtol=1e-15)


def test_layernorm_invariants():
    rng = np.random.default_rng(19)
    x = rng.uniform(100.0, 102.0, (6, 5120))
    y = oracle.layernorm(x, np.ones(5120), None, 0.0)
    assert np.allclose(y.mean(axis=1), 0.0, atol=1e-12)
    assert np.allclose((y * y).mean(axis=1), 1.0, atol=1e-12)
    # translation invariance, bitwise for an exact shift of dyadic values
    xd = np.round(rng.standard_normal((4, 64)) * 64) / 64
    assert np.array_equal(oracle.layernorm(xd, np.ones(64), None, 1e-5),
                          oracle.layernorm(xd + 256.0, np.ones(64), None, 1e-5))


def test_layernorm_matches_torch_fp64():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(20)
    for (M, H, eps, lo, hi) in [(3, 5, 1e-5, -1, 1), (4, 5120, 1e-5, 100, 102), (2, 97, 0.3, -3, 9),
                                (5, 1, 1e-5, -1, 1)]:
        x = rng.uniform(lo, hi, (M, H))
        g = rng.uniform(0.5, 1.5, H)
        b = rng.uniform(-1, 1, H)
        y = oracle.layernorm(x, g, b, eps)
        ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (H,), weight=torch.from_numpy(g),
                                             bias=torch.from_numpy(b), eps=eps).numpy()
        # two fp64 summation orders differ near 1e-12 when the mean is ~100x the spread
        assert np.allclose(y, ref, rtol=1e-10, atol=1e-11), (M, H)
        y0 = oracle.layernorm(x, g, None, eps)
        assert np.allclose(y0, ref - b, rtol=1e-10, atol=1e-11)


# ----------------------------------------------------------------------------
# bf16 rounding: library routine, ties, single rounding, range ends
# ----------------------------------------------------------------------------

def test_round_bf16_matches_torch_on_fp32_values():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(13)
    # fp32 values spread over the whole exponent range, both signs
    bits = rng.integers(0, 2**32, 200000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    ours = oracle.round_bf16(f.astype(np.float64))
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all(), f[~same][:5]


def test_round_bf16_ties_and_single_rounding():
    r = oracle.round_bf16
    u = 2.0 ** -7                     # bf16 spacing on [1, 2)
    cases = [
        (1.0 + u / 2, 1.0),           # tie -> even (1.0)
        (1.0 + 3 * u / 2, 1.0 + 2 * u),   # tie -> even (mantissa ...10)
        (1.0 + u / 2 + 2.0 ** -40, 1.0 + u),  # just above the tie: up (no double rounding)
        (-(1.0 + u / 2 + 2.0 ** -40), -(1.0 + u)),
        (2.0 ** -134, 0.0),           # half the smallest subnormal: tie -> 0
        (1.5 * 2.0 ** -133, 2.0 ** -132),  # subnormal tie -> even
        ((2.0 - 2.0 ** -8) * 2.0 ** 127, math.inf),  # tie above the largest: overflow
        ((2.0 - 2.0 ** -8 - 2.0 ** -30) * 2.0 ** 127, (2.0 - 2.0 ** -7) * 2.0 ** 127),
        (-0.0, -0.0), (math.inf, math.inf),
    ]
    got = r(np.array([c[0] for c in cases]))
    for (v, e), g in zip(cases, got):
        assert g == e and math.copysign(1, g) == math.copysign(1, e), (v, g, e)


# ----------------------------------------------------------------------------
# fused residual add + RMSNorm
# ----------------------------------------------------------------------------

def test_fused_residual_is_rounded_sum_bf16_vs_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(14)
    M, H = 6, 4096
    xb = torch.from_numpy(rng.standard_normal((M, H), dtype=np.float32)).to(torch.bfloat16)
    rb = torch.from_numpy(rng.standard_normal((M, H), dtype=np.float32) * 4).to(torch.bfloat16)
    gb = torch.from_numpy(rng.uniform(0.5, 1.5, H).astype(np.float32)).to(torch.bfloat16)
    x, r, g = (t.to(torch.float64).numpy() for t in (xb, rb, gb))
    h, y = oracle.fused_add_rmsnorm(x, r, g, 1e-6, "bf16")
    # torch's bf16 add rounds the (fp32) sum once to bf16, which equals the
    # correctly rounded sum because fp32 carries more than 2*8+2 bits
    h_ref = (xb + rb).to(torch.float64).numpy()
    assert np.array_equal(h, h_ref)
    # y is RMSNorm of the stored residual (the composition add -> rmsnorm)
    y_ref = torch.nn.functional.rms_norm(torch.from_numpy(h_ref), (H,),
                                         weight=torch.from_numpy(g), eps=1e-6).numpy()
    assert np.allclose(y, y_ref, rtol=1e-13, atol=1e-15)
    # and differs measurably from RMSNorm of the unrounded sum, so a kernel
    # that skipped the rounding would be caught by the bf16 comparison
    y_unrounded = oracle.rmsnorm(x + r, g, 1e-6)
    assert np.max(np.abs(y - y_unrounded)) > 1e-4


def test_fused_f32_and_zero_residual():
    rng = np.random.default_rng(15)
    M, H = 3, 50
    x = rng.standard_normal((M, H)).astype(np.float32).astype(np.float64)
    r = rng.standard_normal((M, H)).astype(np.float32).astype(np.float64)
    g = rng.uniform(0.5, 1.5, H)
    h, y = oracle.fused_add_rmsnorm(x, r, g, 1e-6, "f32")
    assert np.array_equal(h, (x.astype(np.float32) + r.astype(np.float32)).astype(np.float64))
    # zero residual: the fused op reduces to plain RMSNorm of x
    h0, y0 = oracle.fused_add_rmsnorm(x, np.zeros_like(x), g, 1e-6, "f32")
    assert np.array_equal(h0, x)
    assert np.array_equal(y0, oracle.rmsnorm(x, g, 1e-6))


# ----------------------------------------------------------------------------
# softmax: invariants, library routine, brute force against the online method
# ----------------------------------------------------------------------------

def test_softmax_invariants():
    rng = np.random.default_rng(16)
    x = rng.standard_normal((8, 300)) * 8.0
    y = oracle.softmax(x)
    assert np.all(y > 0)
    assert np.allclose(y.sum(axis=1), 1.0, rtol=0, atol=1e-13)
    # order preserving: the same ranking of entries
    assert np.array_equal(np.argsort(x, axis=1, kind="stable"),
                          np.argsort(y, axis=1, kind="stable"))
    # shift invariance, bitwise when the shift is exact (dyadic values)
    xd = np.round(x * 64) / 64
    yd = oracle.softmax(xd)
    assert np.array_equal(yd, oracle.softmax(xd + 1024.0))
    # the normaliser d >= 1 for a row with a finite maximum
    m, d = oracle.softmax_stats(x)
    assert np.all(d >= 1.0)
    assert np.array_equal(m, x.max(axis=1))


def test_softmax_matches_torch_fp64():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(17)
    for (M, N, s) in [(4, 1, 1.0), (3, 7, 3.0), (5, 1024, 8.0), (2, 5000, 30.0)]:
        x = rng.standard_normal((M, N)) * s + 1000.0 * (np.arange(M)[:, None] % 2)
        y = oracle.softmax(x)
        ref = torch.softmax(torch.from_numpy(x), dim=-1).numpy()
        assert np.allclose(y, ref, rtol=1e-12, atol=1e-300), (M, N)


def test_softmax_masked_entries_and_fully_masked_row():
    x = np.array([[0.5, -np.inf, 2.0, -np.inf],
                  [-np.inf, -np.inf, -np.inf, -np.inf],
                  [-np.inf, 3.0, -np.inf, -np.inf]])
    y = oracle.softmax(x)
    assert y[0, 1] == 0.0 and y[0, 3] == 0.0
    assert abs(y[0, 0] - 1 / (1 + math.exp(1.5))) < 1e-15
    assert np.all(np.isnan(y[1]))
    assert np.array_equal(y[2], [0.0, 1.0, 0.0, 0.0])


def test_softmax_no_overflow_at_large_logits():
    # exp(1000) overflows in fp64; only the max-subtracted form stays finite
    y = oracle.softmax(np.array([[1000.0, 1001.0, 999.0, 1e4 - 1e4 + 1000.5]]))
    assert np.all(np.isfinite(y))
    assert abs(y.sum() - 1.0) < 1e-15


def test_log_softmax_pins():
    torch = pytest.importorskip("torch")
    # the pages' example (1000, 1001): y = (0.2689414, 0.7310586), so
    # log y = (-1.3132617, -0.3132617) to the printed precision
    y = oracle.log_softmax(np.array([[1000.0, 1001.0]]))[0]
    assert np.allclose(np.exp(y), [0.2689414, 0.7310586], atol=5e-8)
    assert abs((y[1] - y[0]) - 1.0) < 1e-15
    rng = np.random.default_rng(21)
    x = rng.standard_normal((6, 300)) * 8.0 + 1000.0 * (np.arange(6)[:, None] % 2)
    y = oracle.log_softmax(x)
    ref = torch.log_softmax(torch.from_numpy(x), dim=-1).numpy()
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-12)
    # logsumexp of the output is 0; it equals log of the softmax oracle
    assert np.allclose(np.log(np.exp(y).sum(axis=1)), 0.0, atol=1e-13)
    assert np.allclose(y, np.log(oracle.softmax(x)), rtol=1e-12, atol=1e-12)
    # shift invariance, bitwise for exact shifts of dyadic values
    xd = np.round(x * 64) / 64
    assert np.array_equal(oracle.log_softmax(xd), oracle.log_softmax(xd + 512.0))
    # masked entries give -inf; a fully masked row gives NaN
    z = oracle.log_softmax(np.array([[0.5, -np.inf, 2.0], [-np.inf, -np.inf, -np.inf]]))
    assert z[0, 1] == -np.inf and np.isfinite(z[0, [0, 2]]).all() and np.isnan(z[1]).all()


ALPHABET = [float("-inf"), -2.0, 0.0, 0.5, 3.0, 1000.0]


@pytest.mark.parametrize("length", [1, 2, 3, 4])
def test_online_equals_three_pass_and_every_bracketing(length):
    """Brute force: every row over a small alphabet (with -inf and a +1000
    outlier), the element recurrence, every bracketing of the merge, and the
    three-pass oracle agree on (m, d) and on the probabilities."""
    rows = list(itertools.product(ALPHABET, repeat=length))
    xs = np.array(rows, dtype=np.float64)
    m3, d3 = oracle.softmax_stats(xs)
    y3 = oracle.softmax(xs)
    for i, row in enumerate(rows):
        mo, do = online_ref.online_stats(row)
        finite = any(v != float("-inf") for v in row)
        if not finite:
            assert (mo, do) == online_ref.IDENTITY
            assert np.all(np.isnan(y3[i]))
            assert all(math.isnan(v) for v in online_ref.normalise(row, mo, do))
            continue
        assert mo == m3[i]
        assert abs(do - d3[i]) <= 4e-16 * d3[i], (row, do, d3[i])
        yo = np.array(online_ref.normalise(row, mo, do))
        assert np.allclose(yo, y3[i], rtol=1e-15, atol=0)
        pairs = [online_ref.element_summary(v) for v in row]
        for mb, db in online_ref.all_bracketings(pairs):
            assert mb == m3[i]
            assert abs(db - d3[i]) <= 4e-16 * d3[i], (row, db, d3[i])


def test_merge_identity_and_commutativity():
    rng = np.random.default_rng(18)
    for _ in range(200):
        a = (float(rng.normal() * 10), float(rng.uniform(1, 5)))
        b = (float(rng.normal() * 10), float(rng.uniform(1, 5)))
        assert online_ref.merge(a, online_ref.IDENTITY) == a
        assert online_ref.merge(online_ref.IDENTITY, a) == a
        assert online_ref.merge(a, b) == online_ref.merge(b, a)
        # every rescale factor applied is <= 1
        m = max(a[0], b[0])
        assert math.exp(a[0] - m) <= 1.0 and math.exp(b[0] - m) <= 1.0
