"""Comparison rules between the GPU results and the fp64 oracle.

Bars (stated once here, used by every parity test):
  * fp32 RMSNorm / fused y: max |g - r| / |r| <= 1e-5, and g == 0 where r == 0.
  * fp32 softmax: max |g - r| <= 2e-6 per probability; every output finite and
    >= 0; masked (-inf) inputs give exactly 0; |sum_j g_j - 1| <= 1e-5 per row;
    rows that are entirely -inf give NaN in every position.
  * bf16 outputs: at most 1 bf16 ulp from the oracle rounded to bf16 (round to
    nearest even), measured as a distance between order-preserving integer
    images of the bit patterns, with +0 and -0 equal.
  * bf16 residual_out of the fused op: bit-exact (the rounded sum is unique).
  * log-softmax: the output is (x - m) - log(d).  The subtraction x - m
    and the final subtraction each round once (relative 2^-24 of their
    results); log(d) carries the relative error of d as an absolute error,
    which is the error the softmax bar allows on a probability near 1.
    fp32: |g - r| <= 4e-6 + 1e-6 |r|; masked (-inf) inputs give exactly
    -inf; fully masked rows give NaN.  bf16 output: at most 1 ulp from
    RNE_bf16(r), or within the fp32 bar (outputs near 0, where a bf16 ulp
    is smaller than the fp32 error of log(d)).
  * LayerNorm (f3): the output is (x - mean) * rstd * gamma + beta, so a
    kernel's error scales with the row's spread, i.e. with |gamma_j| (1 + |z|)
    where z is the normalised value, not with |y| itself (y is near beta for
    x near the mean).  fp32: |g - r| <= 1e-5 (|r| + |gamma_j| + |beta_j|);
    bf16: at most 1 ulp from RNE_bf16(r), or |g - r| <= 1e-5 (|gamma_j| +
    |beta_j|).
"""
import numpy as np

import oracle

# bf16 outputs of LayerNorm and log-softmax that pass only through the fp32
# floor (more than 1 ulp from the oracle rounded to bf16, within the fp32
# bar), and all bf16 outputs of those operations checked, over the session;
# reported in the test summary (tests/conftest.py).
FLOOR_ONLY = {"layernorm": 0, "log_softmax": 0}
FLOOR_CHECKED = {"layernorm": 0, "log_softmax": 0}

RMS_F32_RTOL = 1e-5
SOFTMAX_F32_ATOL = 2e-6
SOFTMAX_ROWSUM_ATOL = 1e-5
BF16_MAX_ULP = 1


def to_f64(t) -> np.ndarray:
    """torch tensor (any device, f32/bf16) -> float64 numpy (exact)."""
    import torch
    return t.detach().to("cpu").to(torch.float64).numpy()


def bf16_bits_of_tensor(t) -> np.ndarray:
    import torch
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def bf16_bits_of_values(v: np.ndarray) -> np.ndarray:
    """fp64 values that are exactly bf16 -> their 16-bit patterns."""
    f = np.ascontiguousarray(v, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def ordered_int(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def bf16_ulp_distance(got_bits: np.ndarray, ref_bits: np.ndarray) -> np.ndarray:
    return np.abs(ordered_int(got_bits) - ordered_int(ref_bits))


def check_bf16(got_tensor, ref_f64: np.ndarray, what: str, max_ulp: int = BF16_MAX_ULP):
    """got: bf16 tensor; ref: fp64 oracle values (rounded here to bf16)."""
    ref_bits = bf16_bits_of_values(oracle.round_bf16(ref_f64))
    got_bits = bf16_bits_of_tensor(got_tensor).reshape(ref_bits.shape)
    ref_nan = np.isnan(ref_f64)
    got_f = to_f64(got_tensor).reshape(ref_f64.shape)
    assert np.array_equal(np.isnan(got_f), ref_nan), f"{what}: NaN pattern differs"
    fin = ~ref_nan
    dist = bf16_ulp_distance(got_bits[fin], ref_bits[fin])
    worst = int(dist.max()) if dist.size else 0
    assert worst <= max_ulp, f"{what}: {worst} bf16 ulp (> {max_ulp}); count>0: {int((dist > 0).sum())}"
    return {"max_ulp": worst, "n_1ulp": int((dist == 1).sum()), "n": int(dist.size)}


def check_bf16_exact(got_tensor, ref_f64: np.ndarray, what: str):
    return check_bf16(got_tensor, ref_f64, what, max_ulp=0)


def check_rms_f32(got_tensor, ref_f64: np.ndarray, what: str):
    g = to_f64(got_tensor).reshape(ref_f64.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    zero = ref_f64 == 0.0
    assert np.all(g[zero] == 0.0), f"{what}: nonzero where the oracle is 0"
    nz = ~zero
    rel = np.abs(g[nz] - ref_f64[nz]) / np.abs(ref_f64[nz])
    worst = float(rel.max()) if rel.size else 0.0
    assert worst <= RMS_F32_RTOL, f"{what}: max rel err {worst:.3e} > {RMS_F32_RTOL}"
    return {"max_rel": worst}


def check_softmax(got_tensor, x_f64: np.ndarray, ref_f64: np.ndarray, what: str):
    """Softmax bars; dispatches on the output dtype."""
    import torch
    M = ref_f64.shape[0]
    nan_rows = np.all(np.isneginf(x_f64), axis=1)
    if got_tensor.dtype == torch.bfloat16:
        info = check_bf16(got_tensor, ref_f64, what)
        g = to_f64(got_tensor).reshape(ref_f64.shape)
    else:
        g = to_f64(got_tensor).reshape(ref_f64.shape)
        ok = ~nan_rows
        if ok.any():
            err = np.abs(g[ok] - ref_f64[ok])
            worst = float(err.max())
            assert worst <= SOFTMAX_F32_ATOL, f"{what}: max abs err {worst:.3e} > {SOFTMAX_F32_ATOL}"
        else:
            worst = 0.0
        info = {"max_abs": worst}
    # properties that hold whatever the dtype
    if nan_rows.any():
        assert np.all(np.isnan(g[nan_rows])), f"{what}: fully masked rows must be NaN"
    ok = ~nan_rows
    gk = g[ok]
    assert np.all(np.isfinite(gk)), f"{what}: non-finite probability"
    assert np.all(gk >= 0.0), f"{what}: negative probability"
    masked = np.isneginf(x_f64[ok])
    assert np.all(gk[masked] == 0.0), f"{what}: masked entry not exactly 0"
    if got_tensor.dtype != torch.bfloat16 and gk.size:
        rs = np.abs(gk.sum(axis=1) - 1.0)
        assert rs.max() <= SOFTMAX_ROWSUM_ATOL, f"{what}: row sum off by {rs.max():.3e}"
        info["max_rowsum_err"] = float(rs.max())
    info["rows"] = M
    return info


LN_TOL = 1e-5


def check_layernorm(got_tensor, ref_f64: np.ndarray, gamma_f64: np.ndarray, beta_f64, what: str):
    import torch
    g = to_f64(got_tensor).reshape(ref_f64.shape)
    scale = np.abs(gamma_f64)[None, :] + (np.abs(beta_f64)[None, :] if beta_f64 is not None else 0.0)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    if got_tensor.dtype == torch.bfloat16:
        ref_bits = bf16_bits_of_values(oracle.round_bf16(ref_f64))
        got_bits = bf16_bits_of_tensor(got_tensor).reshape(ref_bits.shape)
        dist = bf16_ulp_distance(got_bits, ref_bits)
        floor_ok = np.abs(g - ref_f64) <= LN_TOL * scale
        bad = (dist > BF16_MAX_ULP) & ~floor_ok
        assert not bad.any(), f"{what}: {int(bad.sum())} outputs beyond 1 ulp and the floor"
        n_floor = int(((dist > BF16_MAX_ULP) & floor_ok).sum())
        FLOOR_ONLY["layernorm"] += n_floor
        FLOOR_CHECKED["layernorm"] += int(dist.size)
        return {"max_ulp": int(dist.max()), "n_floor": n_floor}
    err = np.abs(g - ref_f64) / (np.abs(ref_f64) + scale)
    worst = float(err.max())
    assert worst <= LN_TOL, f"{what}: scaled error {worst:.3e} > {LN_TOL}"
    return {"max_scaled_err": worst}


LOGSM_ATOL = 4e-6
LOGSM_RTOL = 1e-6


def check_log_softmax(got_tensor, x_f64: np.ndarray, ref_f64: np.ndarray, what: str):
    import torch
    g = to_f64(got_tensor).reshape(ref_f64.shape)
    nan_rows = np.all(np.isneginf(x_f64), axis=1)
    if nan_rows.any():
        assert np.all(np.isnan(g[nan_rows])), f"{what}: fully masked rows must be NaN"
    ok = ~nan_rows
    gk, rk, xk = g[ok], ref_f64[ok], x_f64[ok]
    masked = np.isneginf(xk)
    assert np.all(np.isneginf(gk[masked])), f"{what}: masked entry not exactly -inf"
    kept = ~masked
    gv, rv = gk[kept], rk[kept]
    assert np.all(np.isfinite(gv)), f"{what}: non-finite log-probability"
    bar = LOGSM_ATOL + LOGSM_RTOL * np.abs(rv)
    err = np.abs(gv - rv)
    if got_tensor.dtype == torch.bfloat16:
        ref_bits = bf16_bits_of_values(oracle.round_bf16(rv))
        got_bits = bf16_bits_of_tensor(got_tensor).reshape(ref_f64.shape)[ok][kept]
        dist = bf16_ulp_distance(got_bits, ref_bits)
        bad = (dist > BF16_MAX_ULP) & (err > bar)
        assert not bad.any(), f"{what}: {int(bad.sum())} outputs beyond 1 ulp and the fp32 bar"
        n_floor = int((dist > BF16_MAX_ULP).sum())
        FLOOR_ONLY["log_softmax"] += n_floor
        FLOOR_CHECKED["log_softmax"] += int(dist.size)
        return {"max_ulp": int(dist.max()) if dist.size else 0, "n_floor": n_floor,
                "rows": int(ref_f64.shape[0])}
    worst = float((err / bar).max()) if err.size else 0.0
    assert worst <= 1.0, f"{what}: error {worst:.3f} x the bar (max abs {float(err.max()):.3e})"
    # exp of the output is the softmax: its rows sum to 1
    rs = np.abs(np.exp(gk).sum(axis=1) - 1.0)
    if rs.size:
        assert rs.max() <= SOFTMAX_ROWSUM_ATOL, f"{what}: exp rows sum off by {rs.max():.3e}"
    return {"max_abs": float(err.max()) if err.size else 0.0, "rows": int(ref_f64.shape[0])}
