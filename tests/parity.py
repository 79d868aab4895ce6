"""Parity rules between the HIP path and the fp64 oracle.

Codes and sign bits: bit-exact, except that a coordinate may differ when the
oracle's rotated, normalised value lies within 1e-5 of a decision boundary
(codes; 1e-5 * ||x|| at input scale) or when the oracle's sketch value
|z| <= 1e-5 (signs); such differences must number at most 1e-5 of all code
and sign coordinates.  A differing code must be a neighbouring cell.  Sign
bits, residual norms and logits are judged against the oracle recomputed
with the GPU's codes, so that one boundary flip is not counted twice.

Norms: ||x|| within 1e-6 relative (float32), or (float16) equal, or one ulp
apart only where the fp64 value is within 1e-6 relative of a float16
rounding midpoint.  ||x|| ||r||: the same with 1e-5 -- the residual is the
rotated coordinate minus its centroid, so the rotation's float32-grade
error (about 2^-22 of ||y^|| = 1 per coordinate) is an absolute error on
r^, and relative to ||r^|| (about 0.1 for 4-bit codes, 0.34 for 2-bit) it
grows to about 2.5e-6 at 4 bits; 1e-5 leaves a 4x margin.

Logits: |gpu - ref| <= 1e-4 + 1e-3 |ref| elementwise.  Decode: per
(batch, head) row, ||gpu - ref||_2 <= 2e-3 ||ref||_2.
"""

import numpy as np

import oracle

BAND = 1e-5
MAX_MISMATCH_FRACTION = 1e-5


def _f16_ok(gpu16, ref64, rel_window):
    """gpu16: float16 array; ref64: fp64 reference values."""
    ref16 = ref64.astype(np.float16)
    eq = gpu16 == ref16
    if np.all(eq):
        return True, 0
    bad = ~eq
    g = gpu16[bad].astype(np.float64)
    r = ref64[bad]
    r16 = ref16[bad].astype(np.float64)
    # the neighbour on the other side of r
    other = np.where(g > r16, np.nextafter(ref16[bad], np.float16(np.inf)),
                     np.nextafter(ref16[bad], np.float16(-np.inf))).astype(np.float64)
    one_ulp = np.isclose(g, other, rtol=0, atol=0)
    mid = 0.5 * (r16 + other)
    near_mid = np.abs(r - mid) <= rel_window * np.abs(r)
    ok = one_ulp & near_mid
    return bool(np.all(ok)), int(np.sum(~ok))


def check_norms(gpu, ref, dtype, rtol32):
    gpu = np.asarray(gpu)
    ref = np.asarray(ref, dtype=np.float64)
    if dtype == "f32":
        err = np.abs(gpu.astype(np.float64) - ref)
        ok = err <= rtol32 * np.abs(ref) + 1e-30
        return bool(np.all(ok)), float(np.max(err / np.maximum(np.abs(ref), 1e-30), initial=0.0))
    ok, nbad = _f16_ok(gpu.astype(np.float16), ref, rtol32)
    return ok, nbad


def check_key_stream(X, idx_gpu, signs_gpu, norm_gpu, rnorm_gpu, Pi, S, c, t, norm_dtype):
    """X [n, d] fp64 inputs (exact values); idx_gpu [n, d] ints; signs_gpu [n, m]
    bools; norms as stored.  Returns a report dict; 'ok' is the verdict."""
    # the keys' first stage is the values' quantizer; the sketch is computed
    # once, from the GPU's codes (the oracle's own codes only gate the codes)
    ref = oracle.quantize_values(X, Pi, c, t)
    rep = _check_codes(ref, idx_gpu, t)
    with_gpu = oracle.residual_and_sketch(ref["yhat"], idx_gpu, c, S, ref["norm"])
    sdiff = signs_gpu != with_gpu["signs"]
    s_inband = np.abs(with_gpu["z"]) <= BAND
    rep["sign_mismatch"] = int(np.sum(sdiff))
    rep["sign_mismatch_out_of_band"] = int(np.sum(sdiff & ~s_inband))
    total = idx_gpu.size + signs_gpu.size
    rep["mismatch_fraction"] = (rep["code_mismatch"] + rep["sign_mismatch"]) / total
    ok_n, en = check_norms(norm_gpu, ref["norm"], norm_dtype, 1e-6)
    ok_r, er = check_norms(rnorm_gpu, with_gpu["rnorm"], norm_dtype, 1e-5)
    rep.update(norm_ok=ok_n, norm_err=en, rnorm_ok=ok_r, rnorm_err=er)
    rep["ok"] = (rep["codes_ok"] and rep["sign_mismatch_out_of_band"] == 0
                 and rep["mismatch_fraction"] <= MAX_MISMATCH_FRACTION and ok_n and ok_r)
    return rep


def check_value_stream(X, idx_gpu, norm_gpu, Pi, c, t, norm_dtype):
    ref = oracle.quantize_values(X, Pi, c, t)
    rep = _check_codes(ref, idx_gpu, t)
    rep["mismatch_fraction"] = rep["code_mismatch"] / idx_gpu.size
    ok_n, en = check_norms(norm_gpu, ref["norm"], norm_dtype, 1e-6)
    rep.update(norm_ok=ok_n, norm_err=en)
    rep["ok"] = rep["codes_ok"] and rep["mismatch_fraction"] <= MAX_MISMATCH_FRACTION and ok_n
    return rep


def _check_codes(ref, idx_gpu, t):
    diff = idx_gpu != ref["idx"]
    dist = np.full(ref["yhat"].shape, np.inf)
    t = np.asarray(t, dtype=np.float64)
    # distance to the nearest boundary (t: one codebook's boundaries, or one
    # row per coordinate for a split width, padded with +inf)
    for ti in (t if t.ndim == 1 else t.T):
        dist = np.minimum(dist, np.abs(ref["yhat"] - ti))
    inband = dist <= BAND
    neighbour = np.abs(idx_gpu - ref["idx"]) <= 1
    return dict(code_mismatch=int(np.sum(diff)),
                code_mismatch_out_of_band=int(np.sum(diff & ~(inband & neighbour))),
                codes_ok=bool(np.sum(diff & ~(inband & neighbour)) == 0))


def logits_close(gpu, ref, atol=1e-4, rtol=1e-3):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bad = np.abs(gpu - ref) > atol + rtol * np.abs(ref)
    return (not bool(np.any(bad))), int(np.sum(bad)), float(np.max(np.abs(gpu - ref), initial=0.0))


def decode_close(gpu, ref, rtol=2e-3):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.linalg.norm(gpu - ref, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    rel = num / np.maximum(den, 1e-300)
    return bool(np.all(rel <= rtol)), float(np.max(rel, initial=0.0))
