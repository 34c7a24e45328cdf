"""Element-by-element comparison of GPU results with the oracle.

Tolerances (stated for the rotary-embedding apply, arithmetic in binary32 with
fma and one rounding to the storage type):
  float16: |gpu - oracle| <= 1 ulp of the oracle value, where the ulp of a
           binary16 value v is 2^(floor(log2|v|) - 10) for |v| >= 2^-14 and
           2^-24 below (the binary32 result is correctly rounded, so only the
           second rounding to binary16 can differ from the oracle's single
           rounding, by at most one unit).
  bfloat16 (uint16 bit patterns): |gpu - oracle| <= 1 ulp of the oracle value,
           2^(floor(log2|v|) - 7) for |v| >= 2^-126 and 2^-133 below (same
           argument: 8 significant bits instead of 11).
  float32: |gpu - oracle| <= 2e-6 * max(1, |oracle|) (the stated bound; the
           kernels form float32 rotations in binary64 exactly as the oracle
           does, so tests of float32 data also compare bits where that holds).
Pass-through elements (tail, out-of-range pairs) and gathered coefficient
probes are compared bit for bit.
"""
import numpy as np


def bits(a):
    a = np.ascontiguousarray(a)
    return a.view({2: np.uint16, 4: np.uint32, 8: np.uint64}[a.dtype.itemsize])


def values(a):
    """float64 values; uint16 arrays are bfloat16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def ulp_bf16(v):
    a = np.abs(v)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.exp2(e - 7)


def ulp_f16(v):
    a = np.abs(v.astype(np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return np.exp2(e - 10)


def compare(got, want):
    assert got.shape == want.shape and got.dtype == want.dtype, (got.shape, want.shape, got.dtype, want.dtype)
    g = values(got).reshape(-1)
    w = values(want).reshape(-1)
    nan_w = np.isnan(w)
    nan_bad = int(np.count_nonzero(nan_w != np.isnan(g)))
    finite = ~nan_w & ~np.isnan(g)
    diff = np.zeros_like(w)
    with np.errstate(invalid="ignore"):  # inf - inf of equal infinities; cleared below
        diff[finite] = np.abs(g[finite] - w[finite])
    diff[~np.isfinite(diff)] = np.inf
    same_inf = np.isinf(w) & (g == w)
    diff[same_inf] = 0.0
    if got.dtype == np.float16:
        tol = ulp_f16(w)
        ulps = np.where(finite, diff / tol, 0.0)
    elif got.dtype == np.uint16:
        tol = ulp_bf16(w)
        ulps = np.where(finite, diff / tol, 0.0)
    else:
        tol = 2e-6 * np.maximum(1.0, np.abs(w))
        ulps = np.zeros_like(w)
    over = finite & (diff > tol)
    return {
        "n": int(w.size),
        "max_abs": float(diff[finite].max()) if finite.any() else 0.0,
        "max_ulp": float(ulps.max()) if ulps.size else 0.0,
        "n_over_tol": int(np.count_nonzero(over)) + nan_bad,
        "n_bit_diff": int(np.count_nonzero(bits(got).reshape(-1) != bits(want).reshape(-1))),
    }


def assert_parity(got, want, what=""):
    r = compare(got, want)
    assert r["n_over_tol"] == 0, "%s: %s" % (what, r)
    return r


def assert_bitwise(got, want, what=""):
    bg, bw = bits(got).reshape(-1), bits(want).reshape(-1)
    bad = np.flatnonzero(bg != bw)
    assert bad.size == 0, "%s: %d of %d differ bitwise; first at %d: %r vs %r" % (
        what, bad.size, bg.size, bad[0], got.reshape(-1)[bad[0]], want.reshape(-1)[bad[0]])


def ulp_of(want):
    """One unit in the last place of each oracle value in its storage type."""
    v = np.abs(values(want))
    if want.dtype == np.float16:
        return np.exp2(np.floor(np.log2(np.maximum(v, 2.0 ** -14))) - 10)
    if want.dtype == np.uint16:
        return np.exp2(np.floor(np.log2(np.maximum(v, 2.0 ** -126))) - 7)
    return np.exp2(np.floor(np.log2(np.maximum(v, 2.0 ** -126))) - 23)


def assert_parity_norm(got, want, zmax, what=""):
    """QK-norm + RoPE tolerance: |gpu - oracle| <= 1 ulp of the oracle value
    + 2^-18 * zmax, zmax the largest |z_j| = |x_j w_j| / rms of the element's
    head row (broadcast to the output's shape). Worst-case first-order bound
    for the binary32 path, u = 2^-24: the sum of squares has at most ~22
    roundings of positive terms (16 in a lane, log2 W across lanes); the
    mean and epsilon add ~2.5, so the reciprocal square root (v_rsq_f32,
    taken as 2u) is within ~14.3u relative; each rotated term x*(w*c)
    carries 3 more roundings and the scale by 1/rms one, so before the final
    rounding |error| <= ~18.3u * (|z1 c| + |z2 s|) <= ~18.3u * 2 * zmax * 1.25
    ~ 2^-18.5 * zmax for coefficients up to 1.25. The final rounding to the
    storage type adds one unit."""
    g = values(got).reshape(-1)
    w = values(want).reshape(-1)
    tol = ulp_of(want).reshape(-1) + 2.0 ** -18 * np.broadcast_to(zmax, got.shape).reshape(-1)
    bad_nan = np.isnan(g) != np.isnan(w)
    diff = np.abs(g - w)
    over = (diff > tol) & ~np.isnan(w)
    n = int(np.count_nonzero(over)) + int(np.count_nonzero(bad_nan))
    assert n == 0, "%s: %d of %d outside tolerance; max diff/tol %.3g" % (
        what, n, w.size, float(np.nanmax(diff / tol)))
    return {"n": int(w.size), "max_abs": float(np.nanmax(diff)), "max_over_tol": float(np.nanmax(diff / tol))}
