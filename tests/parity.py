"""Element-wise comparison of kernel output with the oracle, for bf16, fp16
and fp32 outputs.

Each report gives the largest error in output ulps over all elements
("max_ulp") and over those the floor does not cover ("max_ulp_outside_floor"),
and the largest ratio of error to tolerance ("max_tol_ratio", at most 1 for a
pass).

Rule, per element: |gpu - ref16| <= max(ulp16(ref16), 2^-16 * m), where
ref16 is the oracle's binary32 result rounded to bf16 (nearest-even),
ulp16(v) = 2^(floor(log2|v|) - 7) is the bf16 spacing at v's binade (the
smallest subnormal spacing 2^-133 for v = 0 or subnormal v, so zeros must
match up to sign), and m is the oracle's magnitude sum of the two terms an
output is the sum of: |a c| + |b s| for a rotated output, |n (1 + scale)| +
|shift| for a modulated one, m = 0 for plain RMSNorm.  The floor term only
binds where those two terms cancel more than ~8 bits.  NaN must meet NaN.

fp16 outputs use the same rule with the binary16 spacing 2^(floor(log2|v|)
- 10) (2^-24 for subnormals).  fp32 outputs are the kernel's own binary32
result, so the bound is the evaluation error itself: |gpu - ref32| <=
F32_REL * (|ref32| + m) with F32_REL = 2^-20, 16 units of 2^-24.  The sum of
squares is the only long chain: at most 32 binary32 terms per lane, a
6-level tree and up to 16 cross-wavefront partials; rows beyond the
register budget are summed in chunks of 2048 vectors (8 terms per lane, a
tree, 4 partials) whose sums are added 33 at most per lane and by a second
tree.  With round-to-nearest errors of either sign its relative error is a
few units of 2^-24; the square root halves it, and the scaling, rotation or
modulation adds at most three roundings.  The largest error measured over full-size
workloads is 4 units (RMSNorm) and 3 units of |ref32| + m (RoPE, AdaLN), so
the bound keeps a margin of four while an evaluation ten times less accurate
fails.  This is the "1 bf16 ulp against the oracle's binary32 result rounded
to bf16" bar; the derivation of the floor is in the design notes.
"""
from __future__ import annotations

import numpy as np

FLOOR = 2.0 ** -16
MIN_ULP = 2.0 ** -133
F32_REL = 2.0 ** -20


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ulp16(v: np.ndarray) -> np.ndarray:
    _, e = np.frexp(np.abs(v))
    u = np.ldexp(1.0, e - 8)
    return np.maximum(u, MIN_ULP)


def ulp_f16(v: np.ndarray) -> np.ndarray:
    _, e = np.frexp(np.abs(v))
    return np.maximum(np.ldexp(1.0, e - 11), 2.0 ** -24)


def compare(got, ref, mag=None, ref32=None) -> dict:
    """Compare kernel output `got` with the oracle's rounded output `ref`:
    uint16 arrays are bf16 bit patterns, float16 and float32 arrays values."""
    ref = np.asarray(ref)
    if ref.dtype == np.uint16:
        return compare_bf16(got, ref, mag, ref32)
    got = np.asarray(got, dtype=ref.dtype).reshape(-1)
    ref = ref.reshape(-1)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    g = got.astype(np.float64)
    r = ref.astype(np.float64)
    m = np.zeros_like(r) if mag is None else np.asarray(mag, dtype=np.float64).reshape(-1)
    gnan, rnan = np.isnan(g), np.isnan(r)
    both = ~(gnan | rnan)
    with np.errstate(invalid="ignore"):
        diff = np.where(both & (g != r), np.abs(g - r), 0.0)  # inf == inf is a match
    if ref.dtype == np.float16:
        u = ulp_f16(np.where(both, r, 1.0))
        tol = np.maximum(u, FLOOR * m)
    else:
        u = np.maximum(np.abs(np.spacing(np.where(both, r, 1.0).astype(np.float32))).astype(np.float64),
                       2.0 ** -149)
        tol = F32_REL * (np.abs(np.where(both, r, 0.0)) + m)
        tol = np.maximum(tol, 2.0 ** -149)
    bad = (diff > tol) | (gnan != rnan)
    # elements that pass only thanks to the magnitude term m
    own = u if ref.dtype == np.float16 else F32_REL * np.abs(np.where(both, r, 0.0))
    floor_bound = (diff > own) & (diff <= tol)
    rep = {"n": int(g.size), "pass": bool(not bad.any()), "n_bad": int(bad.sum()),
           "n_exact": int((g == r).sum() + (gnan & rnan).sum()),
           "max_ulp": float((diff / u).max()) if diff.size else 0.0,
           "max_ulp_outside_floor": float(np.where(floor_bound, 0.0, diff / u).max()) if diff.size else 0.0,
           "max_tol_ratio": float((diff / tol).max()) if diff.size else 0.0,
           "n_floor_bound": int(floor_bound.sum())}
    if ref32 is not None:
        r32 = np.asarray(ref32, dtype=np.float32).reshape(-1).astype(np.float64)
        ok = both & ~np.isnan(r32) & np.isfinite(g)
        rep["max_abs_err"] = float(np.abs(g[ok] - r32[ok]).max()) if ok.any() else 0.0
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        rep["first_bad"] = {"index": i, "got": float(g[i]), "ref": float(r[i]), "tol": float(tol[i])}
    return rep


def compare_bf16(got_bits, ref16, mag=None, ref32=None) -> dict:
    got_bits = np.asarray(got_bits, dtype=np.uint16).reshape(-1)
    ref16 = np.asarray(ref16, dtype=np.uint16).reshape(-1)
    assert got_bits.shape == ref16.shape, (got_bits.shape, ref16.shape)
    g = bf16_to_f64(got_bits)
    r = bf16_to_f64(ref16)
    gnan, rnan = np.isnan(g), np.isnan(r)
    both = ~(gnan | rnan)
    with np.errstate(invalid="ignore"):
        diff = np.where(both, np.abs(g - r), 0.0)
    u = ulp16(np.where(both, r, 1.0))
    tol = u
    floor_bound = np.zeros_like(diff, dtype=bool)
    if mag is not None:
        fl = FLOOR * np.asarray(mag, dtype=np.float64).reshape(-1)
        floor_bound = (diff > u) & (diff <= fl)
        tol = np.maximum(u, fl)
    bad = (diff > tol) | (gnan != rnan)
    rep = {
        "n": int(got_bits.size),
        "pass": bool(not bad.any()),
        "n_bad": int(bad.sum()),
        "n_bit_exact": int((got_bits == ref16).sum()),
        "max_ulp": float((diff / u).max()) if diff.size else 0.0,
        "max_ulp_outside_floor": float(np.where(floor_bound, 0.0, diff / u).max()) if diff.size else 0.0,
        "max_tol_ratio": float((diff / tol).max()) if diff.size else 0.0,
        "n_floor_bound": int(floor_bound.sum()),
    }
    if ref32 is not None:
        r32 = np.asarray(ref32, dtype=np.float32).reshape(-1).astype(np.float64)
        ok = both & ~np.isnan(r32)
        rep["max_abs_err"] = float(np.abs(g[ok] - r32[ok]).max()) if ok.any() else 0.0
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        rep["first_bad"] = {"index": i, "got": float(g[i]), "ref16": float(r[i]),
                            "tol": float(tol[i])}
    return rep
