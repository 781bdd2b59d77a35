"""Element-wise comparison of bf16 kernel output with the oracle.

Rule, per element: |gpu - ref16| <= max(ulp16(ref16), 2^-16 * m), where
ref16 is the oracle's binary32 result rounded to bf16 (nearest-even),
ulp16(v) = 2^(floor(log2|v|) - 7) is the bf16 spacing at v's binade (the
smallest subnormal spacing 2^-133 for v = 0 or subnormal v, so zeros must
match up to sign), and m is the oracle's magnitude sum of the two terms an
output is the sum of: |a c| + |b s| for a rotated output, |n (1 + scale)| +
|shift| for a modulated one, m = 0 for plain RMSNorm.  The floor term only
binds where those two terms cancel more than ~8 bits.  NaN must meet NaN.  This is the "1 bf16 ulp against the oracle's binary32 result
rounded to bf16" bar; the derivation of the floor is in the design notes.
"""
from __future__ import annotations

import numpy as np

FLOOR = 2.0 ** -16
MIN_ULP = 2.0 ** -133


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ulp16(v: np.ndarray) -> np.ndarray:
    _, e = np.frexp(np.abs(v))
    u = np.ldexp(1.0, e - 8)
    return np.maximum(u, MIN_ULP)


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
