"""Pins for the CPU oracle: checks against facts that do not come from the
oracle itself (closed forms, invariants, textbook routines, exact arithmetic
on tiny inputs).  Each pin is a function taking an ``oracle.Oracle`` and
raising AssertionError on failure, so the same pins run against the real
oracle (test_oracle_pins.py) and against copies with planted mistakes
(test_oracle_mutants.py), which every pin set must reject.

What is being pinned: RMSNorm over the innermost dimension with an optional
weight and eps default 1e-6 (Hugging Face cuda-kernels skill page, section
"Kernel-Specific Guidelines", RMSNorm), read as
y = x / sqrt(mean(x^2) + eps) * w; and rms_norm_rope (LTX-2 ltx-kernels
README, introduction) read as that RMSNorm followed by rotate-half RoPE per
head over the 1D [batch, seq, heads, head_dim] layout (skill page, RoPE).
"""
from __future__ import annotations

import cmath
import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np

import datagen

EPS32 = float(np.float32(1e-6))  # the binary32 epsilon both sides actually use


def _bf16(vals) -> np.ndarray:
    """Exact bf16 bit patterns for values that are exactly representable."""
    f = np.asarray(vals, dtype=np.float32)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exactly representable in bf16"
    return (u >> 16).astype(np.uint16)


def _val(bits) -> np.ndarray:
    return datagen.bf16_bits_to_f32(bits).astype(np.float64)


def _rand_bf16(rng, shape, scale=1.0):
    return datagen.to_bf16_bits(rng.standard_normal(shape) * scale)


# --------------------------------------------------------------------------
# RMSNorm pins
# --------------------------------------------------------------------------

def pin_eps_inside_root(o):
    """Constant row c = 2^-10, no weight, eps = 1e-6 (binary32).  mean(x^2) is
    c^2 = 2^-20, so y = c / sqrt(2^-20 + eps32) = 0.698672999...  (eps added
    outside the root would give 0.998977, a sum instead of a mean 0.123988)."""
    x = _bf16(np.full((2, 64), 2.0 ** -10))
    y = o.rmsnorm(x, None, 1e-6)
    # 2^-10 / sqrt(2^-20 + 9.999999974752427e-07), evaluated at 40 digits
    # with Python's decimal module
    expected = 0.69867299943694822
    assert np.allclose(y, expected, rtol=1e-13, atol=0), (y[0, 0], expected)


def pin_constant_row_gives_weight(o):
    """Constant row c with |c| >= 0.1: eps shifts rstd by < 5e-5 relative,
    below half a bf16 ulp, so the bf16 output is exactly sign(c) * w."""
    rng = np.random.default_rng(11)
    w = datagen.to_bf16_bits(rng.uniform(0.5, 1.5, 96))
    for c in (0.125, -0.5, 3.0, -96.0, 0.1015625):
        x = _bf16(np.full((3, 96), c, dtype=np.float32))
        _, ref16 = o.round(o.rmsnorm(x, w, 1e-6))
        want = w if c > 0 else (w ^ np.uint16(0x8000))
        assert np.array_equal(ref16, np.broadcast_to(want, ref16.shape)), c


def pin_constant_row_small_value(o):
    """Constant row c = 0.01 (bf16 0.010009765625), unit weight: y =
    c / sqrt(c^2 + eps32), a closed form that depends on eps at 0.5 %."""
    c = float(np.float32(datagen.bf16_bits_to_f32(datagen.to_bf16_bits(np.array([0.01])))[0]))
    assert c == 0.010009765625
    x = _bf16(np.full((1, 32), c))
    y = o.rmsnorm(x, None, 1e-6)
    # c^2 = 1.00195407867431640625e-04 (exact), + eps32 = 1.0119540786490688e-04,
    # sqrt = 1.0059592827987964e-02, so y = 0.99504679723722674 (40 digits)
    assert np.allclose(y, 0.99504679723722674, rtol=1e-14, atol=0)


def pin_zero_row(o):
    """A zero row normalises to exact zeros (rstd = 1/sqrt(eps) is finite),
    and zero elements in a nonzero row give zero outputs."""
    rng = np.random.default_rng(3)
    x = _rand_bf16(rng, (4, 40))
    x[1] = 0
    x[2, ::3] = 0
    y = o.rmsnorm(x, datagen.to_bf16_bits(rng.uniform(0.5, 1.5, 40)), 1e-6)
    assert np.all(y[1] == 0.0)
    assert np.all(y[2, ::3] == 0.0)
    assert np.all(np.isfinite(y))


def pin_scale_invariance(o):
    """With eps = 0, x -> 2^k x leaves the output bit-identical (powers of two
    scale exactly; the norm divides them out)."""
    rng = np.random.default_rng(5)
    x = _rand_bf16(rng, (5, 72))
    w = datagen.to_bf16_bits(rng.uniform(0.5, 1.5, 72))
    base = o.rmsnorm(x, w, 0.0)
    for k in (-8, -3, 1, 4, 8):
        xs = datagen.to_bf16_bits(_val(x) * 2.0 ** k)
        assert np.array_equal(o.rmsnorm(xs, w, 0.0), base), k


def pin_sign_symmetry(o):
    """y(-x) = -y(x) exactly."""
    rng = np.random.default_rng(7)
    x = _rand_bf16(rng, (3, 50))
    w = datagen.to_bf16_bits(rng.uniform(0.5, 1.5, 50))
    assert np.array_equal(o.rmsnorm(x ^ np.uint16(0x8000), w, 1e-6), -o.rmsnorm(x, w, 1e-6))


def pin_textbook_norm(o):
    """Unit weight, eps = 0: y = sqrt(H) * x / ||x||_2 with the Euclidean
    norm from numpy.linalg.norm."""
    rng = np.random.default_rng(9)
    for hidden in (1, 7, 64, 3072):
        x = _rand_bf16(rng, (3, hidden))
        xv = _val(x)
        want = math.sqrt(hidden) * xv / np.linalg.norm(xv, axis=1, keepdims=True)
        assert np.allclose(o.rmsnorm(x, None, 0.0), want, rtol=1e-13, atol=0), hidden


def pin_none_weight_is_ones(o):
    """An absent weight behaves exactly as a weight of ones (skill page,
    section "Diffusers Critical Pitfalls", item 1)."""
    rng = np.random.default_rng(13)
    x = _rand_bf16(rng, (4, 24))
    ones = _bf16(np.ones(24))
    assert np.array_equal(o.rmsnorm(x, None, 1e-6), o.rmsnorm(x, ones, 1e-6))


def pin_rows_independent(o):
    """Each row depends only on itself: any subset of rows gives the same
    values as the full call."""
    rng = np.random.default_rng(17)
    x = _rand_bf16(rng, (9, 32))
    w = datagen.to_bf16_bits(rng.uniform(0.5, 1.5, 32))
    full = o.rmsnorm(x, w, 1e-6)
    for sel in ([4], [0, 8], [2, 3, 5]):
        assert np.array_equal(o.rmsnorm(x[sel], w, 1e-6), full[sel])


def pin_permutation(o):
    """Permuting the elements of x and w together permutes y (up to the
    rounding of the sum in a different order)."""
    rng = np.random.default_rng(19)
    x = _rand_bf16(rng, (3, 48))
    w = datagen.to_bf16_bits(rng.uniform(0.5, 1.5, 48))
    perm = rng.permutation(48)
    a = o.rmsnorm(x, w, 1e-6)[:, perm]
    b = o.rmsnorm(x[:, perm], w[perm], 1e-6)
    assert np.allclose(a, b, rtol=1e-14, atol=0)


def _exact_rms_row(xv, wv, eps):
    """Exact sum of squares with fractions, root and products at 60 digits."""
    getcontext().prec = 60
    ss = sum(Fraction(v) * Fraction(v) for v in xv)
    ms = ss / len(xv) + Fraction(eps)
    ms_dec = Decimal(ms.numerator) / Decimal(ms.denominator)
    rstd = 1 / ms_dec.sqrt()
    return [Decimal(v) * rstd * Decimal(wj) for v, wj in zip(xv, wv)]


def pin_brute_force_exact(o):
    """Tiny rows, random and adversarial (mixed magnitudes, magnitudes so
    small that eps dominates, a single nonzero) against exact rational /
    60-digit arithmetic: the double result within (H + 8) * 2^-53 relative
    (H rounded additions plus a few rounded operations), and the binary32
    reference within one binary32 ulp of the exact value."""
    rng = np.random.default_rng(23)
    rows = []
    for hidden in (1, 2, 3, 7, 8, 16, 64):
        rows.append(_rand_bf16(rng, (hidden,)))
        rows.append(_rand_bf16(rng, (hidden,), scale=1e-5))
        mixed = rng.standard_normal(hidden) * np.where(rng.random(hidden) < 0.2, 300.0, 1e-3)
        rows.append(datagen.to_bf16_bits(mixed))
        single = np.zeros(hidden)
        single[hidden // 2] = -2.5
        rows.append(datagen.to_bf16_bits(single))
    for x in rows:
        hidden = x.size
        w = datagen.to_bf16_bits(rng.uniform(0.5, 1.5, hidden))
        xv, wv = _val(x), _val(w)
        exact = _exact_rms_row(xv, wv, EPS32)
        y = o.rmsnorm(x[None, :], w, 1e-6)[0]
        ref32, _ = o.round(y)
        for j in range(hidden):
            e = exact[j]
            if e == 0:
                assert y[j] == 0.0
                continue
            tol = Decimal((hidden + 8) * 2.0 ** -53)
            assert abs(Decimal(y[j]) - e) <= abs(e) * tol, (hidden, j, y[j], e)
            f = np.float32(float(e))
            ulp = np.spacing(np.float32(abs(f)))
            assert abs(float(ref32[j]) - float(e)) <= float(ulp), (hidden, j)


# --------------------------------------------------------------------------
# RMSNorm + RoPE pins
# --------------------------------------------------------------------------

def _tables(positions, head_dim, theta=10000.0):
    return datagen.rope_tables(0, head_dim, theta, positions=np.asarray(positions))


def pin_rope_position_zero_is_rmsnorm(o):
    """cos = 1, sin = 0 rotates by nothing: RMSNorm+RoPE at position 0 is the
    plain RMSNorm, exactly."""
    rng = np.random.default_rng(29)
    heads, d = 4, 16
    x = _rand_bf16(rng, (3, heads * d))
    w = datagen.to_bf16_bits(rng.uniform(0.5, 1.5, heads * d))
    c, s = _tables([0], d)
    assert np.all(c == 1.0) and np.all(s == 0.0)
    y = o.rmsnorm_rope(x, w, c, s, heads, d, 1e-6)
    assert np.array_equal(y, o.rmsnorm(x, w, 1e-6))


def pin_rope_complex_rotation(o):
    """Each rotate-half pair (i, i + d/2) is the complex number a + ib turned
    by the unit phasor c + is (Python complex multiplication); checked against
    RMSNorm from the same oracle for the un-rotated values."""
    rng = np.random.default_rng(31)
    heads, d, seq = 3, 8, 5
    x = _rand_bf16(rng, (seq, heads * d))
    w = datagen.to_bf16_bits(rng.uniform(0.5, 1.5, heads * d))
    c, s = _tables(np.arange(seq), d)
    y = o.rmsnorm_rope(x, w, c, s, heads, d, 1e-6)
    z = o.rmsnorm(x, w, 1e-6)
    for r in range(seq):
        for h in range(heads):
            for i in range(d // 2):
                a, b = z[r, h * d + i], z[r, h * d + i + d // 2]
                rot = complex(a, b) * complex(float(c[r, i]), float(s[r, i]))
                assert cmath.isclose(complex(y[r, h * d + i], y[r, h * d + i + d // 2]), rot,
                                     rel_tol=1e-14, abs_tol=1e-300), (r, h, i)


def pin_rope_pair_norm(o):
    """The rotation preserves each pair's norm: o1^2 + o2^2 = (a^2 + b^2)(c^2 + s^2)."""
    rng = np.random.default_rng(37)
    heads, d = 2, 32
    x = _rand_bf16(rng, (6, heads * d))
    c, s = _tables(np.arange(6) * 37, d)
    y = o.rmsnorm_rope(x, None, c, s, heads, d, 1e-6)
    z = o.rmsnorm(x, None, 1e-6)
    hd = d // 2
    for h in range(heads):
        a, b = z[:, h * d:h * d + hd], z[:, h * d + hd:(h + 1) * d]
        o1, o2 = y[:, h * d:h * d + hd], y[:, h * d + hd:(h + 1) * d]
        cc, ss = c.astype(np.float64), s.astype(np.float64)
        assert np.allclose(o1 ** 2 + o2 ** 2, (a ** 2 + b ** 2) * (cc ** 2 + ss ** 2), rtol=1e-13, atol=1e-300)


def pin_rope_constant_row(o):
    """Constant positive x and unit weight normalise to exactly 1 (in double,
    up to eps); the output is then cos - sin in the first half of each head and
    cos + sin in the second half."""
    heads, d = 2, 16
    x = _bf16(np.full((3, heads * d), 0.75))
    c, s = _tables([1, 2, 9], d)
    y = o.rmsnorm_rope(x, None, c, s, heads, d, 0.0)
    cc, ss = c.astype(np.float64), s.astype(np.float64)
    for h in range(heads):
        assert np.allclose(y[:, h * d:h * d + d // 2], cc - ss, rtol=1e-15, atol=1e-15)
        assert np.allclose(y[:, h * d + d // 2:(h + 1) * d], cc + ss, rtol=1e-15, atol=1e-15)


def pin_rope_row_position(o):
    """Row r uses table row r mod seq_len: each row alone, given a one-row
    table holding just that position, gives the same result."""
    rng = np.random.default_rng(41)
    heads, d, seq = 2, 8, 3
    x = _rand_bf16(rng, (8, heads * d))
    w = datagen.to_bf16_bits(rng.uniform(0.5, 1.5, heads * d))
    c, s = _tables([5, 11, 17], d)
    y = o.rmsnorm_rope(x, w, c, s, heads, d, 1e-6)
    for r in range(8):
        p = [0, 1, 2][r % seq]
        yr = o.rmsnorm_rope(x[r:r + 1], w, c[p:p + 1], s[p:p + 1], heads, d, 1e-6)
        assert np.array_equal(yr[0], y[r]), r


def pin_rope_composition(o):
    """Rotations compose: turning a normalised row by position p1's table and
    the result by p2's equals one turn by p1 + p2, since each pair's angle is
    linear in the position (inv_freq_i * p), in both pairings.  The
    intermediate row passes through binary32 (the oracle's input type) and
    the tables are binary32 values, so agreement is to about 1e-6; the single
    turns differ by far more."""
    rng = np.random.default_rng(53)
    heads, d = 3, 16
    x = rng.standard_normal((2, heads * d)).astype(np.float32)
    for il in (False, True):
        for p1, p2 in ((3, 5), (100, 17)):
            c, s = _tables([p1, p2, p1 + p2], d)
            y1 = o.rmsnorm_rope(x, None, c[0:1], s[0:1], heads, d, 0.0, interleaved=il)
            y2 = o.rmsnorm_rope(y1.astype(np.float32), None, c[1:2], s[1:2], heads, d, 0.0, interleaved=il)
            y12 = o.rmsnorm_rope(x, None, c[2:3], s[2:3], heads, d, 0.0, interleaved=il)
            assert np.abs(y2 - y12).max() <= 4e-6, (il, p1, p2, np.abs(y2 - y12).max())
            assert np.abs(y1 - y12).max() > 1e-2, (il, p1, p2)


def pin_rope_mag(o):
    """The magnitude sum returned with the rotation is |a c| + |b s| (first
    half) and |b c| + |a s| (second half): it bounds the rotated value and
    equals its magnitude when the two products do not cancel."""
    rng = np.random.default_rng(43)
    heads, d = 2, 8
    x = _rand_bf16(rng, (4, heads * d))
    c, s = _tables([1, 2, 3, 4], d)
    y, mag = o.rmsnorm_rope(x, None, c, s, heads, d, 1e-6, with_mag=True)
    z = o.rmsnorm(x, None, 1e-6)
    assert np.all(np.abs(y) <= mag * (1 + 1e-15))
    hd = d // 2
    for h in range(heads):
        a, b = z[:, h * d:h * d + hd], z[:, h * d + hd:(h + 1) * d]
        cc, ss = c.astype(np.float64), s.astype(np.float64)
        assert np.allclose(mag[:, h * d:h * d + hd], np.abs(a * cc) + np.abs(b * ss), rtol=1e-15)
        assert np.allclose(mag[:, h * d + hd:(h + 1) * d], np.abs(b * cc) + np.abs(a * ss), rtol=1e-15)


# --------------------------------------------------------------------------
# RMSNorm + interleaved RoPE pins (adjacent pairs 2i, 2i + 1)
# --------------------------------------------------------------------------

def pin_rope_il_position_zero_is_rmsnorm(o):
    rng = np.random.default_rng(53)
    heads, d = 3, 16
    x = _rand_bf16(rng, (4, heads * d))
    w = datagen.to_bf16_bits(rng.uniform(0.5, 1.5, heads * d))
    c, s = _tables([0], d)
    y = o.rmsnorm_rope(x, w, c, s, heads, d, 1e-6, interleaved=True)
    assert np.array_equal(y, o.rmsnorm(x, w, 1e-6))


def pin_rope_il_complex_rotation(o):
    """Adjacent pair (2i, 2i + 1) = complex a + ib turned by c_i + i s_i."""
    rng = np.random.default_rng(59)
    heads, d, seq = 2, 8, 4
    x = _rand_bf16(rng, (seq, heads * d))
    w = datagen.to_bf16_bits(rng.uniform(0.5, 1.5, heads * d))
    c, s = _tables(np.arange(seq) * 3 + 1, d)
    y = o.rmsnorm_rope(x, w, c, s, heads, d, 1e-6, interleaved=True)
    z = o.rmsnorm(x, w, 1e-6)
    for r in range(seq):
        for h in range(heads):
            for i in range(d // 2):
                a, b = z[r, h * d + 2 * i], z[r, h * d + 2 * i + 1]
                rot = complex(a, b) * complex(float(c[r, i]), float(s[r, i]))
                got = complex(y[r, h * d + 2 * i], y[r, h * d + 2 * i + 1])
                assert cmath.isclose(got, rot, rel_tol=1e-14, abs_tol=1e-300), (r, h, i)


def pin_rope_small_and_odd_halves(o):
    """Heads of 2, 6 and 10 elements (half heads of 1, 3 and 5 pairs; rows
    that are not whole 16-byte vectors), both pairings: every pair is the
    complex product of its normalised values and the phasor c + is."""
    rng = np.random.default_rng(61)
    for d, heads in ((2, 5), (6, 3), (10, 7)):
        seq = 3
        x = _rand_bf16(rng, (seq, heads * d))
        w = datagen.to_bf16_bits(rng.uniform(0.5, 1.5, heads * d))
        c, s = _tables(np.arange(seq) * 5 + 2, d)
        z = o.rmsnorm(x, w, 1e-6)
        for interleaved in (False, True):
            y = o.rmsnorm_rope(x, w, c, s, heads, d, 1e-6, interleaved=interleaved)
            for r in range(seq):
                for h in range(heads):
                    for i in range(d // 2):
                        ia, ib = (h * d + 2 * i, h * d + 2 * i + 1) if interleaved else (h * d + i, h * d + i + d // 2)
                        rot = complex(z[r, ia], z[r, ib]) * complex(float(c[r, i]), float(s[r, i]))
                        got = complex(y[r, ia], y[r, ib])
                        assert cmath.isclose(got, rot, rel_tol=1e-14, abs_tol=1e-300), (d, interleaved, r, h, i)


def pin_rope_il_matches_rotate_half_after_reorder(o):
    """Reordering each head as [evens, odds] turns adjacent pairs into
    rotate-half pairs: interleaved(x, w) equals rotate-half of the reordered
    x and w, read back in the original order."""
    rng = np.random.default_rng(61)
    heads, d = 4, 32
    x = _rand_bf16(rng, (5, heads * d))
    w = datagen.to_bf16_bits(rng.uniform(0.5, 1.5, heads * d))
    c, s = _tables([0, 7, 100, 2047, 4095], d)
    within = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])
    perm = np.concatenate([h * d + within for h in range(heads)])
    il = o.rmsnorm_rope(x, w, c, s, heads, d, 1e-6, interleaved=True)
    rh = o.rmsnorm_rope(x[:, perm], w[perm], c, s, heads, d, 1e-6)
    back = np.empty_like(rh)
    back[:, perm] = rh
    assert np.allclose(il, back, rtol=1e-14, atol=1e-300)


def pin_rope_il_constant_row(o):
    heads, d = 2, 16
    x = _bf16(np.full((2, heads * d), 1.5))
    c, s = _tables([3, 11], d)
    y = o.rmsnorm_rope(x, None, c, s, heads, d, 0.0, interleaved=True)
    cc, ss = c.astype(np.float64), s.astype(np.float64)
    for h in range(heads):
        assert np.allclose(y[:, h * d:(h + 1) * d:2], cc - ss, rtol=1e-15, atol=1e-15)
        assert np.allclose(y[:, h * d + 1:(h + 1) * d:2], cc + ss, rtol=1e-15, atol=1e-15)


def pin_rope_il_mag(o):
    rng = np.random.default_rng(67)
    heads, d = 2, 8
    x = _rand_bf16(rng, (3, heads * d))
    c, s = _tables([1, 5, 9], d)
    y, mag = o.rmsnorm_rope(x, None, c, s, heads, d, 1e-6, with_mag=True, interleaved=True)
    z = o.rmsnorm(x, None, 1e-6)
    cc, ss = np.repeat(c.astype(np.float64), 2, axis=1), np.repeat(s.astype(np.float64), 2, axis=1)
    for h in range(heads):
        zh = z[:, h * d:(h + 1) * d]
        partner = zh.reshape(3, d // 2, 2)[:, :, ::-1].reshape(3, d)
        assert np.allclose(mag[:, h * d:(h + 1) * d], np.abs(zh * cc) + np.abs(partner * ss), rtol=1e-15)
    assert np.all(np.abs(y) <= mag * (1 + 1e-15))


# --------------------------------------------------------------------------
# AdaLN pins: y = norm(x) * w * (1 + scale[b]) + shift[b], b = r // S
# --------------------------------------------------------------------------

def pin_adaln_zero_modulation_is_rmsnorm(o):
    rng = np.random.default_rng(71)
    x = _rand_bf16(rng, (6, 40))
    w = datagen.to_bf16_bits(rng.uniform(0.5, 1.5, 40))
    zeros = np.zeros((3, 40), dtype=np.uint16)
    assert np.array_equal(o.rmsnorm_adaln(x, w, None, None, 2), o.rmsnorm(x, w, 1e-6))
    assert np.array_equal(o.rmsnorm_adaln(x, w, zeros, zeros, 2), o.rmsnorm(x, w, 1e-6))


def pin_adaln_scale_minus_one_gives_shift(o):
    """1 + scale = 0 removes the normalised value: the output is the shift."""
    rng = np.random.default_rng(73)
    x = _rand_bf16(rng, (4, 24))
    minus1 = np.full((2, 24), 0xBF80, dtype=np.uint16)
    shift = _rand_bf16(rng, (2, 24))
    y = o.rmsnorm_adaln(x, None, minus1, shift, 2)
    assert np.array_equal(y, np.repeat(_val(shift), 2, axis=0))


def pin_adaln_exact_closed_form(o):
    """Constant row c = 2^-3 with eps = 0 normalises to exactly 1, so
    y = w * (1 + scale) + shift, evaluated exactly with fractions."""
    rng = np.random.default_rng(79)
    hidden, S = 16, 3
    x = _bf16(np.full((2 * S, hidden), 0.125))
    w = datagen.to_bf16_bits(rng.uniform(0.5, 1.5, hidden))
    scale = _rand_bf16(rng, (2, hidden), scale=0.3)
    shift = _rand_bf16(rng, (2, hidden), scale=0.3)
    y = o.rmsnorm_adaln(x, w, scale, shift, S, eps=0.0)
    for r in range(2 * S):
        b = r // S
        for j in range(hidden):
            want = (Fraction(float(_val(w[j]))) * (1 + Fraction(float(_val(scale[b, j]))))
                    + Fraction(float(_val(shift[b, j]))))
            assert Fraction(y[r, j]) == want, (r, j)


def pin_adaln_sample_rows(o):
    """Row r uses sample r // S: each row alone with its own sample's
    modulation rows (S = 1) gives the same values."""
    rng = np.random.default_rng(83)
    hidden, S = 24, 3
    x = _rand_bf16(rng, (8, hidden))
    w = datagen.to_bf16_bits(rng.uniform(0.5, 1.5, hidden))
    scale = _rand_bf16(rng, (3, hidden), scale=0.2)
    shift = _rand_bf16(rng, (3, hidden), scale=0.2)
    y = o.rmsnorm_adaln(x, w, scale, shift, S)
    for r in range(8):
        b = r // S
        yr = o.rmsnorm_adaln(x[r:r + 1], w, scale[b:b + 1], shift[b:b + 1], 1)
        assert np.array_equal(yr[0], y[r]), r


def pin_adaln_brute_force(o):
    """Tiny rows against exact fractions / 60-digit decimals."""
    rng = np.random.default_rng(89)
    for hidden in (1, 8, 32):
        x = _rand_bf16(rng, (4, hidden))
        w = datagen.to_bf16_bits(rng.uniform(0.5, 1.5, hidden))
        scale = _rand_bf16(rng, (2, hidden), scale=0.4)
        shift = _rand_bf16(rng, (2, hidden), scale=0.4)
        y = o.rmsnorm_adaln(x, w, scale, shift, 2)
        for r in range(4):
            b = r // 2
            n = _exact_rms_row(_val(x[r]), _val(w), EPS32)
            for j in range(hidden):
                e = n[j] * (1 + Decimal(float(_val(scale[b, j])))) + Decimal(float(_val(shift[b, j])))
                tol = Decimal((hidden + 12) * 2.0 ** -53) * (abs(n[j]) * 2 + abs(e) + Decimal(1e-300))
                assert abs(Decimal(y[r, j]) - e) <= tol, (hidden, r, j)


def pin_adaln_mag(o):
    """The magnitude sum is |n (1 + scale)| + |shift| with n the RMSNorm
    value: it bounds the output and equals its magnitude when the two terms
    have one sign."""
    rng = np.random.default_rng(97)
    x = _rand_bf16(rng, (4, 16))
    w = datagen.to_bf16_bits(rng.uniform(0.5, 1.5, 16))
    scale = _rand_bf16(rng, (2, 16), scale=0.5)
    shift = _rand_bf16(rng, (2, 16), scale=0.5)
    y, mag = o.rmsnorm_adaln(x, w, scale, shift, 2, with_mag=True)
    n = o.rmsnorm(x, w, 1e-6)
    sc = np.repeat(_val(scale), 2, axis=0)
    sh = np.repeat(_val(shift), 2, axis=0)
    assert np.allclose(mag, np.abs(n * (1 + sc)) + np.abs(sh), rtol=1e-15)
    assert np.all(np.abs(y) <= mag * (1 + 1e-15))
    same = np.sign(n * (1 + sc)) == np.sign(sh)
    assert np.allclose(np.abs(y[same]), mag[same], rtol=1e-15)


# --------------------------------------------------------------------------
# Rounding pins
# --------------------------------------------------------------------------

def _bf16_nearest_reference(f32: np.ndarray) -> np.ndarray:
    """Independent RNE: take the two bf16 neighbours bracketing the value
    (truncation and the next one away from zero), compare distances in
    double, break ties toward the even mantissa."""
    u = f32.view(np.uint32)
    lo = (u >> 16).astype(np.uint32)
    hi = lo + 1
    v = f32.astype(np.float64)
    vlo = ((lo << 16).astype(np.uint32)).view(np.float32).astype(np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        vhi = ((hi << 16).astype(np.uint32)).view(np.float32).astype(np.float64)
        dlo, dhi = np.abs(v - vlo), np.abs(vhi - v)
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((lo & 1) == 1))
    # the neighbour past the largest finite bf16 is infinity: the value
    # rounds there only if it is at or beyond the midpoint 0x7f7f8000
    top = (u & 0x7FFFFFFF) >= 0x7F7F8000
    edge = ((lo & 0x7FFF) == 0x7F7F)
    pick_hi = np.where(edge, top, pick_hi)
    return np.where(pick_hi, hi, lo).astype(np.uint16)


def pin_bf16_rounding(o):
    """All 2^16 upper halves (every sign, exponent and kept mantissa) times
    the dropped-bit patterns that decide rounding (0, 1, just below half,
    half, just above half, all ones, and random ones), for finite values,
    against the neighbour-distance formulation; NaN stays NaN and quiet;
    +-Inf stays +-Inf."""
    rng = np.random.default_rng(47)
    uppers = np.arange(1 << 16, dtype=np.uint32)
    lows = np.concatenate([np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32),
                           rng.integers(0, 1 << 16, 6, dtype=np.uint32)])
    bits = ((uppers[:, None] << 16) | lows[None, :]).reshape(-1).astype(np.uint32)
    f = bits.view(np.float32)
    got = o.bf16_from_f32(f)
    finite = np.isfinite(f)
    want = _bf16_nearest_reference(f[finite])
    assert np.array_equal(got[finite], want)
    nan = np.isnan(f)
    g = got[nan]
    assert np.all((g & 0x7F80) == 0x7F80) and np.all((g & 0x0040) != 0)
    assert np.array_equal(np.signbit(f[nan]), (g & 0x8000) != 0)
    inf = np.isinf(f)
    assert np.array_equal(got[inf], (bits[inf] >> 16).astype(np.uint16))


_FORK_ORACLE = None  # the oracle under test, inherited by forked workers


def _bf16_block_mismatches(block) -> int:
    """Mismatches of the oracle's bf16 rounding against the neighbour-distance
    formulation over every binary32 pattern whose upper 16 bits lie in
    [u0, u1): all 2^16 dropped-bit patterns of each.  NaN patterns must give a
    quiet NaN of the same sign, infinities themselves."""
    u0, u1 = block
    o = _FORK_ORACLE
    uppers = np.arange(u0, u1, dtype=np.uint32)
    lows = np.arange(1 << 16, dtype=np.uint32)
    bits = ((uppers[:, None] << 16) | lows[None, :]).reshape(-1)
    f = bits.view(np.float32)
    got = o.bf16_from_f32(f)
    finite = np.isfinite(f)
    bad = int(np.count_nonzero(got[finite] != _bf16_nearest_reference(f[finite])))
    nan = np.isnan(f)
    g = got[nan]
    bad += int(np.count_nonzero(((g & 0x7F80) != 0x7F80) | ((g & 0x0040) == 0)
                                | (np.signbit(f[nan]) != ((g & 0x8000) != 0))))
    inf = np.isinf(f)
    bad += int(np.count_nonzero(got[inf] != (bits[inf] >> 16).astype(np.uint16)))
    return bad


def pin_bf16_rounding_exhaustive(o):
    """Every one of the 2^32 binary32 bit patterns: the oracle's bf16 rounding
    equals the neighbour-distance formulation (finite values), NaN stays a
    quiet NaN of the same sign, +-Inf stays +-Inf.  Blocks of 128 upper
    halves (8 M patterns) run in a pool of forked worker processes."""
    import multiprocessing as mp
    import os
    global _FORK_ORACLE
    _FORK_ORACLE = o
    step = 128
    blocks = [(u, u + step) for u in range(0, 1 << 16, step)]
    workers = max(1, min(8, os.cpu_count() or 1))
    with mp.get_context("fork").Pool(workers) as pool:
        bad = sum(pool.map(_bf16_block_mismatches, blocks, chunksize=4))
    assert bad == 0, f"{bad} binary32 patterns round differently"


def pin_round_twice(o):
    """oracle_round: binary32 of the double, then its bf16 (hand-worked cases
    across a tie, a carry into the exponent, and a negative value)."""
    y = np.array([1.0 + 2 ** -8,              # tie -> even 1.0
                  1.0 + 3 * 2 ** -8,          # tie -> even 1 + 2^-6
                  1.0 + 2 ** -8 + 2 ** -20,   # just above the tie -> up
                  1.0 + 2 ** -8 + 2 ** -30,   # binary32 drops 2^-30: a tie again
                  2.0 - 2 ** -9,              # 0.75 ulp dropped: carry to 2.0
                  -1.5 - 2 ** -8 - 2 ** -20,  # above half, negative: -(1.5 + 2^-7)
                  -1.5 - 2 ** -9 - 2 ** -20,  # below half: -1.5
                  0.0])
    ref32, ref16 = o.round(y)
    assert np.array_equal(ref32, y.astype(np.float32))
    assert list(ref16) == [0x3F80, 0x3F82, 0x3F81, 0x3F80, 0x4000, 0xBFC1, 0xBFC0, 0x0000]


# --------------------------------------------------------------------------
# fp16 and fp32 inputs ("Supported Data Types" on the skill page)
# --------------------------------------------------------------------------

def pin_f16_decode_all_patterns(o):
    """Every binary16 bit pattern decodes to numpy's float16 value."""
    bits = np.arange(1 << 16, dtype=np.uint16)
    got = o.decode(bits.view(np.float16))
    want = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def pin_f16_encode(o):
    """binary32 -> binary16 round-to-nearest-even against numpy's
    float32 -> float16 conversion: random values over the whole range,
    exact ties between neighbours (normal and subnormal), the overflow edge
    and the subnormal/normal boundary."""
    rng = np.random.default_rng(101)
    r = rng.standard_normal(200000).astype(np.float32) * np.exp2(
        rng.uniform(-30, 17, 200000)).astype(np.float32)
    neigh = np.arange(0, 0x7C00, 7, dtype=np.uint16).view(np.float16).astype(np.float32)
    nxt = (np.arange(0, 0x7C00, 7, dtype=np.uint16) + 1).view(np.float16).astype(np.float32)
    ties = ((neigh.astype(np.float64) + nxt.astype(np.float64)) / 2).astype(np.float32)
    edges = np.array([65504, 65519.99, 65520, 65536, 1e9, 6.1035156e-05, 6.0975552e-05,
                      2 ** -24, 2 ** -25, 2 ** -25 * 1.0001, 3 * 2 ** -26, 0.0, np.inf],
                     dtype=np.float32)
    f = np.concatenate([r, ties, -ties, edges, -edges])
    got = o.f16_from_f32(f)
    with np.errstate(over="ignore"):
        want = f.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want), f[got != want][:5]
    nan = o.f16_from_f32(np.array([np.nan, -np.nan], dtype=np.float32))
    assert np.all((nan & 0x7C00) == 0x7C00) and np.all((nan & 0x3FF) != 0) and np.all(nan & 0x200)


def pin_lowp_constant_rows(o):
    """Constant rows in fp16 and fp32 with eps = 0 normalise to exactly
    sign(c), so the output equals sign(c) * w in the input type."""
    rng = np.random.default_rng(103)
    for dt in (np.float16, np.float32):
        w = rng.uniform(0.5, 1.5, 40).astype(dt)
        for c in (0.375, -2.0, 1000.0):
            x = np.full((2, 40), c, dtype=dt)
            y = o.rmsnorm(x, w, 0.0)
            assert np.array_equal(y, np.sign(c) * np.broadcast_to(w.astype(np.float64), y.shape)), (dt, c)


def pin_lowp_brute_force(o):
    """fp16 and fp32 rows against exact fractions / 60-digit decimals, and
    the rounded outputs against the exact value rounded by numpy."""
    rng = np.random.default_rng(107)
    for dt, name in ((np.float16, "f16"), (np.float32, "f32")):
        for hidden in (1, 3, 16, 48):
            x = (rng.standard_normal((3, hidden)) * np.exp2(rng.uniform(-6, 6, (3, hidden)))).astype(dt)
            w = rng.uniform(0.5, 1.5, hidden).astype(dt)
            y = o.rmsnorm(x, w, 1e-6)
            ref32, ref = o.round(y, name)
            for r in range(3):
                exact = _exact_rms_row(x[r].astype(np.float64), w.astype(np.float64), EPS32)
                for j in range(hidden):
                    e = exact[j]
                    tol = Decimal((hidden + 8) * 2.0 ** -53) * abs(e)
                    assert abs(Decimal(y[r, j]) - e) <= tol, (name, hidden, r, j)
            assert np.array_equal(ref, ref32.astype(dt)) or name == "f16"
            if name == "f16":
                assert np.array_equal(ref.view(np.uint16), ref32.astype(np.float16).view(np.uint16))


def pin_lowp_rope_matches_widened_bf16_path(o):
    """The same values given as fp32, fp16 or bf16 inputs (all exactly
    representable) give identical double results for every operation."""
    rng = np.random.default_rng(109)
    heads, d = 2, 16
    xb = _rand_bf16(rng, (5, heads * d))
    wb = datagen.to_bf16_bits(rng.uniform(0.5, 1.5, heads * d))
    # bf16 values with |x| in a range fp16 also holds exactly (8 significant bits)
    xb = datagen.to_bf16_bits(np.clip(_val(xb), -60000, 60000))
    xv, wv = _val(xb), _val(wb)
    assert np.all(xv.astype(np.float16).astype(np.float64) == xv)
    c, s = _tables([3, 5, 7, 9, 11], d)
    for conv in (np.float32, np.float16):
        xc, wc = xv.astype(conv), wv.astype(conv)
        assert np.array_equal(o.rmsnorm(xc, wc, 1e-6), o.rmsnorm(xb, wb, 1e-6))
        for il in (False, True):
            assert np.array_equal(o.rmsnorm_rope(xc, wc, c, s, heads, d, 1e-6, interleaved=il),
                                  o.rmsnorm_rope(xb, wb, c, s, heads, d, 1e-6, interleaved=il))
        sc = _rand_bf16(rng, (1, heads * d), scale=0.3)
        sh = _rand_bf16(rng, (1, heads * d), scale=0.3)
        assert np.array_equal(o.rmsnorm_adaln(xc, wc, _val(sc).astype(conv), _val(sh).astype(conv), 5),
                              o.rmsnorm_adaln(xb, wb, sc, sh, 5))


PINS = [
    pin_eps_inside_root, pin_constant_row_gives_weight, pin_constant_row_small_value,
    pin_zero_row, pin_scale_invariance, pin_sign_symmetry, pin_textbook_norm,
    pin_none_weight_is_ones, pin_rows_independent, pin_permutation, pin_brute_force_exact,
    pin_rope_position_zero_is_rmsnorm, pin_rope_complex_rotation, pin_rope_pair_norm,
    pin_rope_constant_row, pin_rope_row_position, pin_rope_mag, pin_rope_composition,
    pin_rope_il_position_zero_is_rmsnorm, pin_rope_il_complex_rotation,
    pin_rope_small_and_odd_halves, pin_rope_il_matches_rotate_half_after_reorder, pin_rope_il_constant_row, pin_rope_il_mag,
    pin_adaln_zero_modulation_is_rmsnorm, pin_adaln_scale_minus_one_gives_shift,
    pin_adaln_exact_closed_form, pin_adaln_sample_rows, pin_adaln_brute_force, pin_adaln_mag,
    pin_bf16_rounding, pin_round_twice,
    pin_f16_decode_all_patterns, pin_f16_encode, pin_lowp_constant_rows, pin_lowp_brute_force,
    pin_lowp_rope_matches_widened_bf16_path,
    pin_bf16_rounding_exhaustive,
]
