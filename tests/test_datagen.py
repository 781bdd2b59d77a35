"""The seeded input generator: published SplitMix64 vectors, determinism,
counter-based slicing, distributions, recipes and the RoPE tables."""
import json
import math
import os

import numpy as np
import pytest

import datagen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_splitmix64_published_vectors():
    """SplitMix64 from state s yields mix(s + k * 0x9E3779B97F4A7C15), k = 1, 2, ...
    The reference implementation's outputs for seed 1234567 and seed 0."""
    g = datagen._GOLDEN
    with np.errstate(over="ignore"):
        seq = [int(datagen._mix(np.uint64(1234567) + np.uint64(k) * g)) for k in range(1, 6)]
        zero = [int(datagen._mix(np.uint64(k) * g)) for k in range(1, 4)]
    assert seq == [6457827717110365317, 3203168211198807973, 9817491932198370423,
                   4593380528125082431, 16408922859458223821]
    assert zero == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_counter_based_slices():
    full = datagen.raw_u64(5, 9, 0, 1000)
    assert np.array_equal(datagen.raw_u64(5, 9, 337, 100), full[337:437])
    assert np.array_equal(datagen.uniform(5, 9, 50, start=10), datagen.uniform(5, 9, 60)[10:])
    x = datagen.make_x(6, 48, seed=3, stream=1)
    assert np.array_equal(datagen.make_x(2, 48, seed=3, stream=1), x[:2])


def test_deterministic_and_streams_differ():
    a = datagen.make_x(4, 64, seed=1, stream=1)
    assert np.array_equal(a, datagen.make_x(4, 64, seed=1, stream=1))
    assert not np.array_equal(a, datagen.make_x(4, 64, seed=1, stream=2))
    assert not np.array_equal(a, datagen.make_x(4, 64, seed=2, stream=1))


def test_distributions():
    u = datagen.uniform(11, 1, 1 << 20)
    assert u.min() > 0.0 and u.max() < 1.0
    assert abs(u.mean() - 0.5) < 2e-3 and abs(u.var() - 1 / 12) < 1e-3
    n = datagen.normal(11, 2, 1 << 20)
    assert abs(n.mean()) < 5e-3 and abs(n.std() - 1.0) < 5e-3
    # fourth moment of N(0,1) is 3
    assert abs((n ** 4).mean() - 3.0) < 0.05
    w = datagen.bf16_bits_to_f32(datagen.make_w(4096, seed=11, stream=3))
    assert w.min() >= 0.5 and w.max() <= 1.5 and abs(w.mean() - 1.0) < 0.02


def test_bf16_encoding_of_inputs():
    # 2^-130 is the binary32 subnormal with bit 19 set: bf16 pattern 0x0008
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 2 ** -130, 0.0])
    assert list(datagen.to_bf16_bits(v)) == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x0008, 0]
    b = np.arange(0, 1 << 16, dtype=np.uint16)
    f = datagen.bf16_bits_to_f32(b)
    ok = np.isfinite(f)
    assert np.array_equal(datagen.to_bf16_bits(f[ok].astype(np.float64)), b[ok])


def test_recipes():
    c = datagen.CONFIGS
    assert c[datagen.HEADLINE].rows == 16384 and c[datagen.HEADLINE].hidden == 3072
    assert c[datagen.HEADLINE].algorithmic_bytes() == 201_332_736
    assert c[datagen.ROPE].algorithmic_bytes() == 68_161_536
    assert c[datagen.ADALN].algorithmic_bytes() == 4 * 8192 * 2048 + 2 * 2048 + 2 * 2 * 2 * 2048
    assert [c[k].algorithmic_bytes() for k in ("rms_1x1024x2048", "rms_2x1024x2048", "rms_4x1024x2048",
                                               "rms_2x4096x3072_outliers")] == \
        [8_392_704, 16_781_312, 33_558_528, 100_669_440]
    inp = datagen.make_inputs(c["rms_2x4096x3072_outliers"], rows=64)
    f = datagen.bf16_bits_to_f32(inp["x"])
    frac = np.mean(np.abs(f) > 12.0)  # |N(0,2)| > 12 is a 6-sigma event: only outliers
    assert 0.004 < frac < 0.012
    r = datagen.make_inputs(c[datagen.ROPE], rows=8)
    assert r["cos"].shape == (4096, 32) and r["cos"].dtype == np.float32


def test_rope_tables_closed_forms():
    cos_t, sin_t = datagen.rope_tables(4096, 64, 10000.0)
    assert np.all(cos_t[0] == 1.0) and np.all(sin_t[0] == 0.0)
    assert abs(cos_t[1, 0] - 0.5403023) < 1e-7 and abs(sin_t[1, 0] - 0.8414710) < 1e-7
    # slowest frequency: 10000^(-62/64) = 1.3335e-4 rad per position
    assert abs(sin_t[1, 31] - math.sin(10000.0 ** (-62 / 64))) < 1e-11
    assert abs(10000.0 ** (-62 / 64) - 1.3335e-4) < 1e-8
    rng = np.random.default_rng(0)
    for p, i in zip(rng.integers(0, 4096, 200), rng.integers(0, 32, 200)):
        ang = p * 10000.0 ** (-2 * i / 64)
        assert cos_t[p, i] == np.float32(math.cos(ang)) or abs(cos_t[p, i] - math.cos(ang)) < 1.2e-7
        assert sin_t[p, i] == np.float32(math.sin(ang)) or abs(sin_t[p, i] - math.sin(ang)) < 1.2e-7


def test_golden_hashes_and_oracle_fixture():
    """Inputs and oracle results still match the committed fixture written by
    tests/golden/make_golden.py (generator and oracle only)."""
    import oracle
    from golden.make_golden import cases, compute
    doc = json.load(open(os.path.join(GOLDEN, "oracle_small.json")))
    o = oracle.Oracle()
    for name, inp in cases():
        want = doc["cases"][name]
        assert datagen.fnv1a64(inp["x"]) == want["x_fnv"], name
        ref32, ref16 = compute(o, inp)
        assert [format(int(v), "08x") for v in ref32.view("uint32").reshape(-1)] == want["ref32_hex"], name
        assert [format(int(v), "04x") for v in ref16.reshape(-1)] == want["ref16_hex"], name


def test_rope_tables_3d():
    c, s = datagen.rope_tables_3d(3, 4, 5, 64)
    assert c.shape == (60, 32) and s.shape == (60, 32)
    # token (t, h, w) = (2, 1, 3) sits at row (2*4 + 1)*5 + 3 = 48
    r = 48
    for i in range(32):
        coord = (2, 1, 3)[i % 3]
        ang = coord * 10000.0 ** (-2 * (i // 3) / 64)
        assert abs(c[r, i] - np.float32(math.cos(ang))) <= 1.2e-7
        assert abs(s[r, i] - np.float32(math.sin(ang))) <= 1.2e-7
    assert np.all(c[0] == 1.0) and np.all(s[0] == 0.0)
