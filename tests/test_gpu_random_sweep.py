"""A seeded random sweep through every path the library picks: operation,
dtype, hidden size (1 to 400000), head size, row count, NULL weight, eps
(including 0), NULL modulation rows, rows_per_sample, table length and
in-place calls, each compared element by element with the oracle under the
rule of parity.py.  The case list is fixed by the seed, so a failure names a
case that can be rerun alone."""
import numpy as np
import pytest

import datagen
import rmsnorm_video_dit_amd as ltx
from parity import compare
from test_gpu_parity import ORC, announce, dev_bf16, dev_f32, host_bits, kind

pytestmark = pytest.mark.gpu

CODE = {"bf16": ltx.BF16, "f16": ltx.F16, "f32": ltx.F32}
OPC = {"rms": ltx.OP_RMSNORM, "adaln": ltx.OP_ADALN, "half": ltx.OP_ROPE, "il": ltx.OP_ROPE_INTERLEAVED}


def _cases(seed=20261204, n=240):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        dtype = str(rng.choice(["bf16", "f16", "f32"]))
        E = 4 if dtype == "f32" else 8
        op = str(rng.choice(["rms", "adaln", "half", "il"]))
        r = rng.random()
        if r < 0.3:
            H = int(rng.integers(1, 2000))
        elif r < 0.6:
            H = int(rng.integers(2000, 20000))
        elif r < 0.85:
            H = int(E * rng.integers(1, 9000))
        else:
            H = int(rng.integers(20000, 400000))
        d = heads = 0
        if op in ("half", "il"):
            d = int(2 * rng.integers(1, max(2, min(H // 2, 800)) + 1))
            heads = max(1, H // d)
            H = heads * d
        rows = int(rng.choice([rng.integers(1, 8), rng.integers(1, 300), rng.integers(1, 4000)]))
        rows = max(1, min(rows, (4_000_000 if H < 100000 else 12_000_000) // H))
        out.append(dict(dtype=dtype, op=op, H=H, d=d, heads=heads, rows=rows, seed=int(rng.integers(1 << 30)),
                        null_w=bool(rng.random() < 0.1), eps=float(rng.choice([1e-6, 1e-5, 0.0])),
                        inplace=bool(rng.random() < 0.2), seq=int(rng.integers(1, rows + 6)),
                        rps=int(rng.integers(1, rows + 1)), null_mod=int(rng.integers(0, 8))))
    return out


CASES = _cases()


def _run(c):
    dt, op, H, rows = c["dtype"], c["op"], c["H"], c["rows"]
    x = datagen.make_x(rows, H, seed=c["seed"], stream=1, dtype=dt)
    w = None if c["null_w"] else datagen.make_w(H, seed=c["seed"], stream=2, dtype=dt)
    xt = dev_bf16(x)
    wt = None if w is None else dev_bf16(w)
    out = xt if c["inplace"] else None
    mag = None
    if op == "rms":
        got = host_bits(ltx.rmsnorm(xt, wt, c["eps"], out=out))
        y = ORC.rmsnorm(x, w, c["eps"])
    elif op == "adaln":
        ns = -(-rows // c["rps"])
        sc = None if c["null_mod"] == 1 else datagen.make_x(ns, H, seed=c["seed"], stream=4, sigma=0.25, dtype=dt)
        sh = None if c["null_mod"] == 2 else datagen.make_x(ns, H, seed=c["seed"], stream=5, sigma=0.25, dtype=dt)
        got = host_bits(ltx.rmsnorm_adaln(xt, wt, None if sc is None else dev_bf16(sc),
                                          None if sh is None else dev_bf16(sh), c["eps"], out=out,
                                          rows_per_sample=c["rps"]))
        y, mag = ORC.rmsnorm_adaln(x, w, sc, sh, c["rps"], c["eps"], with_mag=True)
    else:
        cs, sn = datagen.rope_tables(c["seq"], c["d"])
        il = op == "il"
        got = host_bits(ltx.rmsnorm_rope(xt, wt, dev_f32(cs), dev_f32(sn), c["heads"], c["d"], c["eps"],
                                         out=out, interleaved=il))
        y, mag = ORC.rmsnorm_rope(x, w, cs, sn, c["heads"], c["d"], c["eps"], with_mag=True, interleaved=il)
    ref32, ref = ORC.round(y, kind(x))
    return compare(got, ref, mag, ref32)


@pytest.mark.parametrize("i", range(len(CASES)))
def test_random_sweep(i):
    c = CASES[i]
    desc = ltx.ltxnorm_describe_launch(OPC[c["op"]], c["rows"], c["H"], c["heads"], c["d"], CODE[c["dtype"]])
    announce(f"random sweep {i}: {c} -> {desc.split()[0]}")
    rep = _run(c)
    assert rep["pass"], (c, desc, rep)


def test_random_sweep_reaches_every_kernel_family():
    """The sweep's cases, as the library dispatches them (no GPU work)."""
    seen = set()
    for c in CASES:
        d = ltx.ltxnorm_describe_launch(OPC[c["op"]], c["rows"], c["H"], c["heads"], c["d"], CODE[c["dtype"]])
        seen.add(d.split()[0].split("(")[0])
    assert {"rmsnorm_kernel", "rmsnorm_adaln_kernel", "rmsnorm_general_kernel", "rmsnorm_long_kernel",
            "rmsnorm_split_kernels", "rmsnorm_rope_interleaved_kernel", "rmsnorm_rope_pair_kernel",
            "rmsnorm_short_kernel"} <= seen, seen


def _mid_cases(seed=20261205, n=40):
    """Launches of 500 to 9000 rows of hidden about 1500 to 5200: whole grids
    that a device may hold at once, where the library takes its one-wavefront
    priority and regrouped forms, next to the same shapes' plain splits."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        dtype = str(rng.choice(["bf16", "f16", "f32"]))
        E = 4 if dtype == "f32" else 8
        op = str(rng.choice(["rms", "adaln", "half", "il"]))
        H = int(E * rng.integers(1500 // E, 5200 // E))
        d = heads = 0
        if op in ("half", "il"):
            d = int(rng.choice([32, 64, 128])) if rng.random() < 0.7 else int(2 * rng.integers(1, 200))
            heads = max(1, H // d)
            H = heads * d
        rows = int(min(rng.integers(500, 9000), 40_000_000 // H))
        out.append(dict(dtype=dtype, op=op, H=H, d=d, heads=heads, rows=rows, seed=int(rng.integers(1 << 30)),
                        null_w=bool(rng.random() < 0.1), eps=float(rng.choice([1e-6, 1e-5])),
                        inplace=bool(rng.random() < 0.2), seq=int(rng.integers(1, rows + 6)),
                        rps=int(rng.integers(1, rows + 1)), null_mod=int(rng.integers(0, 8))))
    return out


MID_CASES = _mid_cases()


@pytest.mark.parametrize("i", range(len(MID_CASES)))
def test_random_mid_sweep(i):
    c = MID_CASES[i]
    desc = ltx.ltxnorm_describe_launch(OPC[c["op"]], c["rows"], c["H"], c["heads"], c["d"], CODE[c["dtype"]])
    announce(f"random mid sweep {i}: {c} -> {desc}")
    rep = _run(c)
    assert rep["pass"], (c, desc, rep)


def test_random_mid_sweep_reaches_the_one_wave_forms():
    """The mid-size cases, as the library describes them (no GPU work):
    one-wavefront rows that may take the priority instances, and rows of a
    few wavefronts that may regroup, in RMSNorm, AdaLN and both RoPEs."""
    seen = set()
    for c in MID_CASES:
        d = ltx.ltxnorm_describe_launch(OPC[c["op"]], c["rows"], c["H"], c["heads"], c["d"], CODE[c["dtype"]])
        name = d.split()[0].split("(")[0]
        if "one_wave_vectors_per_lane=" in d:
            seen.add(name + " regroup")
        elif "load_priority=one_wave" in d:
            seen.add(name + " one-wave")
    assert {"rmsnorm_kernel regroup", "rmsnorm_adaln_kernel regroup", "rmsnorm_rope_xor_kernel regroup",
            "rmsnorm_rope_interleaved_kernel regroup", "rmsnorm_kernel one-wave"} <= seen, seen
