"""GPU parity: the HIP kernels, called through the C ABI, against the CPU oracle.

Every comparison uses the rule of parity.py (1 bf16 ulp of the oracle's
binary32 result rounded to bf16; a 2^-16 * m floor for cancelling RoPE
outputs).  Full-size workloads are compared at every element, in the same
launch configuration the benchmark times (the library's own dispatch).
Invariants that must hold bit-exactly on the GPU are checked bit-exactly.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
import rmsnorm_video_dit_amd as ltx
from parity import compare

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
ORC = oracle.Oracle()


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)


def dev_bf16(a):
    """Device tensor of an input array: uint16 bf16 bit patterns become a
    bfloat16 tensor, float16 / float32 arrays keep their type."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


def host_bits(t):
    """Back to numpy: bf16 as uint16 bit patterns, others as values."""
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def kind(a):
    return {np.dtype(np.uint16): "bf16", np.dtype(np.float16): "f16",
            np.dtype(np.float32): "f32"}[np.asarray(a).dtype]


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def run_rms(x, w, eps=1e-6):
    xt = dev_bf16(x)
    wt = None if w is None else dev_bf16(w)
    return host_bits(ltx.rmsnorm(xt, wt, eps))


def run_rope(x, w, c, s, heads, head_dim, eps=1e-6, interleaved=False):
    xt = dev_bf16(x)
    wt = None if w is None else dev_bf16(w)
    return host_bits(ltx.rmsnorm_rope(xt, wt, dev_f32(c), dev_f32(s), heads, head_dim, eps,
                                      interleaved=interleaved))


def check_rms(x, w, eps=1e-6, label=""):
    got = run_rms(x, w, eps)
    ref32, ref = ORC.round(ORC.rmsnorm(x, w, eps), kind(x))
    rep = compare(got, ref, None, ref32)
    print(label, rep, flush=True)
    assert rep["pass"], (label, rep)
    return got, rep


def run_adaln(x, w, scale, shift, rows_per_sample, eps=1e-6):
    xt = dev_bf16(x)
    wt = None if w is None else dev_bf16(w)
    st = None if scale is None else dev_bf16(scale)
    ht = None if shift is None else dev_bf16(shift)
    return host_bits(ltx.rmsnorm_adaln(xt, wt, st, ht, eps, rows_per_sample=rows_per_sample))


def check_adaln(x, w, scale, shift, rows_per_sample, eps=1e-6, label=""):
    got = run_adaln(x, w, scale, shift, rows_per_sample, eps)
    y, mag = ORC.rmsnorm_adaln(x, w, scale, shift, rows_per_sample, eps, with_mag=True)
    ref32, ref = ORC.round(y, kind(x))
    rep = compare(got, ref, mag, ref32)
    print(label, rep, flush=True)
    assert rep["pass"], (label, rep)
    return got, rep


def check_rope(x, w, c, s, heads, head_dim, eps=1e-6, label="", interleaved=False):
    got = run_rope(x, w, c, s, heads, head_dim, eps, interleaved)
    y, mag = ORC.rmsnorm_rope(x, w, c, s, heads, head_dim, eps, with_mag=True,
                              interleaved=interleaved)
    ref32, ref = ORC.round(y, kind(x))
    rep = compare(got, ref, mag, ref32)
    print(label, rep, flush=True)
    assert rep["pass"], (label, rep)
    return got, rep


# ---------------------------------------------------------------------------
# The workloads at full size
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(datagen.CONFIGS))
def test_workload_full_size(name):
    cfg = datagen.CONFIGS[name]
    announce(f"workload {name} rows={cfg.rows} hidden={cfg.hidden} seed={datagen.BASE_SEED}")
    inp = datagen.make_inputs(cfg)
    if cfg.rope:
        got, rep = check_rope(inp["x"], inp["w"], inp["cos"], inp["sin"], cfg.heads, cfg.head_dim,
                              cfg.eps, label=name, interleaved=cfg.interleaved)
    elif cfg.adaln:
        got, rep = check_adaln(inp["x"], inp["w"], inp["scale"], inp["shift"],
                               inp["rows_per_sample"], cfg.eps, label=name)
    else:
        got, rep = check_rms(inp["x"], inp["w"], cfg.eps, label=name)
    if cfg.rope or cfg.adaln:
        # only outputs whose two terms cancel may differ by more than an
        # ulp of their (small) value, and only within the 2^-16 * m floor
        assert rep["n_floor_bound"] <= 1e-5 * rep["n"]
    else:
        assert rep["max_ulp"] <= 1.0
    # nearly every element matches bit for bit; the rest are single rounding flips
    assert rep.get("n_bit_exact", rep.get("n_exact")) >= 0.99 * rep["n"]


@pytest.mark.parametrize("name", list(datagen.LARGE_CONFIGS))
def test_large_workload_full_size(name):
    """The fused operations at the headline's size, every element."""
    cfg = datagen.LARGE_CONFIGS[name]
    announce(f"large workload {name} rows={cfg.rows} hidden={cfg.hidden}")
    inp = datagen.make_inputs(cfg)
    if cfg.rope:
        got, rep = check_rope(inp["x"], inp["w"], inp["cos"], inp["sin"], cfg.heads, cfg.head_dim,
                              cfg.eps, label=name, interleaved=cfg.interleaved)
    else:
        got, rep = check_adaln(inp["x"], inp["w"], inp["scale"], inp["shift"],
                               inp["rows_per_sample"], cfg.eps, label=name)
    assert rep["n_floor_bound"] <= 1e-5 * rep["n"]
    assert rep["n_bit_exact"] >= 0.99 * rep["n"]


# ---------------------------------------------------------------------------
# fp16 and fp32 I/O: every operation at the workloads' full size
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f16", "f32"])
@pytest.mark.parametrize("name", ["rms_4x4096x3072", "rms_2x4096x3072_outliers",
                                  "rope_2x4096x2048_h32d64", "ropei_2x4096x2048_h32d64",
                                  "adaln_2x4096x2048"])
def test_workload_full_size_lowp(name, dtype):
    cfg = datagen.CONFIGS[name]
    announce(f"workload {name} dtype={dtype}")
    inp = datagen.make_inputs(cfg, dtype=dtype)
    if cfg.rope:
        got, rep = check_rope(inp["x"], inp["w"], inp["cos"], inp["sin"], cfg.heads, cfg.head_dim,
                              cfg.eps, label=f"{name} {dtype}", interleaved=cfg.interleaved)
    elif cfg.adaln:
        got, rep = check_adaln(inp["x"], inp["w"], inp["scale"], inp["shift"],
                               inp["rows_per_sample"], cfg.eps, label=f"{name} {dtype}")
    else:
        got, rep = check_rms(inp["x"], inp["w"], cfg.eps, label=f"{name} {dtype}")
    if dtype == "f16":
        assert rep["n_exact"] >= 0.99 * rep["n"]
    elif not (cfg.rope or cfg.adaln):
        # binary32 out, no cancelling sum: a few units of the last place
        # (4 measured; the rule allows 16 units of 2^-24 relative)
        assert rep["max_ulp"] <= 16
    if dtype == "f16":
        # 16-bit outputs: only strongly cancelled outputs need the floor
        assert rep["n_floor_bound"] <= 1e-4 * rep["n"]
    # (binary32 outputs carry an evaluation error proportional to the terms'
    # magnitude m, so any mild cancellation leans on m; the rule itself is
    # the check)


@pytest.mark.parametrize("dtype,hidden", [("f16", 8), ("f16", 1000), ("f16", 3072), ("f16", 12296),
                                          ("f16", 65536), ("f32", 4), ("f32", 36), ("f32", 2052),
                                          ("f32", 3072), ("f32", 6148), ("f32", 32768)])
@pytest.mark.parametrize("rows", [1, 7, 1023])
def test_lowp_edge_shapes(dtype, hidden, rows):
    if rows * hidden > (1 << 23):
        rows = max(1, (1 << 23) // hidden)
    announce(f"rmsnorm {dtype} rows={rows} hidden={hidden}")
    x = datagen.make_x(rows, hidden, seed=hidden + rows, stream=1, dtype=dtype)
    w = datagen.make_w(hidden, seed=hidden + rows, stream=2, dtype=dtype)
    check_rms(x, w, label=f"rms {dtype} {rows}x{hidden}")
    rps = max(1, -(-rows // 2))          # two samples (one when rows == 1)
    samples = -(-rows // rps)
    sc = datagen.make_x(samples, hidden, seed=hidden, stream=4, sigma=0.3, dtype=dtype)
    sh = datagen.make_x(samples, hidden, seed=hidden, stream=5, sigma=0.3, dtype=dtype)
    check_adaln(x, w, sc, sh, rps, label=f"adaln {dtype} {rows}x{hidden}")


# fp32 vectors hold 4 values: the vector kernels take rotate-half head_dim % 8
# (coalesced up to 256) and interleaved % 4; other even head_dims take the
# general kernel
@pytest.mark.parametrize("dtype,heads,head_dim,interleaved", [
    ("f16", 32, 64, False), ("f16", 24, 128, False), ("f16", 5, 48, False), ("f16", 3, 1024, False),
    ("f16", 32, 64, True), ("f16", 5, 24, True),
    ("f32", 4, 8, False), ("f32", 32, 64, False), ("f32", 16, 256, False), ("f32", 4, 512, False),
    ("f32", 6, 40, False), ("f32", 3, 4, True), ("f32", 32, 64, True), ("f32", 5, 12, True),
    ("f32", 2, 1000, True)])
@pytest.mark.parametrize("rows,seq_len", [(7, 3), (300, 4096)])
def test_lowp_rope(dtype, heads, head_dim, interleaved, rows, seq_len):
    hidden = heads * head_dim
    announce(f"rope {dtype} {heads}x{head_dim} il={interleaved} rows={rows}")
    x = datagen.make_x(rows, hidden, seed=hidden + 11, stream=1, dtype=dtype)
    w = datagen.make_w(hidden, seed=hidden + 11, stream=2, dtype=dtype)
    c, s = datagen.rope_tables(seq_len, head_dim)
    check_rope(x, w, c, s, heads, head_dim, interleaved=interleaved,
               label=f"rope {dtype} {heads}x{head_dim} il={interleaved}")


# AdaLN and the fused RoPE kernels spread rows of 257..768 vectors (320 for
# interleaved pairs) over two or three wavefronts with 3-4 vectors per lane
# (rotate-half: four wavefronts with 3 from 577 vectors on): every such
# instance (2, 3 or 4 wavefronts, 3 or 4 vectors, last vector whole or
# masked, shared or per-slot table slices) in the three dtypes, with an odd
# row count so the second row slot of the last workgroup idles.
WIDE_SHAPES = [
    ("bf16", "adaln", 2304, 0), ("bf16", "adaln", 3584, 0), ("bf16", "adaln", 4104, 0),
    ("bf16", "adaln", 4608, 0), ("bf16", "adaln", 5120, 0), ("bf16", "adaln", 6144, 0),
    ("f16", "adaln", 4096, 0), ("f32", "adaln", 1152, 0), ("f32", "adaln", 2560, 0),
    ("f32", "adaln", 3072, 0),
    ("bf16", "half", 2304, 128), ("bf16", "half", 3584, 128), ("bf16", "half", 4224, 128),
    ("bf16", "half", 4608, 128), ("bf16", "half", 5120, 128), ("f16", "half", 6144, 128),
    ("f32", "half", 2048, 128), ("f32", "half", 2304, 128), ("f32", "half", 2560, 128),
    ("bf16", "il", 2304, 128), ("f16", "il", 2560, 128), ("bf16", "il", 2520, 72),
    ("f32", "il", 1152, 64),
    # rotate-half past 768 vectors: 4 vectors per lane over 4..15 wavefronts
    ("bf16", "half", 6656, 128), ("f16", "half", 8192, 128), ("bf16", "half", 10240, 128),
    ("f32", "half", 4224, 128), ("bf16", "half", 13312, 64),
    # head-packed rotate-half (heads not a power of two): the wide split too
    ("bf16", "half", 2304, 72), ("bf16", "half", 2880, 72), ("bf16", "half", 2560, 80),
    ("f16", "half", 3072, 96), ("f32", "half", 2560, 40),
]


@pytest.mark.parametrize("dtype,op,hidden,head_dim", WIDE_SHAPES)
@pytest.mark.parametrize("rows", [37, 1001])
def test_wide_split_shapes(dtype, op, hidden, head_dim, rows):
    code = {"bf16": ltx.BF16, "f16": ltx.F16, "f32": ltx.F32}[dtype]
    opc = {"adaln": ltx.OP_ADALN, "half": ltx.OP_ROPE, "il": ltx.OP_ROPE_INTERLEAVED}[op]
    heads = hidden // head_dim if head_dim else 0
    desc = ltx.ltxnorm_describe_launch(opc, rows, hidden, heads, head_dim, code)
    f = dict(kv.split("=") for kv in desc.split()[1:])
    wpr, per = int(f["wavefronts_per_row"]), int(f["vectors_per_lane"])
    assert (wpr, per) in ((2, 3), (2, 4), (3, 3), (3, 4), (4, 3)) or (op == "half" and per == 4 and wpr >= 4), desc
    announce(f"wide split {dtype} {op} rows={rows} hidden={hidden} d={head_dim}: {desc}")
    seed = hidden + rows + 29
    x = datagen.make_x(rows, hidden, seed=seed, stream=1, dtype=dtype)
    w = datagen.make_w(hidden, seed=seed, stream=2, dtype=dtype)
    if op == "adaln":
        rps = 300
        samples = -(-rows // rps)
        sc = datagen.make_x(samples, hidden, seed=seed, stream=4, sigma=0.3, dtype=dtype)
        sh = datagen.make_x(samples, hidden, seed=seed, stream=5, sigma=0.3, dtype=dtype)
        check_adaln(x, w, sc, sh, rps, label=f"adaln {dtype} {rows}x{hidden}")
    else:
        c, s = datagen.rope_tables(4096 if rows > 100 else 17, head_dim)
        check_rope(x, w, c, s, heads, head_dim, interleaved=op == "il",
                   label=f"rope {dtype} {op} {rows}x{heads}x{head_dim}")


# Rows of up to 160 vectors in segments of 1-32 lanes with 1, 2, 3 or 5 vectors
# per lane (several rows per wavefront): every (lanes, vectors) shape for each
# operation that takes it, in the three dtypes, with per-slot and shared
# interleaved table slices and rotate-half partners up to 16 lanes away; row
# counts leave the last workgroup's segments partly idle.
SEGMENT_SHAPES = [
    # dtype, op, hidden, head_dim, lanes, vectors per lane
    ("bf16", "rms", 320, 0, 16, 3), ("f16", "adaln", 384, 0, 16, 3), ("bf16", "half", 320, 64, 16, 3),
    ("bf16", "il", 360, 72, 16, 3), ("f32", "rms", 160, 0, 16, 3),
    ("bf16", "adaln", 576, 0, 16, 5), ("f16", "half", 576, 64, 16, 5), ("bf16", "il", 576, 72, 16, 5),
    ("f32", "rms", 288, 0, 16, 5), ("f32", "adaln", 320, 0, 16, 5), ("bf16", "rms", 520, 0, 16, 5),
    ("f16", "rms", 704, 0, 32, 3), ("bf16", "adaln", 768, 0, 32, 3), ("bf16", "half", 704, 64, 32, 3),
    ("bf16", "il", 720, 80, 32, 3), ("f32", "half", 352, 32, 32, 3), ("f32", "il", 384, 64, 32, 3),
    ("bf16", "adaln", 1152, 0, 32, 5), ("f32", "adaln", 576, 0, 32, 5), ("bf16", "half", 1152, 64, 32, 5),
    ("bf16", "half", 1280, 256, 32, 5), ("f16", "adaln", 1088, 0, 32, 5),
    # two vectors per lane on half the lanes (rows of up to 64 vectors)
    ("bf16", "rms", 16, 0, 2, 1), ("bf16", "rms", 24, 0, 4, 1), ("bf16", "il", 32, 8, 4, 1),
    ("bf16", "rms", 128, 0, 8, 2), ("bf16", "il", 128, 64, 8, 2), ("f16", "adaln", 256, 0, 16, 2),
    ("bf16", "half", 256, 128, 16, 2), ("f32", "rms", 128, 0, 16, 2), ("bf16", "rms", 512, 0, 32, 2),
    ("bf16", "adaln", 448, 0, 32, 2), ("f32", "half", 256, 64, 32, 2), ("f32", "adaln", 40, 0, 8, 2),
    ("bf16", "rms", 72, 0, 8, 2),
    # rotate-half partners in the lane's other slot (P == lanes, two vectors per lane)
    ("bf16", "half", 128, 128, 8, 2), ("f16", "half", 256, 256, 16, 2), ("f32", "half", 128, 128, 16, 2),
    ("bf16", "half", 512, 512, 32, 2),
    # rows of up to 8 vectors: one vector per lane
    ("bf16", "half", 64, 64, 8, 1),
]


@pytest.mark.parametrize("dtype,op,hidden,head_dim,lanes,per", SEGMENT_SHAPES)
@pytest.mark.parametrize("rows", [37, 1001])
def test_segmented_rows(dtype, op, hidden, head_dim, lanes, per, rows):
    code = {"bf16": ltx.BF16, "f16": ltx.F16, "f32": ltx.F32}[dtype]
    opc = {"rms": ltx.OP_RMSNORM, "adaln": ltx.OP_ADALN, "half": ltx.OP_ROPE,
           "il": ltx.OP_ROPE_INTERLEAVED}[op]
    heads = hidden // head_dim if head_dim else 0
    desc = ltx.ltxnorm_describe_launch(opc, rows, hidden, heads, head_dim, code)
    f = dict(kv.split("=") for kv in desc.split()[1:])
    assert desc.startswith("rmsnorm_short_kernel ") and (int(f["lanes_per_row"]), int(f["vectors_per_lane"])) \
        == (lanes, per), desc
    announce(f"segmented {dtype} {op} rows={rows} hidden={hidden} d={head_dim}: {lanes} x {per}")
    seed = hidden + rows + 41
    x = datagen.make_x(rows, hidden, seed=seed, stream=1, dtype=dtype)
    w = datagen.make_w(hidden, seed=seed, stream=2, dtype=dtype)
    if op == "rms":
        check_rms(x, w, label=f"rms {dtype} {rows}x{hidden}")
        check_rms(x, None, label=f"rms {dtype} {rows}x{hidden} no weight")
    elif op == "adaln":
        rps = 300
        samples = -(-rows // rps)
        sc = datagen.make_x(samples, hidden, seed=seed, stream=4, sigma=0.3, dtype=dtype)
        sh = datagen.make_x(samples, hidden, seed=seed, stream=5, sigma=0.3, dtype=dtype)
        check_adaln(x, w, sc, sh, rps, label=f"adaln {dtype} {rows}x{hidden}")
        check_adaln(x, w, None, sh, rps, label=f"adaln {dtype} {rows}x{hidden} no scale")
    else:
        c, s = datagen.rope_tables(4096 if rows > 100 else 17, head_dim)
        check_rope(x, w, c, s, heads, head_dim, interleaved=op == "il",
                   label=f"rope {dtype} {op} {rows}x{heads}x{head_dim}")


# Both sides of every boundary of the row-split rules (vectors per row):
# one vector per lane up to 8, two from 9, 16 x 3 for 33..48, 32 x 2 from 49,
# 16 x 5 / 32 x 3 / 32 x 5 segments to 160, one wavefront to 256, the wide
# split to 768 (rotate-half: 3 vectors from 513, 4 wavefronts from 577, 4
# vectors past 768; interleaved: to 320).  Interleaved pairs use heads of 8
# so odd vector counts occur; rotate-half uses heads of 16 (even counts).
BOUNDARY_VECTORS = [8, 9, 32, 33, 48, 49, 64, 65, 80, 81, 96, 97, 128, 129, 160, 161,
                    256, 257, 320, 321, 512, 513, 576, 577, 768, 769]


@pytest.mark.parametrize("n", BOUNDARY_VECTORS)
@pytest.mark.parametrize("op", ["rms", "adaln", "il", "half"])
def test_split_rule_boundaries(op, n):
    if op == "half" and n % 2:
        n += 1
    hidden = 8 * n
    rows = 37
    d = {"il": 8, "half": 16}.get(op, 0)
    opc = {"rms": ltx.OP_RMSNORM, "adaln": ltx.OP_ADALN, "il": ltx.OP_ROPE_INTERLEAVED,
           "half": ltx.OP_ROPE}[op]
    desc = ltx.ltxnorm_describe_launch(opc, rows, hidden, hidden // d if d else 0, d)
    announce(f"split boundary {op} vectors={n}: {desc}")
    seed = 1000 + n
    x = datagen.make_x(rows, hidden, seed=seed, stream=1)
    w = datagen.make_w(hidden, seed=seed, stream=2)
    if op == "rms":
        check_rms(x, w, label=f"rms boundary {n}")
    elif op == "adaln":
        sc = datagen.make_x(2, hidden, seed=seed, stream=4, sigma=0.3)
        sh = datagen.make_x(2, hidden, seed=seed, stream=5, sigma=0.3)
        check_adaln(x, w, sc, sh, 20, label=f"adaln boundary {n}")
    else:
        c, s = datagen.rope_tables(29, d)
        check_rope(x, w, c, s, hidden // d, d, interleaved=op == "il", label=f"rope {op} boundary {n}")


def _random_shapes(count, seed):
    """Seeded shapes of every operation and dtype: hidden sizes from 1 to
    about 20000 (whole vectors or not), even head sizes from 2 to 1200,
    1..40 rows; at most 2^21 elements each."""
    rng = np.random.default_rng(seed)
    shapes = []
    while len(shapes) < count:
        dtype = str(rng.choice(["bf16", "f16", "f32"]))
        op = str(rng.choice(["rms", "adaln", "half", "il"]))
        rows = int(rng.integers(1, 41))
        if op in ("half", "il"):
            d = 2 * int(rng.choice([rng.integers(1, 40), rng.integers(1, 600), 32, 36, 64]))
            heads = int(rng.integers(1, max(2, 20000 // d)))
            hidden = heads * d
        else:
            d = heads = 0
            hidden = int(rng.choice([rng.integers(1, 2000), rng.integers(1, 20000),
                                     8 * rng.integers(1, 2500)]))
        if rows * hidden <= (1 << 21):
            shapes.append((dtype, op, rows, hidden, heads, d))
    return shapes


@pytest.mark.parametrize("case", range(4))
def test_random_shapes(case):
    """Every (kernel, row split) the dispatch can reach has a compiled
    instance: seeded random shapes of every operation and dtype, each
    checked element by element against the oracle."""
    for dtype, op, rows, hidden, heads, d in _random_shapes(60, 20261203 + case):
        announce(f"random {dtype} {op} rows={rows} hidden={hidden} heads={heads} d={d}")
        seed = rows * 7919 + hidden
        x = datagen.make_x(rows, hidden, seed=seed, stream=1, dtype=dtype)
        w = datagen.make_w(hidden, seed=seed, stream=2, dtype=dtype)
        if op == "rms":
            check_rms(x, w, label=f"random rms {dtype} {rows}x{hidden}")
        elif op == "adaln":
            rps = max(1, rows // 3)
            samples = -(-rows // rps)
            sc = datagen.make_x(samples, hidden, seed=seed, stream=4, sigma=0.3, dtype=dtype)
            sh = datagen.make_x(samples, hidden, seed=seed, stream=5, sigma=0.3, dtype=dtype)
            check_adaln(x, w, sc, sh, rps, label=f"random adaln {dtype} {rows}x{hidden}")
        else:
            c, s = datagen.rope_tables(23, d)
            check_rope(x, w, c, s, heads, d, interleaved=op == "il",
                       label=f"random rope {op} {dtype} {rows}x{heads}x{d}")


@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_lowp_invariants(dtype):
    """NULL weight = ones; position 0 = RMSNorm; null modulation = RMSNorm;
    in place = out of place; run to run identical."""
    announce(f"invariants {dtype}")
    x = datagen.make_x(200, 2048, seed=21, stream=1, dtype=dtype)
    w = datagen.make_w(2048, seed=21, stream=2, dtype=dtype)
    ones = np.ones(2048, dtype=x.dtype)
    base = run_rms(x, w)
    assert np.array_equal(base, run_rms(x, w))
    assert np.array_equal(run_rms(x, None), run_rms(x, ones))
    # position 0 equals RMSNorm bit for bit where both take the same row
    # split (the split fixes the order of the sum of squares); elsewhere
    # check_rope holds it to the oracle
    c0, s0 = datagen.rope_tables(1, 64)
    code = {"f16": ltx.F16, "f32": ltx.F32}[dtype]
    rms_plan = ltx.ltxnorm_describe_launch(ltx.OP_RMSNORM, 200, 2048, 0, 0, code).split()[1:3]
    for op, il in ((ltx.OP_ROPE, False), (ltx.OP_ROPE_INTERLEAVED, True)):
        if ltx.ltxnorm_describe_launch(op, 200, 2048, 32, 64, code).split()[1:3] == rms_plan:
            assert np.array_equal(run_rope(x, w, c0, s0, 32, 64, interleaved=il), base)
        else:
            check_rope(x, w, c0, s0, 32, 64, interleaved=il, label=f"rope {dtype} position 0")
    assert np.array_equal(run_adaln(x, w, None, None, 100), base)
    xt = dev_bf16(x)
    ltx.rmsnorm(xt, dev_bf16(w), 1e-6, out=xt)
    assert np.array_equal(host_bits(xt), base)


def test_f16_exact_ties_and_overflow():
    """fp16 rounding: rows of 1s and 3s with mean square 4 make y = 1.5 w
    exact in binary32; w = 1 + 3 * 2^-10 puts it half way between two fp16
    values (the even one wins), w = 1 + 2^-10 likewise.  A weight of 60000
    makes 1.5 w = 90000 overflow to infinity."""
    announce("f16 ties")
    pattern = np.array([1, 1, 1, 1, 1, 3, 3, 3], dtype=np.float16)
    x = np.tile(pattern, (3, 8))
    w = np.full(64, 1 + 3 * 2 ** -10, dtype=np.float16)
    w[1::2] = 1 + 2 ** -10
    w[5] = 60000.0
    got = run_rms(x, w, 0.0)
    _, ref = ORC.round(ORC.rmsnorm(x, w, 0.0), "f16")
    assert np.array_equal(got.view(np.uint16), ref.view(np.uint16))
    three = x == 3
    assert np.all(got[three & (np.arange(64) % 2 == 0)[None, :] & (np.arange(64) != 5)[None, :]]
                  == np.float16(1.5 + 4 * 2 ** -10))   # 4.5 units -> even 4
    assert np.all(got[three & ((np.arange(64) % 2 == 1) & (np.arange(64) != 5))[None, :]]
                  == np.float16(1.5 + 2 * 2 ** -10))   # 1.5 units -> even 2
    assert np.all(np.isinf(got[:, 5][three[:, 5]]))


# ---------------------------------------------------------------------------
# Edge shapes: ragged tails, one/several wavefronts per row, the hidden cap
# ---------------------------------------------------------------------------

HIDDENS = [8, 64, 520, 1000, 2048, 3072, 4096, 4104, 6144, 8192, 12296, 16384, 32768, 65536]
ROWS = [1, 3, 5, 1023]


@pytest.mark.parametrize("hidden", HIDDENS)
@pytest.mark.parametrize("rows", ROWS)
def test_rmsnorm_edge_shapes(rows, hidden):
    if rows * hidden > (1 << 24):
        rows = max(1, (1 << 24) // hidden)
    announce(f"rmsnorm rows={rows} hidden={hidden}")
    x = datagen.make_x(rows, hidden, seed=hidden * 7 + rows, stream=1)
    w = datagen.make_w(hidden, seed=hidden * 7 + rows, stream=2)
    check_rms(x, w, label=f"rms {rows}x{hidden}")


# power-of-two head_dim 16..512 takes the coalesced kernel (partner lane
# xor 1..32); other multiples of 16 and head_dim > 512 take pair-in-lane
@pytest.mark.parametrize("heads,head_dim", [(1, 16), (3, 16), (2, 32), (32, 64), (5, 64),
                                            (16, 128), (24, 128), (8, 256), (4, 512),
                                            (6, 512), (64, 128), (96, 128), (512, 128),
                                            (128, 512), (1, 1024), (3, 1024), (3, 48),
                                            (5, 80), (6, 96), (2, 112), (40, 80)])
@pytest.mark.parametrize("rows,seq_len", [(1, 1), (7, 3), (37, 4096), (1000, 17)])
def test_rope_edge_shapes(heads, head_dim, rows, seq_len):
    hidden = heads * head_dim
    if rows * hidden > (1 << 24):
        rows = max(1, (1 << 24) // hidden)
    announce(f"rope rows={rows} heads={heads} head_dim={head_dim} seq_len={seq_len}")
    x = datagen.make_x(rows, hidden, seed=hidden + rows, stream=1)
    w = datagen.make_w(hidden, seed=hidden + rows, stream=2)
    c, s = datagen.rope_tables(seq_len, head_dim, 10000.0)
    check_rope(x, w, c, s, heads, head_dim, label=f"rope {rows}x{heads}x{head_dim} S={seq_len}")


@pytest.mark.parametrize("heads,head_dim", [(1, 8), (3, 16), (5, 24), (32, 64), (16, 128),
                                            (24, 128), (40, 80), (128, 512), (1, 1024),
                                            (512, 128)])
@pytest.mark.parametrize("rows,seq_len", [(1, 1), (7, 3), (37, 4096), (1000, 17)])
def test_rope_interleaved_edge_shapes(heads, head_dim, rows, seq_len):
    hidden = heads * head_dim
    if rows * hidden > (1 << 24):
        rows = max(1, (1 << 24) // hidden)
    announce(f"rope interleaved rows={rows} heads={heads} head_dim={head_dim} seq_len={seq_len}")
    x = datagen.make_x(rows, hidden, seed=hidden + rows + 5, stream=1)
    w = datagen.make_w(hidden, seed=hidden + rows + 5, stream=2)
    c, s = datagen.rope_tables(seq_len, head_dim, 10000.0)
    check_rope(x, w, c, s, heads, head_dim, interleaved=True,
               label=f"rope-il {rows}x{heads}x{head_dim} S={seq_len}")


def test_rope_interleaved_invariants():
    """Position 0 is plain RMSNorm; in place equals out of place; a NULL
    weight equals ones; run to run identical."""
    announce("rope interleaved invariants")
    x = datagen.make_x(300, 3072, seed=15, stream=1)
    w = datagen.make_w(3072, seed=15, stream=2)
    c0, s0 = datagen.rope_tables(1, 128)
    assert np.array_equal(run_rope(x, w, c0, s0, 24, 128, interleaved=True), run_rms(x, w))
    c, s = datagen.rope_tables(77, 128)
    ref = run_rope(x, w, c, s, 24, 128, interleaved=True)
    assert np.array_equal(ref, run_rope(x, w, c, s, 24, 128, interleaved=True))
    xt = dev_bf16(x)
    ltx.rmsnorm_rope(xt, dev_bf16(w), dev_f32(c), dev_f32(s), 24, 128, 1e-6, out=xt,
                     interleaved=True)
    assert np.array_equal(host_bits(xt), ref)
    ones = np.full(3072, 0x3F80, dtype=np.uint16)
    assert np.array_equal(run_rope(x, None, c, s, 24, 128, interleaved=True),
                          run_rope(x, ones, c, s, 24, 128, interleaved=True))


@pytest.mark.parametrize("interleaved", [False, True])
def test_rope_video_3d_tables(interleaved):
    """3D video positions: one table row per t*h*w token ([batch, t*h*w,
    heads, head_dim]); a batch of 2 clips of 7 x 12 x 16 tokens."""
    announce(f"rope 3d tables interleaved={interleaved}")
    c, s = datagen.rope_tables_3d(7, 12, 16, 64)
    rows = 2 * c.shape[0]
    x = datagen.make_x(rows, 2048, seed=16, stream=1)
    w = datagen.make_w(2048, seed=16, stream=2)
    check_rope(x, w, c, s, 32, 64, interleaved=interleaved, label=f"rope 3d il={interleaved}")


def test_rope_outlier_values_and_null_weight():
    announce("rope outliers, weight None")
    x = datagen.make_x(300, 2048, seed=5, stream=1, sigma=2.0, outlier_p=0.01, outlier_scale=50.0)
    c, s = datagen.rope_tables(4096, 64, 10000.0)
    check_rope(x, None, c, s, 32, 64, label="rope outliers")


@pytest.mark.parametrize("hidden", [8, 520, 2048, 3072, 4104, 16384, 65536])
@pytest.mark.parametrize("rows,rows_per_sample", [(1, 1), (7, 3), (1023, 1023), (4000, 1000)])
def test_adaln_edge_shapes(rows, rows_per_sample, hidden):
    if rows * hidden > (1 << 24):
        rows = max(1, (1 << 24) // hidden)
        rows_per_sample = max(1, min(rows_per_sample, rows))
    samples = -(-rows // rows_per_sample)
    announce(f"adaln rows={rows} hidden={hidden} rows_per_sample={rows_per_sample}")
    seed = hidden + rows + 3 * rows_per_sample
    x = datagen.make_x(rows, hidden, seed=seed, stream=1)
    w = datagen.make_w(hidden, seed=seed, stream=2)
    sc = datagen.make_x(samples, hidden, seed=seed, stream=4, sigma=0.3)
    sh = datagen.make_x(samples, hidden, seed=seed, stream=5, sigma=0.3)
    check_adaln(x, w, sc, sh, rows_per_sample, label=f"adaln {rows}x{hidden} S={rows_per_sample}")


def test_adaln_invariants():
    """Null modulation equals RMSNorm bit for bit; null weight equals ones;
    scale = -1 gives the shift exactly; in place equals out of place."""
    announce("adaln invariants")
    x = datagen.make_x(600, 3072, seed=17, stream=1)
    w = datagen.make_w(3072, seed=17, stream=2)
    assert np.array_equal(run_adaln(x, w, None, None, 200), run_rms(x, w))
    sc = datagen.make_x(3, 3072, seed=17, stream=4, sigma=0.3)
    sh = datagen.make_x(3, 3072, seed=17, stream=5, sigma=0.3)
    ones = np.full(3072, 0x3F80, dtype=np.uint16)
    ref = run_adaln(x, w, sc, sh, 200)
    assert np.array_equal(run_adaln(x, None, sc, sh, 200), run_adaln(x, ones, sc, sh, 200))
    minus1 = np.full((3, 3072), 0xBF80, dtype=np.uint16)
    got = run_adaln(x, w, minus1, sh, 200)
    assert np.array_equal(got, np.repeat(sh, 200, axis=0))
    # one NULL row: the kernel reads a NULL scale as +0 and a NULL shift as -0
    zeros = np.zeros((3, 3072), dtype=np.uint16)
    neg_zeros = np.full((3, 3072), 0x8000, dtype=np.uint16)
    assert np.array_equal(run_adaln(x, w, None, sh, 200), run_adaln(x, w, zeros, sh, 200))
    assert np.array_equal(run_adaln(x, w, sc, None, 200), run_adaln(x, w, sc, neg_zeros, 200))
    xt = dev_bf16(x)
    ltx.rmsnorm_adaln(xt, dev_bf16(w), dev_bf16(sc), dev_bf16(sh), 1e-6, out=xt, rows_per_sample=200)
    assert np.array_equal(host_bits(xt), ref)


# ---------------------------------------------------------------------------
# Bit-exact invariants on the GPU
# ---------------------------------------------------------------------------

def test_deterministic_run_to_run():
    announce("determinism 4096x3072 and rope 2048x2048")
    x = datagen.make_x(4096, 3072, seed=1, stream=1)
    w = datagen.make_w(3072, seed=1, stream=2)
    a, b = run_rms(x, w), run_rms(x, w)
    assert np.array_equal(a, b)
    x = datagen.make_x(2048, 2048, seed=2, stream=1)
    c, s = datagen.rope_tables(4096, 64)
    assert np.array_equal(run_rope(x, w[:2048], c, s, 32, 64), run_rope(x, w[:2048], c, s, 32, 64))


@pytest.mark.parametrize("hidden", [3072, 8192])
def test_batch_invariance(hidden):
    """A row's output does not depend on how many rows are in the call."""
    announce(f"batch invariance hidden={hidden}")
    x = datagen.make_x(2000, hidden, seed=3, stream=1)
    w = datagen.make_w(hidden, seed=3, stream=2)
    full = run_rms(x, w)
    for lo, hi in ((0, 1), (17, 18), (5, 1000), (1999, 2000)):
        assert np.array_equal(run_rms(x[lo:hi], w), full[lo:hi]), (lo, hi)


@pytest.mark.parametrize("hidden", [2048, 3072, 16384])
def test_in_place_equals_out_of_place(hidden):
    announce(f"in-place hidden={hidden}")
    x = datagen.make_x(513, hidden, seed=4, stream=1)
    w = datagen.make_w(hidden, seed=4, stream=2)
    ref = run_rms(x, w)
    xt, wt = dev_bf16(x), dev_bf16(w)
    ltx.rmsnorm(xt, wt, 1e-6, out=xt)
    assert np.array_equal(host_bits(xt), ref)
    c, s = datagen.rope_tables(100, 64)
    heads = hidden // 64
    ref = run_rope(x, w, c, s, heads, 64)
    xt = dev_bf16(x)
    ltx.rmsnorm_rope(xt, wt, dev_f32(c), dev_f32(s), heads, 64, 1e-6, out=xt)
    assert np.array_equal(host_bits(xt), ref)


@pytest.mark.parametrize("hidden", [520, 3072, 8192])
def test_null_weight_equals_ones(hidden):
    announce(f"null weight hidden={hidden}")
    x = datagen.make_x(64, hidden, seed=6, stream=1)
    ones = np.full(hidden, 0x3F80, dtype=np.uint16)
    assert np.array_equal(run_rms(x, None), run_rms(x, ones))
    c, s = datagen.rope_tables(9, 64)
    heads = hidden // 64 if hidden % 64 == 0 else None
    if heads:
        assert np.array_equal(run_rope(x, None, c, s, heads, 64), run_rope(x, ones, c, s, heads, 64))


def test_rope_position_zero_is_rmsnorm():
    announce("rope at position 0")
    x = datagen.make_x(50, 2048, seed=8, stream=1)
    w = datagen.make_w(2048, seed=8, stream=2)
    c, s = datagen.rope_tables(1, 64)
    assert np.array_equal(run_rope(x, w, c, s, 32, 64), run_rms(x, w))


def test_sign_symmetry_and_scale_invariance():
    """y(-x) = -y(x); with eps = 0, y(2^k x) = y(x) (correctly rounded divide
    and square root scale exactly by powers of two)."""
    announce("sign and scale")
    x = datagen.make_x(256, 3072, seed=9, stream=1)
    w = datagen.make_w(3072, seed=9, stream=2)
    base = run_rms(x, w, 0.0)
    assert np.array_equal(run_rms(x ^ np.uint16(0x8000), w, 0.0), base ^ np.uint16(0x8000))
    xv = datagen.bf16_bits_to_f32(x).astype(np.float64)
    for k in (-8, -3, 2, 8):
        assert np.array_equal(run_rms(datagen.to_bf16_bits(xv * 2.0 ** k), w, 0.0), base), k


def test_rope_pair_norm():
    """The rotation keeps each pair's norm (within the outputs' bf16 rounding)."""
    announce("rope pair norm")
    x = datagen.make_x(64, 2048, seed=10, stream=1)
    c, s = datagen.rope_tables(4096, 64)
    got = datagen.bf16_bits_to_f32(run_rope(x, None, c, s, 32, 64)).astype(np.float64)
    plain = datagen.bf16_bits_to_f32(run_rms(x, None)).astype(np.float64)
    g = got.reshape(64, 32, 2, 32)
    p = plain.reshape(64, 32, 2, 32)
    n_rot = g[:, :, 0] ** 2 + g[:, :, 1] ** 2
    n_in = p[:, :, 0] ** 2 + p[:, :, 1] ** 2
    assert np.allclose(n_rot, n_in, rtol=2 * 2.0 ** -7, atol=1e-6)


# ---------------------------------------------------------------------------
# Special values
# ---------------------------------------------------------------------------

def test_zero_rows_and_eps_zero_nan():
    announce("zero rows")
    x = datagen.make_x(8, 2048, seed=11, stream=1)
    x[2] = 0
    x[5, ::7] = 0
    got, _ = check_rms(x, datagen.make_w(2048, seed=11, stream=2), 1e-6, label="zeros")
    assert np.all(got[2] == 0) and np.all((got[5, ::7] & 0x7FFF) == 0)
    # eps = 0 and an all-zero row: 0 * inf = NaN on both sides
    got = run_rms(x, None, 0.0)
    assert np.all(np.isnan(datagen.bf16_bits_to_f32(got[2])))
    check_rms(x, None, 0.0, label="eps0 zero row (NaN must meet NaN)")


def test_round_to_nearest_even_on_exact_ties():
    """Rows of 1s and 3s with mean square exactly 4 make rstd = 0.5 exactly,
    so y = x * 0.5 * w is exact in binary32 and the only rounding is the
    final bf16 one; weights 1 + 3*2^-7 put 1.5 * w exactly halfway between
    two bf16 values: the result must be the even one, bit-exactly."""
    announce("exact ties")
    pattern = np.array([1, 1, 1, 1, 1, 3, 3, 3], dtype=np.float64)  # sum of squares 32 = 4 * 8
    x = datagen.to_bf16_bits(np.tile(pattern, (4, 64 // 8)))
    w = np.full(64, 0x3F83, dtype=np.uint16)          # 1 + 3 * 2^-7
    w[1::2] = 0x3F81                                   # 1 + 2^-7: 1.5 w = 1.5 + 1.5 ulp
    got = run_rms(x, w, 0.0)
    _, ref16 = ORC.round(ORC.rmsnorm(x, w, 0.0))
    assert np.array_equal(got, ref16)
    three = x == 0x4040
    assert np.all(got[three & (w == 0x3F83)[None, :]] == 0x3FC4)   # tie 4.5 ulp -> even 4
    assert np.all(got[three & (w == 0x3F81)[None, :]] == 0x3FC2)   # tie 1.5 ulp -> even 2


# ---------------------------------------------------------------------------
# Memory safety and the boundary on the device
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("rows,hidden", [(1, 8), (7, 520), (33, 3072), (5, 12296)])
def test_guard_bands_survive(rows, hidden):
    """Sentinels before and after the output (and the input) are untouched."""
    announce(f"guard bands rows={rows} hidden={hidden}")
    pad = 4096
    x = datagen.make_x(rows, hidden, seed=12, stream=1)
    w = datagen.make_w(hidden, seed=12, stream=2)
    n = rows * hidden
    buf = torch.full((n + 2 * pad,), 0x7A5A, dtype=torch.int16, device=DEV)
    out = buf[pad:pad + n].view(torch.bfloat16).view(rows, hidden)
    xt = dev_bf16(x)
    ltx.rmsnorm(xt, dev_bf16(w), 1e-6, out=out)
    b = host_bits(buf.view(torch.bfloat16))
    assert np.all(b[:pad] == 0x7A5A) and np.all(b[pad + n:] == 0x7A5A)
    assert np.array_equal(b[pad:pad + n].reshape(rows, hidden), run_rms(x, w))
    assert np.array_equal(host_bits(xt), x)  # input untouched
    if hidden % 64 == 0:
        heads = hidden // 64
        c, s = datagen.rope_tables(5, 64)
        buf.fill_(0x7A5A)
        ltx.rmsnorm_rope(xt, dev_bf16(w), dev_f32(c), dev_f32(s), heads, 64, 1e-6, out=out)
        b = host_bits(buf.view(torch.bfloat16))
        assert np.all(b[:pad] == 0x7A5A) and np.all(b[pad + n:] == 0x7A5A)


def test_rejected_calls_write_nothing():
    announce("rejected calls")
    x = dev_bf16(datagen.make_x(4, 2048, seed=13, stream=1))
    buf = torch.full((4 * 2048 + 8,), 0x1234, dtype=torch.int16, device=DEV)
    mis = buf.data_ptr() + 2  # 2-byte offset: misaligned
    st = ltx.ltxnorm_rmsnorm_fwd_status(mis, x, None, 4, 2048, 1e-6, None)
    assert st == ltx.ERR_ALIGN
    st = ltx.ltxnorm_rmsnorm_fwd_status(buf, x, None, 4, ltx.MAX_HIDDEN + 1, 1e-6, None)
    assert st == ltx.ERR_UNSUPPORTED
    assert np.all(host_bits(buf.view(torch.bfloat16)) == 0x1234)


def test_empty_input():
    announce("empty")
    x = torch.empty((0, 2048), dtype=torch.bfloat16, device=DEV)
    assert ltx.rmsnorm(x).shape == (0, 2048)
    c = torch.zeros((4, 32), dtype=torch.float32, device=DEV)
    assert ltx.rmsnorm_rope(x, None, c, c, 32, 64).shape == (0, 2048)


def test_side_stream():
    """Work goes on the caller's stream."""
    announce("side stream")
    x = datagen.make_x(1024, 3072, seed=14, stream=1)
    w = datagen.make_w(3072, seed=14, stream=2)
    xt, wt = dev_bf16(x), dev_bf16(w)
    out = torch.empty_like(xt)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ltx.ltxnorm_rmsnorm_fwd(out, xt, wt, 1024, 3072, 1e-6, s)
    s.synchronize()
    assert np.array_equal(host_bits(out), run_rms(x, w))
