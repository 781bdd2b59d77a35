"""GPU parity of the kernels for rows of any length, through the C ABI,
against the CPU oracle (same rule as every parity test: parity.py).

* Hidden sizes that are not a whole number of 16-byte vectors (rows start
  part-way into a vector; the row's end vectors are shared with the
  neighbouring rows), in bf16, fp16 and fp32, for RMSNorm and AdaLN.
* RoPE head sizes the vector kernels cannot pair (any even head_dim),
  rotate-half (partners exchanged through LDS) and interleaved.
* Rows beyond the register budget (two-pass kernel), every operation.
* In place = out of place, NULL weight = ones, run-to-run identity, and
  guard bands around the output, on each of these paths.
"""
import numpy as np
import pytest
import torch

import datagen
import rmsnorm_video_dit_amd as ltx
from parity import compare
from test_gpu_parity import (DEV, ORC, announce, kind, check_adaln, check_rms, check_rope, dev_bf16,
                             dev_f32, host_bits, run_adaln, run_rms, run_rope)

pytestmark = pytest.mark.gpu

# rows that start inside a 16-byte vector, rows shorter than one vector,
# rows one element past a vector, up to the register budget
ODD_HIDDEN = {
    "bf16": [1, 2, 3, 5, 7, 9, 15, 17, 100, 255, 257, 1001, 2047, 2049, 3070, 3076, 4097, 6150,
             12289, 65529],
    "f16": [1, 3, 7, 9, 1001, 2050, 3076, 6150],
    "f32": [1, 2, 3, 5, 6, 1023, 1025, 2050, 3070, 8191, 32765],
}


def _cases():
    for dt, hs in ODD_HIDDEN.items():
        for h in hs:
            yield dt, h


@pytest.mark.parametrize("dtype,hidden", list(_cases()))
@pytest.mark.parametrize("rows", [1, 7, 333])
def test_any_hidden(dtype, hidden, rows):
    rows = max(1, min(rows, (1 << 22) // hidden))
    announce(f"any-hidden {dtype} rows={rows} hidden={hidden}")
    seed = 3 * hidden + rows
    x = datagen.make_x(rows, hidden, seed=seed, stream=1, dtype=dtype)
    w = datagen.make_w(hidden, seed=seed, stream=2, dtype=dtype)
    got, rep = check_rms(x, w, label=f"rms {dtype} {rows}x{hidden}")
    if dtype != "f32":
        assert rep["max_ulp"] <= 1.0
    rps = max(1, -(-rows // 3))           # three samples (fewer for tiny batches)
    samples = -(-rows // rps)
    sc = datagen.make_x(samples, hidden, seed=seed, stream=4, sigma=0.25, dtype=dtype)
    sh = datagen.make_x(samples, hidden, seed=seed, stream=5, sigma=0.25, dtype=dtype)
    check_adaln(x, w, sc, sh, rps, label=f"adaln {dtype} {rows}x{hidden}")


# beyond the register budget: 65536 bf16/fp16 or 32768 fp32 per row (and rows
# whose vectors straddle one more than that)
LONG = [("bf16", 65537), ("bf16", 65544), ("bf16", 70001), ("bf16", 131072), ("bf16", 262147),
        ("f16", 65544), ("f16", 100003), ("f32", 32767), ("f32", 32772), ("f32", 40001),
        ("f32", 65536)]


@pytest.mark.parametrize("dtype,hidden", LONG)
@pytest.mark.parametrize("rows", [1, 3, 6])
def test_long_rows(dtype, hidden, rows):
    announce(f"long rows {dtype} rows={rows} hidden={hidden}")
    seed = hidden + rows
    x = datagen.make_x(rows, hidden, seed=seed, stream=1, dtype=dtype)
    w = datagen.make_w(hidden, seed=seed, stream=2, dtype=dtype)
    got, rep = check_rms(x, w, label=f"long rms {dtype} {rows}x{hidden}")
    if dtype != "f32":
        assert rep["max_ulp"] <= 1.0
    rps = 2
    samples = -(-rows // rps)
    sc = datagen.make_x(samples, hidden, seed=seed, stream=4, sigma=0.25, dtype=dtype)
    sh = datagen.make_x(samples, hidden, seed=seed, stream=5, sigma=0.25, dtype=dtype)
    check_adaln(x, w, sc, sh, rps, label=f"long adaln {dtype} {rows}x{hidden}")


# (heads, head_dim): head sizes the vector kernels cannot pair, rows that are
# not whole vectors; LONG_ROPE: long rows (head-packed for 129 x 136, the
# two-pass kernel for the rest, except interleaved pairs on rows of 16 chunks
# of 2048 vectors or more: the split kernels, whole and ragged rows)
ROPE_SHAPES = [(1, 2), (33, 2), (5, 6), (7, 10), (4, 24), (16, 72), (32, 40), (3, 130),
               (2, 136), (24, 88), (13, 14), (1, 1000), (9, 18), (20, 52)]
LONG_ROPE = [(129, 136), (2, 40000), (1, 70002), (255, 258), (64, 1026), (1024, 256), (2, 122882)]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("heads,head_dim", ROPE_SHAPES)
@pytest.mark.parametrize("interleaved", [False, True])
@pytest.mark.parametrize("rows,seq_len", [(7, 3), (300, 4096)])
def test_any_head_dim_rope(dtype, heads, head_dim, interleaved, rows, seq_len):
    hidden = heads * head_dim
    announce(f"any-head rope {dtype} {heads}x{head_dim} il={interleaved} rows={rows}")
    seed = hidden + head_dim + rows
    x = datagen.make_x(rows, hidden, seed=seed, stream=1, dtype=dtype)
    w = datagen.make_w(hidden, seed=seed, stream=2, dtype=dtype)
    c, s = datagen.rope_tables(seq_len, head_dim)
    check_rope(x, w, c, s, heads, head_dim, interleaved=interleaved,
               label=f"rope {dtype} {rows}x{heads}x{head_dim} il={interleaved}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("heads,head_dim", LONG_ROPE)
@pytest.mark.parametrize("interleaved", [False, True])
def test_long_rope(dtype, heads, head_dim, interleaved):
    hidden = heads * head_dim
    rows = 3
    announce(f"long rope {dtype} {heads}x{head_dim} il={interleaved}")
    x = datagen.make_x(rows, hidden, seed=hidden + 1, stream=1, dtype=dtype)
    w = datagen.make_w(hidden, seed=hidden + 1, stream=2, dtype=dtype)
    c, s = datagen.rope_tables(5, head_dim)
    check_rope(x, w, c, s, heads, head_dim, interleaved=interleaved,
               label=f"long rope {dtype} {heads}x{head_dim} il={interleaved}")


# one shape per path: general RMSNorm/AdaLN, general rotate-half (LDS),
# general interleaved, two-pass RMSNorm/AdaLN, two-pass rotate-half and
# interleaved, split RMSNorm/AdaLN/interleaved (in place: two-pass)
PATHS = [
    ("rms", 3076, 0), ("adaln", 3070, 0), ("half", 16 * 72, 72), ("il", 7 * 10, 10),
    ("rms", 70001, 0), ("adaln", 65544, 0), ("half", 129 * 136, 136), ("il", 255 * 258, 258),
    ("half", 2 * 40000, 40000),
    ("rms", 262147, 0), ("adaln", 262144, 0), ("il", 1024 * 256, 256),
]


def _run(op, x, w, c, s, d, out=None):
    xt = x if torch.is_tensor(x) else dev_bf16(x)
    wt = None if w is None else dev_bf16(w)
    rows, hidden = xt.shape
    if op == "rms":
        return ltx.rmsnorm(xt, wt, 1e-6, out=out)
    if op == "adaln":
        sc = dev_bf16(datagen.make_x(2, hidden, seed=5, stream=4, sigma=0.25))
        sh = dev_bf16(datagen.make_x(2, hidden, seed=5, stream=5, sigma=0.25))
        return ltx.rmsnorm_adaln(xt, wt, sc, sh, 1e-6, out=out, rows_per_sample=-(-rows // 2))
    return ltx.rmsnorm_rope(xt, wt, dev_f32(c), dev_f32(s), hidden // d, d, 1e-6, out=out,
                            interleaved=(op == "il"))


@pytest.mark.parametrize("op,hidden,d", PATHS)
def test_paths_invariants(op, hidden, d):
    """In place equals out of place; run to run identical; NULL weight equals
    ones; position 0 equals RMSNorm (RoPE); writes stay inside out."""
    rows = 5
    announce(f"path invariants {op} hidden={hidden} d={d}")
    x = datagen.make_x(rows, hidden, seed=hidden, stream=1)
    w = datagen.make_w(hidden, seed=hidden, stream=2)
    c, s = datagen.rope_tables(7, d) if d else (None, None)
    ref = host_bits(_run(op, x, w, c, s, d))
    assert np.array_equal(ref, host_bits(_run(op, x, w, c, s, d)))
    # in place
    xt = dev_bf16(x)
    _run(op, xt, w, c, s, d, out=xt)
    assert np.array_equal(host_bits(xt), ref)
    # NULL weight = ones
    ones = np.full(hidden, 0x3F80, dtype=np.uint16)
    assert np.array_equal(host_bits(_run(op, x, None, c, s, d)), host_bits(_run(op, x, ones, c, s, d)))
    if d:
        c0, s0 = datagen.rope_tables(1, d)
        assert np.array_equal(host_bits(_run(op, x, w, c0, s0, d)), host_bits(_run("rms", x, w, None, None, 0)))
    # guard bands: out is a 16-byte aligned window of a larger buffer filled
    # with a sentinel; nothing outside the window changes
    pad = 64
    big = torch.full((rows * hidden + 2 * pad,), -7.0, dtype=torch.bfloat16, device=DEV)
    out = big[pad: pad + rows * hidden].view(rows, hidden)
    _run(op, x, w, c, s, d, out=out)
    b = host_bits(big)
    sentinel = np.array([-7.0], dtype=np.float32).view(np.uint32)[0] >> 16
    assert np.all(b[:pad] == sentinel) and np.all(b[pad + rows * hidden:] == sentinel)
    assert np.array_equal(b[pad: pad + rows * hidden].reshape(rows, hidden), ref)


# Long rows out of place take the split kernels: chunks of 2048 vectors over
# many workgroups, the partial sums staged in the row's own output.  In place
# they take the two-pass kernel.  Both add a row's squares in the same order.
# rows of 16 or more chunks of 2048 vectors, fewer than 624 rows: whole and
# ragged rows, a last chunk of one vector, the most rows, 2048 chunks
SPLIT = [("bf16", 262144, 37), ("bf16", 1 << 20, 5), ("bf16", 245769, 13), ("f32", 122881, 64),
         ("f16", 262147, 9), ("bf16", 16 * 16384 + 8, 1), ("bf16", 262144, 191), ("f16", 245769, 300),
         ("f32", 1 << 24, 1)]


@pytest.mark.parametrize("dtype,hidden,rows", SPLIT)
def test_split_rows(dtype, hidden, rows):
    """Every element against the oracle (RMSNorm and AdaLN), x untouched by
    the staging, and the in-place result (two-pass kernel) equal bit for bit."""
    code = {"bf16": ltx.BF16, "f16": ltx.F16, "f32": ltx.F32}[dtype]
    desc = ltx.ltxnorm_describe_launch(ltx.OP_RMSNORM, rows, hidden, 0, 0, code)
    assert desc.startswith("rmsnorm_split_kernels"), desc
    announce(f"split rows {dtype} {rows}x{hidden}")
    seed = hidden + 7 * rows
    x = datagen.make_x(rows, hidden, seed=seed, stream=1, dtype=dtype)
    w = datagen.make_w(hidden, seed=seed, stream=2, dtype=dtype)
    got, rep = check_rms(x, w, label=f"split rms {dtype} {rows}x{hidden}")
    if dtype != "f32":
        assert rep["max_ulp"] <= 1.0
    # in place: the two-pass kernel, the same bits
    xt, wt = dev_bf16(x), dev_bf16(w)
    yt = ltx.rmsnorm(xt, wt, 1e-6)
    bits = (lambda a: np.asarray(a).view(np.uint16 if dtype != "f32" else np.uint32))
    assert np.array_equal(bits(host_bits(xt)), bits(x))  # the staging area lives in the output
    assert np.array_equal(bits(host_bits(yt)), bits(got))
    ltx.rmsnorm(xt, wt, 1e-6, out=xt)
    assert np.array_equal(bits(host_bits(xt)), bits(got))
    rps = max(1, -(-rows // 3))
    samples = -(-rows // rps)
    sc = datagen.make_x(samples, hidden, seed=seed, stream=4, sigma=0.25, dtype=dtype)
    sh = datagen.make_x(samples, hidden, seed=seed, stream=5, sigma=0.25, dtype=dtype)
    check_adaln(x, w, sc, sh, rps, label=f"split adaln {dtype} {rows}x{hidden}")


def _random_long_cases():
    """Seeded shapes past the register budget: row counts on both sides of the
    split's bound, widths of 5 to 40 chunks, whole and ragged rows, every
    operation and dtype (a list built once, so pytest ids stay stable)."""
    rng = np.random.default_rng(20261203)
    cases = []
    for i in range(12):
        dtype = ["bf16", "f16", "f32"][i % 3]
        E = 4 if dtype == "f32" else 8
        op = ["rms", "adaln", "il", "half"][i % 4]
        chunks = int(rng.integers(5, 41))
        hidden = int(chunks * 2048 * E - rng.integers(0, 2048 * E))
        if op in ("il", "half"):
            d = 2 * int(rng.integers(8, 200))
            hidden = max(1, hidden // d) * d
        rows = int(rng.choice([rng.integers(1, 12), rng.integers(180, 200)]))
        rows = min(rows, max(1, (24 << 20) // hidden))  # about 24 M elements at most
        cases.append((op, dtype, rows, hidden, d if op in ("il", "half") else 0))
    return cases


RANDOM_LONG = _random_long_cases()


@pytest.mark.parametrize("op,dtype,rows,hidden,d", RANDOM_LONG)
def test_random_long_rows(op, dtype, rows, hidden, d):
    """Every element against the oracle, through whichever long-row kernel
    the library picks; the sample reaches both (asserted in the CPU tests'
    kernel-choice sweep and here by the case list)."""
    code = {"bf16": ltx.BF16, "f16": ltx.F16, "f32": ltx.F32}[dtype]
    opc = {"rms": ltx.OP_RMSNORM, "adaln": ltx.OP_ADALN, "il": ltx.OP_ROPE_INTERLEAVED, "half": ltx.OP_ROPE}[op]
    desc = ltx.ltxnorm_describe_launch(opc, rows, hidden, hidden // d if d else 0, d, code)
    assert desc.split()[0] in ("rmsnorm_split_kernels", "rmsnorm_long_kernel"), desc
    announce(f"random long {op} {dtype} {rows}x{hidden} d={d}: {desc.split()[0]}")
    seed = hidden + 13 * rows
    x = datagen.make_x(rows, hidden, seed=seed, stream=1, dtype=dtype)
    w = datagen.make_w(hidden, seed=seed, stream=2, dtype=dtype)
    label = f"random long {op} {dtype} {rows}x{hidden} d={d}"
    if op == "rms":
        check_rms(x, w, label=label)
    elif op == "adaln":
        rps = max(1, -(-rows // 2))
        samples = -(-rows // rps)
        sc = datagen.make_x(samples, hidden, seed=seed, stream=4, sigma=0.25, dtype=dtype)
        sh = datagen.make_x(samples, hidden, seed=seed, stream=5, sigma=0.25, dtype=dtype)
        check_adaln(x, w, sc, sh, rps, label=label)
    else:
        c, s_ = datagen.rope_tables(7, d)
        check_rope(x, w, c, s_, hidden // d, d, interleaved=(op == "il"), label=label)


def test_random_long_cases_reach_both_kernels():
    kinds = set()
    for op, dtype, rows, hidden, d in RANDOM_LONG:
        code = {"bf16": ltx.BF16, "f16": ltx.F16, "f32": ltx.F32}[dtype]
        opc = {"rms": ltx.OP_RMSNORM, "adaln": ltx.OP_ADALN, "il": ltx.OP_ROPE_INTERLEAVED, "half": ltx.OP_ROPE}[op]
        kinds.add(ltx.ltxnorm_describe_launch(opc, rows, hidden, hidden // d if d else 0, d, code).split()[0])
    assert kinds == {"rmsnorm_split_kernels", "rmsnorm_long_kernel"}, kinds


def test_adaln_null_modulation_any_hidden():
    """NULL scale and shift give RMSNorm bit for bit on the general and
    two-pass kernels too."""
    for hidden in (3076, 70001):
        announce(f"adaln null modulation hidden={hidden}")
        x = datagen.make_x(4, hidden, seed=9, stream=1)
        w = datagen.make_w(hidden, seed=9, stream=2)
        assert np.array_equal(run_adaln(x, w, None, None, 2), run_rms(x, w))


@pytest.mark.parametrize("hidden", [3076, 2048, 70001])
def test_adaln_huge_rows_per_sample(hidden):
    """rows_per_sample far beyond rows (here 2^63 - 1) means one sample: the
    result equals rows_per_sample = rows, on the general, vector and two-pass
    kernels (the sample count is computed without overflow)."""
    rows = 6
    announce(f"adaln rows_per_sample 2^63-1 hidden={hidden}")
    x = datagen.make_x(rows, hidden, seed=hidden, stream=1)
    w = datagen.make_w(hidden, seed=hidden, stream=2)
    sc = datagen.make_x(1, hidden, seed=hidden, stream=4, sigma=0.25)
    sh = datagen.make_x(1, hidden, seed=hidden, stream=5, sigma=0.25)
    got = run_adaln(x, w, sc, sh, (1 << 63) - 1)
    assert np.array_equal(got, run_adaln(x, w, sc, sh, rows))
    check_adaln(x, w, sc, sh, rows, label=f"adaln one sample {hidden}")


def test_rope_position_zero_long():
    announce("rope position zero, two-pass and LDS exchange")
    for heads, d in ((16, 72), (129, 136)):
        hidden = heads * d
        x = datagen.make_x(3, hidden, seed=d, stream=1)
        w = datagen.make_w(hidden, seed=d, stream=2)
        c0, s0 = datagen.rope_tables(1, d)
        base = run_rms(x, w)
        assert np.array_equal(run_rope(x, w, c0, s0, heads, d), base)
        assert np.array_equal(run_rope(x, w, c0, s0, heads, d, interleaved=True), base)


@pytest.mark.parametrize("name", list(datagen.GENERAL_CONFIGS))
def test_general_workload_full_size(name):
    """The benchmark's shapes for the kernels of any row length, every
    element, in the launch configuration the benchmark times."""
    cfg = datagen.GENERAL_CONFIGS[name]
    announce(f"general workload {name} rows={cfg.rows} hidden={cfg.hidden}")
    inp = datagen.make_inputs(cfg)
    if cfg.rope:
        got, rep = check_rope(inp["x"], inp["w"], inp["cos"], inp["sin"], cfg.heads, cfg.head_dim,
                              cfg.eps, label=name, interleaved=cfg.interleaved)
        assert rep["n_floor_bound"] <= 1e-5 * rep["n"]
    else:
        got, rep = check_rms(inp["x"], inp["w"], cfg.eps, label=name)
        assert rep["max_ulp"] <= 1.0
    assert rep.get("n_bit_exact", rep.get("n_exact")) >= 0.99 * rep["n"]


# heads packed into wavefronts: non-power-of-two heads whose halves are whole
# vectors, and (16-bit types) halves of an odd number of 4-element groups
PACKED = [(8, d) for d in (24, 40, 56, 72, 88, 104, 120, 136, 184, 248, 80, 96, 112, 160, 192,
                           240)] + [(4, d) for d in (24, 40, 72, 120)]


@pytest.mark.parametrize("epv,head_dim", PACKED)
@pytest.mark.parametrize("heads", [1, 7, 33])
@pytest.mark.parametrize("rows,seq_len", [(7, 3), (300, 4096)])
def test_rope_packed_heads(epv, head_dim, heads, rows, seq_len):
    dtypes = ["bf16", "f16"] if epv == 8 else ["f32"]
    hidden = heads * head_dim
    for dtype in dtypes:
        announce(f"packed rope {dtype} {heads}x{head_dim} rows={rows}")
        x = datagen.make_x(rows, hidden, seed=hidden + rows + 3, stream=1, dtype=dtype)
        w = datagen.make_w(hidden, seed=hidden + rows + 3, stream=2, dtype=dtype)
        c, s = datagen.rope_tables(seq_len, head_dim)
        check_rope(x, w, c, s, heads, head_dim,
                   label=f"packed rope {dtype} {rows}x{heads}x{head_dim}")


@pytest.mark.parametrize("head_dim", [72, 80, 88])
def test_rope_packed_invariants(head_dim):
    """Position 0 is RMSNorm bit for bit; in place equals out of place."""
    heads = 16
    hidden = heads * head_dim
    announce(f"packed rope invariants d={head_dim}")
    x = datagen.make_x(100, hidden, seed=head_dim, stream=1)
    w = datagen.make_w(hidden, seed=head_dim, stream=2)
    c0, s0 = datagen.rope_tables(1, head_dim)
    assert np.array_equal(run_rope(x, w, c0, s0, heads, head_dim), run_rms(x, w))
    c, s = datagen.rope_tables(50, head_dim)
    ref = run_rope(x, w, c, s, heads, head_dim)
    xt = dev_bf16(x)
    ltx.rmsnorm_rope(xt, dev_bf16(w), dev_f32(c), dev_f32(s), heads, head_dim, 1e-6, out=xt)
    assert np.array_equal(host_bits(xt), ref)


# ---------------------------------------------------------------------------
# Element offsets past 2^31: 64-bit row addressing on every path
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("op,hidden,d", [("rms", 2048, 0), ("rms", 3076, 0), ("half", 2048, 64),
                                         ("il", 2048, 64), ("half", 1152, 72), ("adaln", 2048, 0),
                                         ("rms", 128, 0), ("adaln", 576, 0), ("half", 1152, 64)])
def test_offsets_past_2_31(op, hidden, d):
    """A tensor of more than 2^31 elements built on the device by repeating
    one seeded 4096-row block; the last rows (element offsets past 2^31) and
    the first rows are compared with the oracle's result for that block."""
    block_rows = 4096
    reps = (1 << 31) // (block_rows * hidden) + 2
    rows = reps * block_rows
    assert rows * hidden > (1 << 31)
    announce(f"offsets past 2^31 {op} hidden={hidden} rows={rows}")
    xb = datagen.make_x(block_rows, hidden, seed=hidden + d, stream=1)
    w = datagen.make_w(hidden, seed=hidden + d, stream=2)
    xt = torch.empty((rows, hidden), dtype=torch.bfloat16, device=DEV)
    xt.view(reps, block_rows, hidden).copy_(dev_bf16(xb).unsqueeze(0).expand(reps, block_rows, hidden))
    wt = dev_bf16(w)
    c = s = None
    if op in ("half", "il"):
        # one table row per block row, so every block repeat sees the same positions
        c, s = datagen.rope_tables(block_rows, d)
        y = ltx.rmsnorm_rope(xt, wt, dev_f32(c), dev_f32(s), hidden // d, d, 1e-6,
                             interleaved=(op == "il"))
        ref_y, mag = ORC.rmsnorm_rope(xb, w, c, s, hidden // d, d, 1e-6, with_mag=True,
                                      interleaved=(op == "il"))
    elif op == "adaln":
        sc = datagen.make_x(1, hidden, seed=7, stream=4, sigma=0.25)
        sh = datagen.make_x(1, hidden, seed=7, stream=5, sigma=0.25)
        y = ltx.rmsnorm_adaln(xt, wt, dev_bf16(sc), dev_bf16(sh), 1e-6, rows_per_sample=rows)
        ref_y, mag = ORC.rmsnorm_adaln(xb, w, sc, sh, block_rows, 1e-6, with_mag=True)
    else:
        y = ltx.rmsnorm(xt, wt, 1e-6)
        ref_y, mag = ORC.rmsnorm(xb, w, 1e-6), None
    ref32, ref = ORC.round(ref_y)
    for name, sl in (("first block", slice(0, block_rows)), ("last block", slice(rows - block_rows, rows))):
        got = host_bits(y[sl])
        rep = compare(got, ref, mag, ref32)
        assert rep["pass"], (op, hidden, name, rep)
    del xt, y
    torch.cuda.empty_cache()


@pytest.mark.parametrize("op,dtype", [("rms", "bf16"), ("rms", "f32"), ("half", "bf16"),
                                      ("il", "bf16"), ("adaln", "bf16")])
def test_max_hidden(op, dtype):
    """One row of LTXNORM_MAX_HIDDEN (2^24) elements: the two-pass kernel at
    the largest accepted row; one beyond it is refused."""
    hidden = ltx.MAX_HIDDEN
    announce(f"max hidden {op} {dtype}")
    x = datagen.make_x(1, hidden, seed=99, stream=1, dtype=dtype)
    w = datagen.make_w(hidden, seed=99, stream=2, dtype=dtype)
    if op in ("half", "il"):
        d = 4096
        c, s = datagen.rope_tables(1, d)
        check_rope(x, w, c, s, hidden // d, d, interleaved=(op == "il"), label=f"max hidden {op}")
    elif op == "adaln":
        sc = datagen.make_x(1, hidden, seed=98, stream=4, sigma=0.25, dtype=dtype)
        sh = datagen.make_x(1, hidden, seed=98, stream=5, sigma=0.25, dtype=dtype)
        check_adaln(x, w, sc, sh, 1, label="max hidden adaln")
    else:
        check_rms(x, w, label=f"max hidden rms {dtype}")
    xt = dev_bf16(x)
    st = ltx.ltxnorm_rmsnorm_fwd_dt_status(xt, xt, None, 1, hidden + 1, 1e-6,
                                           {"bf16": ltx.BF16, "f16": ltx.F16, "f32": ltx.F32}[dtype], None)
    assert st == ltx.ERR_UNSUPPORTED


# ---------------------------------------------------------------------------
# HIP graph capture: the entry points enqueue kernels only (no memset, no
# allocation), so a captured sequence replays like the eager calls
# ---------------------------------------------------------------------------

def test_graph_capture_replays():
    """Capture one call of each operation (vector, head-packed, general,
    split and two-pass kernels; one-wavefront rows through the wave-priority
    instances, the one with the weight in LDS, and the plain instance of a
    launch too large to be resident at once) into a graph; replay it three
    times with new inputs written eagerly between replays; every replay
    equals the eager result."""
    announce("graph capture")
    shapes = [("rms", 512, 2048, 0), ("adaln", 512, 2048, 0), ("half", 512, 2048, 64),
              ("il", 512, 2048, 64), ("half", 512, 1152, 72), ("rms", 256, 3076, 0),
              ("rms", 2, 70001, 0), ("adaln", 4, 65544, 0), ("il", 3, 255 * 258, 258),
              ("half", 2, 2 * 40000, 40000), ("half", 8192, 2048, 64), ("rms", 16384, 1024, 0)]
    s = torch.cuda.Stream()
    bufs = []
    for op, rows, hidden, d in shapes:
        xt = torch.empty((rows, hidden), dtype=torch.bfloat16, device=DEV)
        yt = torch.empty_like(xt)
        wt = dev_bf16(datagen.make_w(hidden, seed=hidden, stream=2))
        extra = {}
        if d:
            c, sn = datagen.rope_tables(rows, d)
            extra = dict(c=dev_f32(c), s=dev_f32(sn))
        if op == "adaln":
            extra = dict(sc=dev_bf16(datagen.make_x(2, hidden, seed=4, stream=4, sigma=0.25)),
                         sh=dev_bf16(datagen.make_x(2, hidden, seed=4, stream=5, sigma=0.25)))
        bufs.append((op, rows, hidden, d, xt, yt, wt, extra))

    def enqueue():
        for op, rows, hidden, d, xt, yt, wt, e in bufs:
            if op == "rms":
                ltx.rmsnorm(xt, wt, 1e-6, out=yt)
            elif op == "adaln":
                ltx.rmsnorm_adaln(xt, wt, e["sc"], e["sh"], 1e-6, out=yt, rows_per_sample=rows // 2)
            else:
                ltx.rmsnorm_rope(xt, wt, e["c"], e["s"], hidden // d, d, 1e-6, out=yt,
                                 interleaved=(op == "il"))

    def fill(seed):
        for i, (op, rows, hidden, d, xt, yt, wt, e) in enumerate(bufs):
            xt.copy_(dev_bf16(datagen.make_x(rows, hidden, seed=seed * 100 + i, stream=1)))

    fill(1)
    with torch.cuda.stream(s):
        enqueue()  # warm up on the capture stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        enqueue()
    torch.cuda.synchronize()
    for seed in (2, 3, 4):
        fill(seed)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        replayed = [host_bits(b[5]).copy() for b in bufs]
        for b in bufs:
            b[5].zero_()
        enqueue()  # eager, on the current stream
        torch.cuda.synchronize()
        for b, r in zip(bufs, replayed):
            assert np.array_equal(host_bits(b[5]), r), (seed, b[:4])


def _random_cases(n=96, seed=20261202):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = ["bf16", "f16", "f32"][int(rng.integers(0, 3))]
        op = ["rms", "adaln", "half", "il"][int(rng.integers(0, 4))]
        if op in ("half", "il"):
            d = 2 * int(rng.choice([rng.integers(1, 40), rng.integers(1, 300), 32, 36, 64]))
            heads = int(rng.integers(1, max(2, min(64, 40000 // d))))
            hidden = heads * d
        else:
            d = heads = 0
            hidden = int(rng.choice([rng.integers(1, 5000), rng.integers(1, 70000), 8 * rng.integers(1, 3000)]))
        rows = int(rng.integers(1, max(2, min(64, 400000 // hidden))))
        cases.append((i, dtype, op, rows, hidden, heads, d))
    return cases


@pytest.mark.parametrize("case", _random_cases(), ids=lambda c: f"{c[0]}-{c[1]}-{c[2]}-{c[3]}x{c[4]}")
def test_random_shapes(case):
    """Seeded random shapes across operations and dtypes (whichever kernel
    the library picks for each) against the oracle."""
    i, dtype, op, rows, hidden, heads, d = case
    announce(f"random shape {case} -> "
             + ltx.ltxnorm_describe_launch({"rms": ltx.OP_RMSNORM, "adaln": ltx.OP_ADALN, "half": ltx.OP_ROPE,
                                            "il": ltx.OP_ROPE_INTERLEAVED}[op], rows, hidden, heads, d,
                                           {"bf16": ltx.BF16, "f16": ltx.F16, "f32": ltx.F32}[dtype]))
    x = datagen.make_x(rows, hidden, seed=1000 + i, stream=1, dtype=dtype)
    w = datagen.make_w(hidden, seed=1000 + i, stream=2, dtype=dtype)
    if op in ("half", "il"):
        c, s = datagen.rope_tables(int(1 + i % 7), d)
        check_rope(x, w, c, s, heads, d, interleaved=(op == "il"), label=str(case))
    elif op == "adaln":
        rps = max(1, rows // 2)
        samples = -(-rows // rps)
        sc = datagen.make_x(samples, hidden, seed=2000 + i, stream=4, sigma=0.25, dtype=dtype)
        sh = datagen.make_x(samples, hidden, seed=2000 + i, stream=5, sigma=0.25, dtype=dtype)
        check_adaln(x, w, sc, sh, rps, label=str(case))
    else:
        check_rms(x, w, label=str(case))


# ---------------------------------------------------------------------------
# The general kernel's grid holds only the workgroups the device keeps
# resident at once, and each workgroup loops over rows.  Row counts several
# times that capacity exercise the loop: weight chunks reused across rows,
# the rotate-half LDS row reused, cross-wavefront partial sums alternating
# between their two buffers.
# ---------------------------------------------------------------------------

RESIDENT = [  # dtype, op, rows, hidden, head_dim
    ("bf16", "rms", 20000, 1028, 0),     # one wavefront per row, four rows per workgroup
    ("f16", "adaln", 9000, 3076, 0),     # four wavefronts per row, nine samples
    ("bf16", "half", 20000, 1040, 52),   # rotate-half through LDS, four rows per workgroup
    ("f32", "half", 6000, 4100, 82),     # rotate-half through LDS, nine wavefronts per row
    ("bf16", "il", 20000, 1000, 10),     # interleaved pairs, two vectors per lane
    ("f32", "rms", 12000, 1027, 0),      # three wavefronts per row, two rows per workgroup
]
_OPS = {"rms": ltx.OP_RMSNORM, "adaln": ltx.OP_ADALN, "half": ltx.OP_ROPE, "il": ltx.OP_ROPE_INTERLEAVED}
_DT = {"bf16": ltx.BF16, "f16": ltx.F16, "f32": ltx.F32}


@pytest.mark.parametrize("dtype,op,rows,hidden,d", RESIDENT)
def test_resident_grid_many_rows(dtype, op, rows, hidden, d):
    heads = hidden // d if d else 0
    desc = ltx.ltxnorm_describe_launch(_OPS[op], rows, hidden, heads, d, _DT[dtype])
    announce(f"resident grid {dtype} {op} rows={rows} hidden={hidden} d={d} -> {desc}")
    assert desc.startswith("rmsnorm_general_kernel ") and desc.endswith(" grid=resident"), desc
    seed = rows + hidden
    x = datagen.make_x(rows, hidden, seed=seed, stream=1, dtype=dtype)
    w = datagen.make_w(hidden, seed=seed, stream=2, dtype=dtype)
    if op == "rms":
        check_rms(x, w, label=f"resident rms {dtype} {rows}x{hidden}")
    elif op == "adaln":
        rps = 1000
        samples = -(-rows // rps)
        sc = datagen.make_x(samples, hidden, seed=seed, stream=4, sigma=0.25, dtype=dtype)
        sh = datagen.make_x(samples, hidden, seed=seed, stream=5, sigma=0.25, dtype=dtype)
        check_adaln(x, w, sc, sh, rps, label=f"resident adaln {dtype} {rows}x{hidden}")
    else:
        c, s_ = datagen.rope_tables(4096, d)
        check_rope(x, w, c, s_, heads, d, interleaved=(op == "il"),
                   label=f"resident rope {op} {dtype} {rows}x{heads}x{d}")


def test_graph_capture_first_general_launch():
    """The general kernel's first launch at a new size and LDS footprint
    happens inside graph capture, so its occupancy query runs during capture
    too; the captured graph replays to the eager result."""
    heads, d, rows = 7, 38, 9000           # hidden 266: rotate-half through LDS
    hidden = heads * d
    announce("graph capture, first general launch")
    x = dev_bf16(datagen.make_x(rows, hidden, seed=266, stream=1))
    w = dev_bf16(datagen.make_w(hidden, seed=266, stream=2))
    c, sn = datagen.rope_tables(333, d)
    ct, st = dev_f32(c), dev_f32(sn)
    y = torch.empty_like(x)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ltx.rmsnorm_rope(x, w, ct, st, heads, d, 1e-6, out=y)
    torch.cuda.synchronize()
    for _ in range(3):
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(y), host_bits(ltx.rmsnorm_rope(x, w, ct, st, heads, d, 1e-6)))


def test_resident_grid_threads():
    """Eight host threads launch at once, each on its own stream.  Each uses
    rotate-half shapes whose LDS size is new to the process, so the threads
    add to the library's occupancy table concurrently.  Every result matches
    the oracle, and repeats are bit-identical."""
    import threading
    # (heads, head_dim): head sizes only the general kernel pairs (LDS row
    # exchange), a distinct hidden size per thread
    shapes = [(37, 14), (23, 22), (19, 26), (17, 30), (13, 34), (11, 38), (29, 42), (7, 46)]
    rows = 4099
    announce(f"resident grid, {len(shapes)} threads")
    inputs = []
    for heads, d in shapes:
        hidden = heads * d
        x = datagen.make_x(rows, hidden, seed=hidden, stream=1)
        w = datagen.make_w(hidden, seed=hidden, stream=2)
        c, s_ = datagen.rope_tables(97, d)
        inputs.append((heads, d, x, w, c, s_))
    results = [None] * len(shapes)
    errors = []
    barrier = threading.Barrier(len(shapes))

    def work(i):
        try:
            heads, d, x, w, c, s_ = inputs[i]
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                xt, wt, ct, st = dev_bf16(x), dev_bf16(w), dev_f32(c), dev_f32(s_)
                stream.synchronize()
                barrier.wait()
                outs = [ltx.rmsnorm_rope(xt, wt, ct, st, heads, d, 1e-6) for _ in range(3)]
                stream.synchronize()
            results[i] = [host_bits(o) for o in outs]
        except Exception as e:  # reported below, in the test's thread
            errors.append((i, repr(e)))
            barrier.abort()

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(shapes))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not errors, errors
    assert all(not t.is_alive() for t in threads)
    for (heads, d, x, w, c, s_), outs in zip(inputs, results):
        assert all(np.array_equal(outs[0], o) for o in outs[1:])
        y, mag = ORC.rmsnorm_rope(x, w, c, s_, heads, d, 1e-6, with_mag=True)
        ref32, ref = ORC.round(y, "bf16")
        rep = compare(outs[0], ref, mag, ref32)
        assert rep["pass"], (heads, d, rep)


def test_split_streams_concurrent():
    """Four host threads, each on its own stream, run the split kernels at
    once on their own rows: each call stages its partial sums in its own
    output, so concurrent calls do not interfere.  Repeats are bit-identical
    and every result matches the oracle."""
    import threading
    shapes = [("bf16", 262144, 8), ("bf16", 262151, 5), ("f16", 300000, 6), ("f32", 131075, 7)]
    announce(f"split, {len(shapes)} threads on their own streams")
    inputs = []
    for dtype, hidden, rows in shapes:
        code = {"bf16": ltx.BF16, "f16": ltx.F16, "f32": ltx.F32}[dtype]
        desc = ltx.ltxnorm_describe_launch(ltx.OP_RMSNORM, rows, hidden, 0, 0, code)
        assert desc.startswith("rmsnorm_split_kernels"), desc
        x = datagen.make_x(rows, hidden, seed=hidden + rows, stream=1, dtype=dtype)
        w = datagen.make_w(hidden, seed=hidden + rows, stream=2, dtype=dtype)
        inputs.append((x, w))
    results = [None] * len(shapes)
    errors = []
    barrier = threading.Barrier(len(shapes))

    def work(i):
        try:
            x, w = inputs[i]
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                xt, wt = dev_bf16(x), dev_bf16(w)
                stream.synchronize()
                barrier.wait()
                outs = [ltx.rmsnorm(xt, wt, 1e-6) for _ in range(3)]
                stream.synchronize()
            results[i] = [host_bits(o) for o in outs]
        except Exception as e:  # reported below, in the test's thread
            errors.append((i, repr(e)))
            barrier.abort()

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(shapes))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not errors, errors
    assert all(not t.is_alive() for t in threads)
    for (x, w), outs in zip(inputs, results):
        assert all(np.array_equal(outs[0], o) for o in outs[1:])
        ref32, ref = ORC.round(ORC.rmsnorm(x, w, 1e-6), kind(x))
        rep = compare(outs[0], ref, None, ref32)
        assert rep["pass"], rep


# ---------------------------------------------------------------------------
# Short rows (at most 32 vectors): several rows per wavefront
# ---------------------------------------------------------------------------

SHORT = {"bf16": [8, 16, 24, 40, 64, 96, 128, 192, 256], "f16": [8, 64, 128, 256],
         "f32": [4, 8, 12, 20, 32, 64, 96, 128]}


@pytest.mark.parametrize("dtype,hidden", [(dt, h) for dt, hs in SHORT.items() for h in hs])
@pytest.mark.parametrize("rows", [1, 5, 63, 1000, 4097])
def test_short_rows(dtype, hidden, rows):
    announce(f"short rows {dtype} rows={rows} hidden={hidden}")
    seed = 7 * hidden + rows
    x = datagen.make_x(rows, hidden, seed=seed, stream=1, dtype=dtype)
    w = datagen.make_w(hidden, seed=seed, stream=2, dtype=dtype)
    got, rep = check_rms(x, w, label=f"short rms {dtype} {rows}x{hidden}")
    if dtype != "f32":
        assert rep["max_ulp"] <= 1.0
    rps = max(1, rows // 3)
    samples = -(-rows // rps)
    sc = datagen.make_x(samples, hidden, seed=seed, stream=4, sigma=0.25, dtype=dtype)
    sh = datagen.make_x(samples, hidden, seed=seed, stream=5, sigma=0.25, dtype=dtype)
    check_adaln(x, w, sc, sh, rps, label=f"short adaln {dtype} {rows}x{hidden}")
    E = 4 if dtype == "f32" else 8
    # RoPE with one or two heads per row (per-head rows), both pairings
    for heads in (1, 2):
        d = hidden // heads
        if hidden % heads or d % 2:
            continue
        c, s_ = datagen.rope_tables(int(1 + rows % 11), d)
        P = d // (2 * E) if d % (2 * E) == 0 else 0
        check_rope(x, w, c, s_, heads, d, label=f"short rope {dtype} {rows}x{heads}x{d}")
        check_rope(x, w, c, s_, heads, d, interleaved=True, label=f"short rope-il {dtype} {rows}x{heads}x{d}")


def test_short_rows_invariants():
    """Per-head rows: NULL weight = ones, in place = out of place, run to run
    identical, position 0 = RMSNorm, NULL modulation = RMSNorm."""
    announce("short rows invariants")
    x = datagen.make_x(3000, 128, seed=5, stream=1)
    w = datagen.make_w(128, seed=5, stream=2)
    base = run_rms(x, w)
    assert np.array_equal(base, run_rms(x, w))
    assert np.array_equal(run_rms(x, None), run_rms(x, np.full(128, 0x3F80, dtype=np.uint16)))
    xt = dev_bf16(x)
    ltx.rmsnorm(xt, dev_bf16(w), 1e-6, out=xt)
    assert np.array_equal(host_bits(xt), base)
    c0, s0 = datagen.rope_tables(1, 128)
    assert np.array_equal(run_rope(x, w, c0, s0, 1, 128), base)
    assert np.array_equal(run_rope(x, w, c0, s0, 1, 128, interleaved=True), base)
    assert np.array_equal(run_adaln(x, w, None, None, 1000), base)
    # in place with rotation (partners exchanged between lanes)
    c, s = datagen.rope_tables(17, 128)
    ref = run_rope(x, w, c, s, 1, 128)
    xt = dev_bf16(x)
    ltx.rmsnorm_rope(xt, dev_bf16(w), dev_f32(c), dev_f32(s), 1, 128, 1e-6, out=xt)
    assert np.array_equal(host_bits(xt), ref)


# One-wavefront rows: a launch whose whole grid is resident at once takes the
# instance that raises the wave priority for its loads (load_priority=one_wave
# in the describe line); a larger launch of the same shape takes the plain
# instance.  RMSNorm rows of 3 or 4 wavefronts likewise take one wavefront of
# 6 or 8 vectors per lane (one_wave_vectors_per_lane), adding in the split's
# order.  Neither changes a bit: the first rows of a large call and the same
# rows called alone must agree bit for bit, and both with the oracle.
# (dtype, op, hidden, head_dim, rows called alone)
ONE_WAVE = [
    ("bf16", "rms", 2048, 0, 1024), ("f16", "rms", 1024, 0, 1024), ("f32", "rms", 1024, 0, 1024),
    ("bf16", "adaln", 2048, 0, 1024), ("f32", "adaln", 512, 0, 1024),
    ("bf16", "half", 2048, 64, 1024),   # power-of-two half heads (lane exchange)
    ("bf16", "il", 2048, 64, 1024),     # interleaved, one table slice per row
    ("bf16", "il", 1152, 72, 1024),     # interleaved, a table slice per slot
    ("bf16", "half", 1152, 72, 1024),   # heads packed into wavefronts, odd groups
    ("bf16", "half", 1280, 80, 1024),   # heads packed into wavefronts, whole vectors
    # lane exchange at more rows than the register-weight instance holds at
    # once: the instance with the weight in LDS (4, 3 and 4 masked vectors
    # per lane)
    ("bf16", "half", 2048, 64, 8192), ("f16", "half", 1536, 64, 8192), ("bf16", "half", 2032, 16, 7000),
    # AdaLN's priority instance (weight in LDS, modulation after the
    # reduction) at the most rows it holds at once, whole and masked
    ("bf16", "adaln", 2048, 0, 8192), ("f32", "adaln", 1024, 0, 8192), ("f16", "adaln", 2040, 0, 6000),
    # RMSNorm rows of 3 or 4 wavefronts x 2 vectors: alone, one wavefront of
    # 6 or 8 vectors per lane adding in the same order (whole and masked
    # rows); inside the large call, the split itself
    ("bf16", "rms", 3072, 0, 8192), ("bf16", "rms", 2560, 0, 8192), ("bf16", "rms", 4096, 0, 4096),
    ("f16", "rms", 3584, 0, 6000), ("f32", "rms", 2048, 0, 8192), ("f32", "rms", 1028, 0, 8192),
    # AdaLN and rotate-half RoPE rows of 2 wavefronts x 3 or 4 vectors, and
    # interleaved RoPE rows of 2 x 3, 3 x 2 or 4 x 2, regrouped the same way
    ("bf16", "adaln", 3072, 0, 4096), ("bf16", "adaln", 2304, 0, 8000), ("f32", "adaln", 2048, 0, 6000),
    ("f16", "adaln", 4096, 0, 3000),
    ("bf16", "half", 3072, 128, 4096), ("bf16", "half", 4096, 128, 3000), ("f32", "half", 2048, 64, 6000),
    ("bf16", "il", 3072, 128, 8192), ("bf16", "il", 2560, 128, 6000), ("f16", "il", 4096, 128, 4096),
    # head-packed rotate-half at more rows than its register-weight priority
    # instance holds: the form with the weight in LDS (odd and even groups)
    ("bf16", "half", 1152, 72, 8192), ("f16", "half", 1280, 80, 8192), ("bf16", "half", 1080, 24, 7500),
    # interleaved with a table slice per slot, the same way
    ("bf16", "il", 1152, 72, 8192), ("f16", "il", 1152, 24, 8000),
    # segmented rows (8-32 per workgroup): the large call needs more rows to
    # exceed one wave
    ("bf16", "rms", 576, 0, 16384, 131072), ("bf16", "adaln", 1152, 0, 8192, 65536),
    ("f16", "rms", 256, 0, 32768, 262144), ("bf16", "il", 576, 64, 16384, 131072),
]
ONE_WAVE = [c if len(c) == 6 else c + (16384,) for c in ONE_WAVE]


@pytest.mark.parametrize("dtype,op,hidden,d,small,big", ONE_WAVE)
def test_one_wave_priority_instances_agree(dtype, op, hidden, d, small, big):
    # big: more workgroups (4096 of 4 one-wavefront rows, or of 8-32
    # segmented rows) than any device holds at once
    heads = hidden // d if d else 0
    desc = ltx.ltxnorm_describe_launch(_OPS[op], big, hidden, heads, d, _DT[dtype])
    announce(f"one-wave priority {dtype} {op} hidden={hidden} d={d} rows={small} -> {desc}")
    assert ("load_priority=one_wave" in desc and (" wavefronts_per_row=1 " in desc or " lanes_per_row=" in desc)
            or " one_wave_vectors_per_lane=" in desc), desc
    seed = 7 * hidden + d
    x = datagen.make_x(big, hidden, seed=seed, stream=1, dtype=dtype)
    w = datagen.make_w(hidden, seed=seed, stream=2, dtype=dtype)
    rps = 512
    sc = datagen.make_x(-(-big // rps), hidden, seed=seed, stream=4, sigma=0.25, dtype=dtype)
    sh = datagen.make_x(-(-big // rps), hidden, seed=seed, stream=5, sigma=0.25, dtype=dtype)
    c, s_ = datagen.rope_tables(3000, d) if d else (None, None)

    def call(rows):
        xt, wt = dev_bf16(x[:rows]), dev_bf16(w)
        if op == "rms":
            y = ltx.rmsnorm(xt, wt, 1e-6)
        elif op == "adaln":
            n = -(-rows // rps)
            y = ltx.rmsnorm_adaln(xt, wt, dev_bf16(sc[:n]), dev_bf16(sh[:n]), 1e-6, rows_per_sample=rps)
        else:
            y = ltx.rmsnorm_rope(xt, wt, dev_f32(c), dev_f32(s_), heads, d, 1e-6, interleaved=(op == "il"))
        b = host_bits(y)
        return b.view(np.uint32) if b.dtype == np.float32 else b.view(np.uint16)

    alone = call(small)
    assert np.array_equal(alone, call(big)[:small])
    xs = x[:small]
    if op == "rms":
        ref32, ref = ORC.round(ORC.rmsnorm(xs, w, 1e-6), kind(xs))
        mag = None
    elif op == "adaln":
        y, mag = ORC.rmsnorm_adaln(xs, w, sc[:-(-small // rps)], sh[:-(-small // rps)], rps, 1e-6, with_mag=True)
        ref32, ref = ORC.round(y, kind(xs))
    else:
        y, mag = ORC.rmsnorm_rope(xs, w, c, s_, heads, d, 1e-6, with_mag=True, interleaved=(op == "il"))
        ref32, ref = ORC.round(y, kind(xs))
    got = {"f32": alone.view(np.float32), "f16": alone.view(np.float16)}.get(dtype, alone)
    rep = compare(got, ref, mag, ref32)
    assert rep["pass"], rep
