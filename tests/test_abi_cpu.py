"""The C-ABI library without a GPU: it loads, exports every function the
header declares, and rejects bad arguments on the host before any HIP call.

Only calls that fail validation (or have rows == 0) are made here; those
return before the library touches the HIP runtime, so fake addresses are
never dereferenced."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import rmsnorm_video_dit_amd as ltx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ltxnorm.h")

A = 0x10000  # a 16-byte aligned fake device address (never dereferenced)
MB = 1 << 20
OK_IF_VALID = "shape accepted"  # sentinel: the shape passes, alignment is what fails


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ltxnorm_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    ops = ["ltxnorm_rmsnorm_adaln_fwd", "ltxnorm_rmsnorm_fwd", "ltxnorm_rmsnorm_rope_fwd",
           "ltxnorm_rmsnorm_rope_interleaved_fwd"]
    assert declared_functions() == sorted(ops + [o + "_dt" for o in ops] +
                                          ["ltxnorm_describe_launch", "ltxnorm_status_str",
                                           "ltxnorm_version"])


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(ltx.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", ltx.LIB_PATH], capture_output=True, text=True)
    exported = set(re.findall(r"\bT (ltxnorm_\w+)", nm.stdout))
    assert exported == set(declared_functions())


def test_library_targets_gfx950_only():
    """The offload bundle inside the library (built here) names one target."""
    data = open(ltx.LIB_PATH, "rb").read()
    targets = set(re.findall(rb"amdgcn-amd-amdhsa-+(gfx[0-9a-z]+)", data))
    assert targets == {b"gfx950"}, targets


def test_version_and_status_strings():
    assert ltx.ltxnorm_version() == 4
    seen = set()
    for code in range(8):
        s = ltx.ltxnorm_status_str(code)
        assert s and s not in seen
        seen.add(s)
    assert ltx.ltxnorm_status_str(99) == "unknown ltxnorm status"
    assert ltx.ltxnorm_status_str(0) == "ok"


def rms(out=A, x=A + 64 * MB, w=None, rows=4, hidden=2048, eps=1e-6):
    return ltx.ltxnorm_rmsnorm_fwd_status(out, x, w, rows, hidden, eps, 0)


def rope(out=A, x=A + 64 * MB, w=None, c=A + 128 * MB, s=A + 129 * MB, rows=4, hidden=2048,
         heads=32, head_dim=64, seq_len=16, eps=1e-6):
    return ltx.ltxnorm_rmsnorm_rope_fwd_status(out, x, w, c, s, rows, hidden, heads, head_dim,
                                               seq_len, eps, 0)


@pytest.mark.parametrize("kw,status", [
    (dict(rows=-1), ltx.ERR_SHAPE),
    (dict(hidden=0), ltx.ERR_SHAPE),
    (dict(hidden=-8), ltx.ERR_SHAPE),
    (dict(hidden=(1 << 24) + 1), ltx.ERR_UNSUPPORTED),
    (dict(hidden=1 << 30), ltx.ERR_UNSUPPORTED),
    (dict(hidden=2047, out=A + 2), ltx.ERR_ALIGN),   # any H passes the shape check
    (dict(hidden=1, out=A + 2), ltx.ERR_ALIGN),
    (dict(hidden=65544, out=A + 2), ltx.ERR_ALIGN),  # beyond the registers: two-pass
    (dict(rows=1 << 62), ltx.ERR_SHAPE),
    (dict(eps=-1e-6), ltx.ERR_VALUE),
    (dict(eps=float("nan")), ltx.ERR_VALUE),
    (dict(eps=float("inf")), ltx.ERR_VALUE),
    (dict(out=None), ltx.ERR_NULL),
    (dict(x=None), ltx.ERR_NULL),
    (dict(out=A + 2), ltx.ERR_ALIGN),
    (dict(x=A + 64 * MB + 8), ltx.ERR_ALIGN),
    (dict(w=A + 200 * MB + 4), ltx.ERR_ALIGN),
    (dict(x=A + 4096), ltx.ERR_ALIAS),            # partial overlap, out before x
    (dict(out=A + 64 * MB + 16), ltx.ERR_ALIAS),  # partial overlap, out after x
    (dict(w=A + 1024), ltx.ERR_ALIAS),            # weight inside out
])
def test_rmsnorm_validation(kw, status):
    assert rms(**kw) == status


def test_rmsnorm_empty_is_ok_without_pointers():
    assert rms(out=None, x=None, rows=0) == ltx.OK
    assert rope(out=None, x=None, c=None, s=None, rows=0) == ltx.OK


@pytest.mark.parametrize("kw,status", [
    (dict(hidden=2048, heads=16), ltx.ERR_SHAPE),         # hidden != heads * head_dim
    (dict(hidden=1280, heads=32, head_dim=40, out=A + 2), ltx.ERR_ALIGN),  # any even head_dim
    (dict(hidden=256, heads=32, head_dim=8, out=A + 2), ltx.ERR_ALIGN),
    (dict(hidden=66, heads=33, head_dim=2, out=A + 2), ltx.ERR_ALIGN),
    (dict(hidden=96, heads=32, head_dim=3), ltx.ERR_SHAPE),    # odd head_dim
    (dict(hidden=0, heads=32, head_dim=0), ltx.ERR_SHAPE),
    (dict(heads=0), ltx.ERR_SHAPE),
    (dict(seq_len=0), ltx.ERR_SHAPE),
    (dict(c=None), ltx.ERR_NULL),
    (dict(s=None), ltx.ERR_NULL),
    (dict(c=A + 128 * MB + 8), ltx.ERR_ALIGN),
    (dict(s=A + 129 * MB + 4), ltx.ERR_ALIGN),
    (dict(c=A + 256), ltx.ERR_ALIAS),
    (dict(s=A - 64), ltx.ERR_ALIAS),   # table [A-64, A-64+8192) reaches into out
    (dict(x=A + 2), ltx.ERR_ALIGN),
    (dict(eps=-0.5), ltx.ERR_VALUE),
])
def test_rope_validation(kw, status):
    assert rope(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(hidden=2048, heads=16, head_dim=64), ltx.ERR_SHAPE),   # hidden != heads * head_dim
    (dict(hidden=96, heads=8, head_dim=12), OK_IF_VALID),     # any even head_dim
    (dict(hidden=192, heads=8, head_dim=24), OK_IF_VALID),
    (dict(hidden=88, heads=8, head_dim=11), ltx.ERR_SHAPE),    # odd head_dim
    (dict(seq_len=0), ltx.ERR_SHAPE),
    (dict(c=None), ltx.ERR_NULL),
    (dict(s=A + 129 * MB + 8), ltx.ERR_ALIGN),
    (dict(c=A + 512), ltx.ERR_ALIAS),
])
def test_rope_interleaved_validation(kw, status):
    args = dict(out=A, x=A + 64 * MB, w=None, c=A + 128 * MB, s=A + 129 * MB, rows=4,
                hidden=2048, heads=32, head_dim=64, seq_len=16, eps=1e-6)
    args.update(kw)
    if status == OK_IF_VALID:
        # a valid call would launch: check instead that the shape passes by
        # making only the alignment wrong
        args["out"] = A + 2
        status = ltx.ERR_ALIGN
    st = ltx.ltxnorm_rmsnorm_rope_interleaved_fwd_status(
        args["out"], args["x"], args["w"], args["c"], args["s"], args["rows"], args["hidden"],
        args["heads"], args["head_dim"], args["seq_len"], args["eps"], 0)
    assert st == status


@pytest.mark.parametrize("kw,status", [
    (dict(rows_per_sample=0), ltx.ERR_SHAPE),
    (dict(hidden=(1 << 24) + 8), ltx.ERR_UNSUPPORTED),
    (dict(hidden=12, out=A + 2), ltx.ERR_ALIGN),   # any H passes the shape check
    (dict(eps=-1.0), ltx.ERR_VALUE),
    (dict(out=None), ltx.ERR_NULL),
    (dict(scale=A + 200 * MB + 2), ltx.ERR_ALIGN),
    (dict(shift=A + 201 * MB + 8), ltx.ERR_ALIGN),
    (dict(scale=A + 1024), ltx.ERR_ALIAS),
    (dict(shift=A - 64), ltx.ERR_ALIAS),
    (dict(rows=0, out=None, x=None), ltx.OK),
    # a huge rows_per_sample means one sample: its row overlaps out's last
    # 16 bytes (the sample count must not overflow on the way)
    (dict(rows_per_sample=(1 << 63) - 1, scale=A + 8 * 2048 * 2 - 16), ltx.ERR_ALIAS),
    (dict(rows_per_sample=(1 << 63) - 1, shift=A + 8 * 2048 * 2 - 16), ltx.ERR_ALIAS),
])
def test_adaln_validation(kw, status):
    args = dict(out=A, x=A + 64 * MB, w=None, scale=A + 200 * MB, shift=A + 201 * MB, rows=8,
                hidden=2048, rows_per_sample=4, eps=1e-6)
    args.update(kw)
    st = ltx.ltxnorm_rmsnorm_adaln_fwd_status(args["out"], args["x"], args["w"], args["scale"],
                                              args["shift"], args["rows"], args["hidden"],
                                              args["rows_per_sample"], args["eps"], 0)
    assert st == status


# (dtype, hidden) -> status; only shapes the library rejects (a valid call
# would launch)
@pytest.mark.parametrize("dtype,hidden,status", [
    (3, 2048, ltx.ERR_UNSUPPORTED),             # unknown dtype
    (-1, 2048, ltx.ERR_UNSUPPORTED),
    (ltx.F16, (1 << 24) + 2, ltx.ERR_UNSUPPORTED),   # above LTXNORM_MAX_HIDDEN
    (ltx.F32, (1 << 24) + 1, ltx.ERR_UNSUPPORTED),
    (ltx.F32, 0, ltx.ERR_SHAPE),
])
def test_dtype_validation(dtype, hidden, status):
    assert ltx.ltxnorm_rmsnorm_fwd_dt_status(A, A + 64 * MB, None, 4, hidden, 1e-6, dtype, 0) == status
    assert ltx.ltxnorm_rmsnorm_adaln_fwd_dt_status(A, A + 64 * MB, None, None, None, 4, hidden, 2,
                                                   1e-6, dtype, 0) == status


@pytest.mark.parametrize("dtype,hidden", [
    (ltx.F32, 2052), (ltx.F32, 32768), (ltx.F16, 2056), (ltx.F16, 2044), (ltx.F32, 2042),
    (ltx.F32, 32772), (ltx.F16, 65544), (ltx.BF16, 1 << 24), (ltx.F32, 1 << 24), (ltx.F16, 3),
])
def test_dtype_shapes_that_pass_validation(dtype, hidden):
    """Any hidden from 1 to LTXNORM_MAX_HIDDEN is accepted in every dtype:
    shown by making only the alignment wrong."""
    assert ltx.ltxnorm_rmsnorm_fwd_dt_status(A + 4, A + 64 * MB, None, 4, hidden, 1e-6, dtype, 0) == ltx.ERR_ALIGN


@pytest.mark.parametrize("dtype,interleaved,head_dim,status", [
    (ltx.F32, False, 8, ltx.ERR_ALIGN),
    (ltx.F32, False, 12, ltx.ERR_ALIGN),
    (ltx.F32, True, 4, ltx.ERR_ALIGN),
    (ltx.F32, True, 6, ltx.ERR_ALIGN),
    (ltx.F16, False, 16, ltx.ERR_ALIGN),
    (ltx.F16, False, 8, ltx.ERR_ALIGN),
    (ltx.F16, True, 8, ltx.ERR_ALIGN),
    (ltx.F16, True, 12, ltx.ERR_ALIGN),
    (ltx.F16, True, 7, ltx.ERR_SHAPE),       # odd head_dim: no pairs
    (ltx.F32, False, 5, ltx.ERR_SHAPE),
    (ltx.BF16, False, 0, ltx.ERR_SHAPE),
])
def test_rope_dtype_head_dim_rules(dtype, interleaved, head_dim, status):
    """Any even head_dim passes in every dtype (ERR_ALIGN: the shape passed;
    out is deliberately misaligned)."""
    heads = 24
    fn = (ltx.ltxnorm_rmsnorm_rope_interleaved_fwd_dt_status if interleaved
          else ltx.ltxnorm_rmsnorm_rope_fwd_dt_status)
    st = fn(A + 2, A + 64 * MB, None, A + 128 * MB, A + 129 * MB, 4, heads * head_dim, heads,
            head_dim, 16, 1e-6, dtype, 0)
    assert st == status


def test_python_front_end_refuses_host_tensors():
    import torch
    x = torch.zeros(2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ltx.rmsnorm(x)
    with pytest.raises(ValueError):
        ltx.rmsnorm(x.to(torch.float16))
    with pytest.raises(ValueError):
        ltx.rmsnorm_rope(x, None, torch.zeros(4, 8), torch.zeros(4, 8), 4, 16)


class FakeDeviceTensor:
    """Stands in for a GPU tensor in the binding's argument checks: a shape, a
    dtype and a fake aligned address that nothing dereferences (every call
    below fails its checks before any launch)."""
    is_cuda = True

    def __init__(self, shape, dtype, addr):
        self.shape, self.dtype, self.addr = tuple(shape), dtype, addr

    def is_contiguous(self):
        return True

    def numel(self):
        return int(np.prod(self.shape)) if self.shape else 1

    def dim(self):
        return len(self.shape)

    def data_ptr(self):
        return self.addr


@pytest.mark.parametrize("op", ["rmsnorm", "rope", "adaln"])
@pytest.mark.parametrize("wlen", [2047, 2049, 1])
def test_front_end_refuses_a_weight_of_the_wrong_length(op, wlen):
    """The kernels read hidden weight values: a shorter (or longer) weight is
    refused by the binding before the library is called."""
    import torch
    bf = torch.bfloat16
    x = FakeDeviceTensor((2, 4, 2048), bf, A + 64 * MB)
    out = FakeDeviceTensor((2, 4, 2048), bf, A)
    w = FakeDeviceTensor((wlen,), bf, A + 128 * MB)
    with pytest.raises(ValueError, match="weight must hold"):
        if op == "rmsnorm":
            ltx.rmsnorm(x, w, out=out)
        elif op == "rope":
            tab = FakeDeviceTensor((4, 32), torch.float32, A + 130 * MB)
            ltx.rmsnorm_rope(x, w, tab, tab, 32, 64, out=out)
        else:
            ltx.rmsnorm_adaln(x, w, None, None, out=out)


@pytest.mark.parametrize("rps", [0, -1, -4096])
def test_front_end_passes_rows_per_sample_to_the_library(rps, monkeypatch):
    """rows_per_sample below 1 reaches the C ABI unchanged, which refuses it
    with LTXNORM_ERR_SHAPE before any HIP call (the stream handle is never
    used)."""
    import torch
    monkeypatch.setattr(ltx, "_stream", lambda s: 0)
    bf = torch.bfloat16
    x = FakeDeviceTensor((8, 2048), bf, A + 64 * MB)
    out = FakeDeviceTensor((8, 2048), bf, A)
    with pytest.raises(ltx.LtxnormError) as e:
        ltx.rmsnorm_adaln(x, None, None, None, out=out, rows_per_sample=rps)
    assert e.value.status == ltx.ERR_SHAPE


def test_error_raises_with_status():
    with pytest.raises(ltx.LtxnormError) as e:
        ltx.ltxnorm_rmsnorm_fwd(A, A + 64 * MB, None, 4, (1 << 24) + 1, 1e-6, 0)
    assert e.value.status == ltx.ERR_UNSUPPORTED


# ---------------------------------------------------------------------------
# Kernel choice (host logic): which kernel and row split serve a shape
# ---------------------------------------------------------------------------

def _describe(op, hidden, heads=0, head_dim=0, dtype=ltx.BF16, rows=16384):
    d = ltx.ltxnorm_describe_launch(op, rows, hidden, heads, head_dim, dtype)
    name, *fields = d.split()
    return name, dict(f.split("=") for f in fields)


@pytest.mark.parametrize("op,hidden,heads,head_dim,dtype,kernel,wpr,per", [
    # the measured plans: one wavefront x 4 vectors at 2048, 3 x 2 at 3072
    (ltx.OP_RMSNORM, 2048, 0, 0, ltx.BF16, "rmsnorm_kernel", 1, 4),
    (ltx.OP_RMSNORM, 3072, 0, 0, ltx.BF16, "rmsnorm_kernel", 3, 2),
    (ltx.OP_RMSNORM, 3072, 0, 0, ltx.F16, "rmsnorm_kernel", 3, 2),
    (ltx.OP_RMSNORM, 3072, 0, 0, ltx.F32, "rmsnorm_kernel", 6, 2),
    (ltx.OP_RMSNORM, 65536, 0, 0, ltx.BF16, "rmsnorm_kernel", 16, 8),
    (ltx.OP_ADALN, 2048, 0, 0, ltx.BF16, "rmsnorm_adaln_kernel", 1, 4),
    # AdaLN and the fused RoPE kernels: rows of 257..768 vectors over 2-3
    # wavefronts with 3-4 vectors per lane; longer rows keep the 2-vector split
    (ltx.OP_ADALN, 2304, 0, 0, ltx.BF16, "rmsnorm_adaln_kernel", 2, 3),
    (ltx.OP_ADALN, 3072, 0, 0, ltx.BF16, "rmsnorm_adaln_kernel", 2, 3),
    (ltx.OP_ADALN, 4096, 0, 0, ltx.F16, "rmsnorm_adaln_kernel", 2, 4),
    (ltx.OP_ADALN, 5120, 0, 0, ltx.BF16, "rmsnorm_adaln_kernel", 3, 4),
    (ltx.OP_ADALN, 2048, 0, 0, ltx.F32, "rmsnorm_adaln_kernel", 2, 4),
    (ltx.OP_ADALN, 8192, 0, 0, ltx.BF16, "rmsnorm_adaln_kernel", 8, 2),
    # rows that are not whole vectors, and rows past the register budget
    (ltx.OP_RMSNORM, 3076, 0, 0, ltx.BF16, "rmsnorm_general_kernel", 4, 2),
    (ltx.OP_RMSNORM, 1, 0, 0, ltx.BF16, "rmsnorm_general_kernel", 1, 1),
    (ltx.OP_ADALN, 3070, 0, 0, ltx.F32, "rmsnorm_general_kernel", 7, 2),
    # (16384 rows fill the GPU with one workgroup per row: two passes)
    (ltx.OP_RMSNORM, 65544, 0, 0, ltx.BF16, "rmsnorm_long_kernel", None, None),
    (ltx.OP_RMSNORM, 32772, 0, 0, ltx.F32, "rmsnorm_long_kernel", None, None),
    (ltx.OP_ADALN, 262144, 0, 0, ltx.BF16, "rmsnorm_long_kernel", None, None),
    # rotate-half: power-of-two half heads, head-packed lanes, pairs in a lane,
    # LDS exchange, two passes
    (ltx.OP_ROPE, 2048, 32, 64, ltx.BF16, "rmsnorm_rope_xor_kernel", 1, 4),
    (ltx.OP_ROPE, 3072, 24, 128, ltx.BF16, "rmsnorm_rope_xor_kernel", 2, 3),
    (ltx.OP_ROPE, 4608, 36, 128, ltx.BF16, "rmsnorm_rope_xor_kernel", 3, 3),
    (ltx.OP_ROPE, 5120, 40, 128, ltx.BF16, "rmsnorm_rope_xor_kernel", 4, 3),
    (ltx.OP_ROPE, 6144, 48, 128, ltx.BF16, "rmsnorm_rope_xor_kernel", 4, 3),
    (ltx.OP_ROPE, 8192, 64, 128, ltx.BF16, "rmsnorm_rope_xor_kernel", 4, 4),      # 4 vectors past 768
    (ltx.OP_ROPE, 16384, 128, 128, ltx.BF16, "rmsnorm_rope_xor_kernel", 8, 4),
    (ltx.OP_ROPE, 65536, 512, 128, ltx.BF16, "rmsnorm_rope_xor_kernel", 16, 8),
    (ltx.OP_ROPE_INTERLEAVED, 8192, 64, 128, ltx.BF16, "rmsnorm_rope_interleaved_kernel(shared)", 8, 2),
    (ltx.OP_ROPE, 1152, 16, 72, ltx.BF16, "rmsnorm_rope_packed_kernel(odd)", 1, 3),
    (ltx.OP_ROPE, 2560, 32, 80, ltx.BF16, "rmsnorm_rope_packed_kernel", 2, 3),
    (ltx.OP_ROPE, 3072, 32, 96, ltx.BF16, "rmsnorm_rope_packed_kernel", 2, 4),
    (ltx.OP_ROPE, 2304, 32, 72, ltx.BF16, "rmsnorm_rope_packed_kernel(odd)", 2, 3),
    (ltx.OP_ROPE, 960, 24, 40, ltx.F32, "rmsnorm_rope_packed_kernel", 1, 4),
    (ltx.OP_ROPE, 3072, 3, 1024, ltx.BF16, "rmsnorm_rope_pair_kernel", 3, 1),
    (ltx.OP_ROPE, 1040, 20, 52, ltx.BF16, "rmsnorm_general_kernel", 1, 3),
    (ltx.OP_ROPE, 17544, 129, 136, ltx.BF16, "rmsnorm_rope_packed_kernel(odd)", 16, 3),
    (ltx.OP_ROPE, 80000, 2, 40000, ltx.BF16, "rmsnorm_long_kernel", None, None),
    (ltx.OP_ROPE, 65790, 255, 258, ltx.BF16, "rmsnorm_long_kernel", None, None),
    # interleaved: one table slice per row when a head's vectors divide the lanes
    (ltx.OP_ROPE_INTERLEAVED, 2048, 32, 64, ltx.BF16, "rmsnorm_rope_interleaved_kernel(shared)", 1, 4),
    (ltx.OP_ROPE_INTERLEAVED, 1728, 24, 72, ltx.BF16, "rmsnorm_rope_interleaved_kernel", 1, 4),
    # ... the wide split only for 257..320 vectors
    (ltx.OP_ROPE_INTERLEAVED, 2304, 18, 128, ltx.BF16, "rmsnorm_rope_interleaved_kernel(shared)", 2, 3),
    (ltx.OP_ROPE_INTERLEAVED, 2520, 35, 72, ltx.BF16, "rmsnorm_rope_interleaved_kernel", 2, 3),
    (ltx.OP_ROPE_INTERLEAVED, 3072, 24, 128, ltx.BF16, "rmsnorm_rope_interleaved_kernel(shared)", 3, 2),
    (ltx.OP_ROPE_INTERLEAVED, 70, 7, 10, ltx.BF16, "rmsnorm_general_kernel", 1, 1),
    # short rows (at most 32 vectors): lanes per row given in the wpr column
    # (two vectors per lane on half the lanes; per column: vectors per lane)
    (ltx.OP_RMSNORM, 128, 0, 0, ltx.BF16, "rmsnorm_short_kernel", 8, 2),
    (ltx.OP_RMSNORM, 8, 0, 0, ltx.BF16, "rmsnorm_short_kernel", 1, 1),
    (ltx.OP_RMSNORM, 16, 0, 0, ltx.BF16, "rmsnorm_short_kernel", 2, 1),
    (ltx.OP_RMSNORM, 72, 0, 0, ltx.BF16, "rmsnorm_short_kernel", 8, 2),
    (ltx.OP_ROPE, 128, 1, 128, ltx.BF16, "rmsnorm_short_kernel", 8, 2),   # partner in the lane's other slot
    (ltx.OP_RMSNORM, 96, 0, 0, ltx.F16, "rmsnorm_short_kernel", 8, 2),
    (ltx.OP_RMSNORM, 128, 0, 0, ltx.F32, "rmsnorm_short_kernel", 16, 2),
    (ltx.OP_ADALN, 256, 0, 0, ltx.BF16, "rmsnorm_short_kernel", 16, 2),
    (ltx.OP_ROPE, 64, 1, 64, ltx.BF16, "rmsnorm_short_kernel", 8, 1),    # partner 4 lanes away
    (ltx.OP_ROPE, 256, 2, 128, ltx.BF16, "rmsnorm_short_kernel", 16, 2),
    (ltx.OP_ROPE_INTERLEAVED, 128, 2, 64, ltx.BF16, "rmsnorm_short_kernel", 8, 2),
    (ltx.OP_ROPE, 144, 2, 72, ltx.BF16, "rmsnorm_rope_packed_kernel(odd)", 1, 1),   # not a power of two
    # rows of 33..160 vectors in segments of 16 or 32 lanes with 3 or 5 vectors
    # per lane where that fills more of a wavefront (wpr column: lanes, per:
    # vectors per lane); rows near a multiple of 64 vectors keep one wavefront
    (ltx.OP_RMSNORM, 264, 0, 0, ltx.BF16, "rmsnorm_short_kernel", 16, 3),             # 33 vectors
    (ltx.OP_RMSNORM, 320, 0, 0, ltx.BF16, "rmsnorm_short_kernel", 16, 3),
    (ltx.OP_ADALN, 576, 0, 0, ltx.BF16, "rmsnorm_short_kernel", 16, 5),
    (ltx.OP_RMSNORM, 704, 0, 0, ltx.F16, "rmsnorm_short_kernel", 32, 3),
    (ltx.OP_ADALN, 1152, 0, 0, ltx.BF16, "rmsnorm_short_kernel", 32, 5),
    (ltx.OP_ADALN, 576, 0, 0, ltx.F32, "rmsnorm_short_kernel", 32, 5),               # 144 fp32 vectors
    (ltx.OP_ROPE, 1152, 18, 64, ltx.BF16, "rmsnorm_short_kernel", 32, 5),
    (ltx.OP_ROPE_INTERLEAVED, 1152, 16, 72, ltx.BF16, "rmsnorm_rope_interleaved_kernel", 1, 3),  # no 32 x 5
    (ltx.OP_RMSNORM, 1152, 0, 0, ltx.BF16, "rmsnorm_kernel", 1, 3),
    (ltx.OP_ROPE_INTERLEAVED, 576, 8, 72, ltx.BF16, "rmsnorm_short_kernel", 16, 5),
    (ltx.OP_ROPE, 640, 5, 128, ltx.BF16, "rmsnorm_short_kernel", 16, 5),
    (ltx.OP_ROPE, 640, 2, 320, ltx.BF16, "rmsnorm_rope_pair_kernel", 1, 1),          # not a power of two
    (ltx.OP_ROPE, 1280, 5, 256, ltx.BF16, "rmsnorm_short_kernel", 32, 5),            # partner 16 lanes away
    (ltx.OP_RMSNORM, 1000, 0, 0, ltx.BF16, "rmsnorm_kernel", 1, 2),                  # 125 vectors
    (ltx.OP_RMSNORM, 512, 0, 0, ltx.BF16, "rmsnorm_short_kernel", 32, 2),             # 64 vectors
    (ltx.OP_RMSNORM, 1024, 0, 0, ltx.BF16, "rmsnorm_kernel", 1, 2),                  # 128 vectors
])
def test_kernel_choice(op, hidden, heads, head_dim, dtype, kernel, wpr, per):
    name, f = _describe(op, hidden, heads, head_dim, dtype)
    assert name == kernel, (name, f)
    if name == "rmsnorm_short_kernel":
        lanes = int(f["lanes_per_row"])
        assert lanes == wpr and int(f["rows_per_wavefront"]) == 64 // lanes
        assert int(f["rows_per_block"]) == 4 * (64 // lanes) and f["threads"] == "256"
        assert int(f["vectors_per_lane"]) == (per or 1)
    elif wpr is not None:
        assert int(f["wavefronts_per_row"]) == wpr
        per_key = "pairs_per_lane" if "pair" in name else "vectors_per_lane"
        assert int(f[per_key]) == per
        assert int(f["threads"]) == 64 * wpr * int(f["rows_per_block"])
        assert (f.get("grid") == "resident") == (name == "rmsnorm_general_kernel"), f
    elif name == "rmsnorm_split_kernels":
        E = 4 if dtype == ltx.F32 else 8
        touched = hidden // E if hidden % E == 0 else (hidden + 2 * E - 2) // E
        assert int(f["chunks_per_row"]) == per == -(-touched // 2048)
        assert f["launches"] == "3" and f["vectors_per_chunk"] == "2048" and f["threads"] == "256"
        assert f["in_place"] == "rmsnorm_long_kernel"
    else:
        assert f["passes"] == "2" and f["threads"] == "1024"


@pytest.mark.parametrize("op,hidden,heads,head_dim,dtype,rows,chunks", [
    # fewer than 624 rows of at least 16 chunks of 2048 vectors: the split
    (ltx.OP_RMSNORM, 262144, 0, 0, ltx.BF16, 191, 16),
    (ltx.OP_RMSNORM, 245761, 0, 0, ltx.BF16, 1, 16),      # 30722 vectors touched
    (ltx.OP_RMSNORM, 1 << 20, 0, 0, ltx.BF16, 64, 64),
    (ltx.OP_RMSNORM, 131072, 0, 0, ltx.F32, 100, 16),
    (ltx.OP_ADALN, 262144, 0, 0, ltx.F16, 7, 16),
    (ltx.OP_ROPE_INTERLEAVED, 1 << 24, 1024, 1 << 14, ltx.BF16, 3, 1024),
    (ltx.OP_RMSNORM, 1 << 24, 0, 0, ltx.F32, 1, 2048),
    # otherwise two passes in one workgroup per row
    (ltx.OP_RMSNORM, 262144, 0, 0, ltx.BF16, 623, 16),
    (ltx.OP_RMSNORM, 262144, 0, 0, ltx.BF16, 624, None),
    (ltx.OP_RMSNORM, 131072, 0, 0, ltx.BF16, 300, None),  # 8 chunks
    (ltx.OP_RMSNORM, 245752, 0, 0, ltx.BF16, 1, None),     # 30719 vectors: 15 chunks
    (ltx.OP_RMSNORM, 65544, 0, 0, ltx.BF16, 64, None),
    (ltx.OP_RMSNORM, (1 << 24) - 1, 0, 0, ltx.F32, 1, None),  # 2049 chunks
    (ltx.OP_ROPE, 1 << 20, 1024, 1024, ltx.BF16, 1, None),  # rotate-half
])
def test_kernel_choice_long_rows(op, hidden, heads, head_dim, dtype, rows, chunks):
    """Rows past the register budget: chunks over many workgroups for a few
    rows of many chunks, the two-pass kernel otherwise.  The describe line
    of the split names the two-pass kernel an in-place call takes."""
    name, f = _describe(op, hidden, heads, head_dim, dtype, rows=rows)
    if chunks is None:
        assert name == "rmsnorm_long_kernel"
        assert f["passes"] == "2" and f["threads"] == "1024"
    else:
        assert name == "rmsnorm_split_kernels"
        assert int(f["chunks_per_row"]) == chunks
        assert f["launches"] == "3" and f["vectors_per_chunk"] == "2048" and f["threads"] == "256"
        assert f["in_place"] == "rmsnorm_long_kernel"
        # the second launch's slots per row: every chunk, padded to a multiple
        # of the 8 XCDs where one XCD then runs at most 2 % less work
        n = chunks
        slots = int(f["slots_per_row"])
        assert slots == (n + 7) // 8 * 8 if (n + 7) // 8 * 8 * 50 <= n * 51 else slots == n


def test_split_slots_padding():
    """Chunk slots per row: a count that is a multiple of 8 needs no padding;
    63 chunks pad to 64 (one XCD 1.6 % short); 17 and 125 chunks stay
    unpadded (one XCD would run 30 / 2.4 % short)."""
    for hidden, dtype, slots in ((262144, ltx.BF16, 16), (524288, ltx.BF16, 32), (1 << 20, ltx.BF16, 64),
                                 (63 * 16384, ltx.BF16, 64), (1 << 21, ltx.BF16, 128), (1 << 24, ltx.F32, 2048),
                                 (17 * 16384, ltx.BF16, 17), (16 * 16384 + 8, ltx.BF16, 17),
                                 (125 * 16384, ltx.BF16, 125)):
        name, f = _describe(ltx.OP_RMSNORM, hidden, dtype=dtype, rows=4)
        assert name == "rmsnorm_split_kernels" and int(f["slots_per_row"]) == slots, (hidden, f)


def test_kernel_choice_lds_and_limits():
    """The LDS exchange takes one binary32 row per row slot; shapes that the
    entry points refuse are refused with the same status; no rows, no launch."""
    name, f = _describe(ltx.OP_ROPE, 1040, 20, 52)
    assert int(f["lds_bytes"]) == 1040 * 4 * int(f["rows_per_block"])
    assert ltx.ltxnorm_describe_launch(ltx.OP_RMSNORM, 0, 2048) == "none"
    for args, status in (((ltx.OP_ROPE, 16, 2048, 16, 64), ltx.ERR_SHAPE),
                         ((ltx.OP_ROPE, 16, 96, 32, 3), ltx.ERR_SHAPE),
                         ((ltx.OP_RMSNORM, 16, (1 << 24) + 1, 0, 0), ltx.ERR_UNSUPPORTED),
                         ((ltx.OP_RMSNORM, -1, 2048, 0, 0), ltx.ERR_SHAPE),
                         ((7, 16, 2048, 0, 0), ltx.ERR_UNSUPPORTED)):
        with pytest.raises(ltx.LtxnormError) as e:
            ltx.ltxnorm_describe_launch(*args)
        assert e.value.status == status, args
    lib = ltx.lib()
    assert lib.ltxnorm_describe_launch(0, 16, 2048, 0, 0, 0, None, 0) == ltx.OK
    assert lib.ltxnorm_describe_launch(0, 16, 2048, 0, 0, 0, None, 8) == ltx.ERR_NULL
    buf = ctypes.create_string_buffer(8)
    assert lib.ltxnorm_describe_launch(0, 16, 3072, 0, 0, 0, buf, 8) == ltx.OK
    assert buf.value == b"rmsnorm"  # truncated, NUL-terminated


def test_kernel_choice_covers_the_benchmark_workloads():
    """Every benchmark workload maps to the kernel its profile names."""
    import datagen
    expect = {"rms_4x4096x3072": "rmsnorm_kernel", "rope_2x4096x2048_h32d64": "rmsnorm_rope_xor_kernel",
              "ropei_2x4096x2048_h32d64": "rmsnorm_rope_interleaved_kernel(shared)",
              "adaln_2x4096x2048": "rmsnorm_adaln_kernel", "rms_4x4096x3076": "rmsnorm_general_kernel",
              "rope_2x4096x1152_h16d72": "rmsnorm_rope_packed_kernel(odd)",
              "rms_1x512x131072": "rmsnorm_long_kernel", "rms_1x64x1048576": "rmsnorm_split_kernels"}
    for name, kernel in expect.items():
        cfg = {**datagen.CONFIGS, **datagen.GENERAL_CONFIGS}[name]
        op = (ltx.OP_ADALN if cfg.adaln else ltx.OP_ROPE_INTERLEAVED if cfg.interleaved
              else ltx.OP_ROPE if cfg.rope else ltx.OP_RMSNORM)
        got = ltx.ltxnorm_describe_launch(op, cfg.rows, cfg.hidden, cfg.heads, cfg.head_dim)
        assert got.split()[0] == kernel, (name, got)


def test_kernel_choice_always_covers_the_row():
    """For seeded random shapes in every dtype and operation, the plan the
    library picks covers every vector (or pair unit) of the row with its
    lanes, within the kernel's limits: the property every launch relies on."""
    rng = np.random.default_rng(20261202)
    epv = {ltx.BF16: 8, ltx.F16: 8, ltx.F32: 4}
    seen = set()
    for _ in range(1500):
        dtype = int(rng.choice([ltx.BF16, ltx.F16, ltx.F32]))
        E = epv[dtype]
        op = int(rng.integers(0, 4))
        if op in (ltx.OP_ROPE, ltx.OP_ROPE_INTERLEAVED):
            d = 2 * int(rng.choice([rng.integers(1, 40), rng.integers(1, 600), 32, 36, 64]))
            heads = int(rng.integers(1, max(2, min(200, 70000 // d))))
            H = heads * d
        else:
            d = heads = 0
            H = int(rng.choice([rng.integers(1, 9000), rng.integers(1, 80000), 8 * rng.integers(1, 9000),
                                rng.integers(1, 1 << 19)]))
        rows = int(rng.choice([rng.integers(1, 5000), rng.integers(1, 300)]))
        desc = ltx.ltxnorm_describe_launch(op, rows, H, heads, d, dtype)
        name, *fields = desc.split()
        f = dict(x.split("=") for x in fields)
        seen.add(name)
        whole = H % E == 0
        touched = H // E if whole else (H + 2 * E - 2) // E
        chunks = -(-touched // 2048)
        if name == "rmsnorm_long_kernel":
            assert f["threads"] == "1024"
            assert op == ltx.OP_ROPE or not 16 <= chunks <= 2048 or rows >= 624, desc
            continue
        if name == "rmsnorm_split_kernels":
            assert op != ltx.OP_ROPE and int(f["chunks_per_row"]) == chunks and 16 <= chunks <= 2048, desc
            assert rows < 624, desc
            continue
        if name == "rmsnorm_short_kernel":
            lanes, per, n = int(f["lanes_per_row"]), int(f["vectors_per_lane"]), H // E
            assert whole and lanes <= 32 and lanes & (lanes - 1) == 0
            assert int(f["rows_per_wavefront"]) * lanes == 64
            if per == 1:    # one vector: rows of up to 8, or rotate-half partners too far
                assert n <= 8 or (op == ltx.OP_ROPE and n <= 32), desc
                assert lanes >= n and (lanes == 1 or lanes // 2 < n)
            elif per == 2:  # 9..64 vectors: half the power of two at or above n
                assert 9 <= n <= 64 and not 32 < n <= 48, desc
                assert lanes == 1 << ((n - 1).bit_length() - 1), desc
            else:           # segments: fewer slots than one wavefront per row
                assert (lanes, per) in ((16, 3), (16, 5), (32, 3), (32, 5)), desc
                assert (lanes, per) != (32, 5) or op in (ltx.OP_ADALN, ltx.OP_ROPE), desc
                assert 32 < n <= lanes * per < 64 * -(-n // 64), desc
            if op == ltx.OP_ROPE:
                P = d // (2 * E)
                assert d % (2 * E) == 0 and P & (P - 1) == 0
                assert 2 * P <= lanes or (per == 2 and P == lanes), desc
            if op == ltx.OP_ROPE_INTERLEAVED:
                assert d % E == 0
            continue
        wpr, rpb, threads = int(f["wavefronts_per_row"]), int(f["rows_per_block"]), int(f["threads"])
        assert 1 <= wpr <= 16 and threads == 64 * wpr * rpb <= 1024
        wide = (name in ("rmsnorm_adaln_kernel", "rmsnorm_rope_xor_kernel") and 256 < touched <= 768) or \
            (name.startswith("rmsnorm_rope_packed_kernel") and 256 < -(-touched * 64 // (64 - 64 % (d // E))) <= 768) or \
            (name.startswith("rmsnorm_rope_interleaved_kernel") and 256 < touched <= 320)
        if wide:  # two or three wavefronts with 3-4 vectors per lane, or four with 3
            per = int(f["vectors_per_lane"])
            four = name == "rmsnorm_rope_xor_kernel" and touched > 576
            assert (wpr, per) == (4, 3) if four else (wpr in (2, 3) and 3 <= per <= 4), desc
        else:
            assert wpr != 2, desc
        if name == "rmsnorm_rope_xor_kernel" and touched > 768:  # 4 vectors per lane
            assert int(f["vectors_per_lane"]) == 4 or wpr == 16, desc
        assert rpb == (4 if wpr == 1 else 2 if wpr <= 3 else 1)
        if name == "rmsnorm_rope_pair_kernel":
            per = int(f["pairs_per_lane"])
            assert whole and d % (2 * E) == 0 and 64 * wpr * per >= H // (2 * E) and per <= 4
            continue
        per = int(f["vectors_per_lane"])
        if name == "rmsnorm_general_kernel":
            assert 64 * wpr * per >= touched and per <= 5
            if op == ltx.OP_ROPE:
                assert int(f["lds_bytes"]) == 4 * H * rpb <= 64 * 1024 - 256
            continue
        assert whole and int(f["lds_bytes"]) == 0 and per <= 8
        nvec = H // E
        if name.startswith("rmsnorm_rope_packed_kernel"):
            vph = d // E
            lw = 64 - 64 % vph
            assert vph <= 32 and lw * wpr * per >= nvec
            assert (d % (2 * E) == 0) != name.endswith("(odd)")
            continue
        assert 64 * wpr * per >= nvec
        if name == "rmsnorm_rope_xor_kernel":
            P = d // (2 * E)
            assert d % (2 * E) == 0 and P & (P - 1) == 0 and P <= 32
        elif name.startswith("rmsnorm_rope_interleaved_kernel"):
            assert d % E == 0
            assert name.endswith("(shared)") == ((64 * wpr) % (d // E) == 0)
        else:
            assert name in ("rmsnorm_kernel", "rmsnorm_adaln_kernel"), desc
    # the sample reaches every kernel family
    assert {"rmsnorm_kernel", "rmsnorm_adaln_kernel", "rmsnorm_rope_xor_kernel",
            "rmsnorm_rope_packed_kernel", "rmsnorm_rope_packed_kernel(odd)", "rmsnorm_rope_pair_kernel",
            "rmsnorm_rope_interleaved_kernel", "rmsnorm_rope_interleaved_kernel(shared)",
            "rmsnorm_general_kernel", "rmsnorm_long_kernel", "rmsnorm_split_kernels",
            "rmsnorm_short_kernel"} <= seen, seen


@pytest.mark.parametrize("op,rows,hidden,heads,head_dim,dtype,want", [
    # rows of several wavefronts: always (RMSNorm, AdaLN); never (RoPE)
    (ltx.OP_RMSNORM, 16384, 3072, 0, 0, ltx.BF16, "always"),
    (ltx.OP_ADALN, 16384, 3072, 0, 0, ltx.BF16, "always"),
    (ltx.OP_ROPE, 16384, 3072, 24, 128, ltx.BF16, "never"),
    (ltx.OP_ROPE_INTERLEAVED, 16384, 3072, 24, 128, ltx.BF16, "never"),
    # one-wavefront rows: when the grid is resident at once
    (ltx.OP_RMSNORM, 8192, 2048, 0, 0, ltx.BF16, "one_wave"),
    (ltx.OP_ADALN, 8192, 2048, 0, 0, ltx.F16, "one_wave"),
    (ltx.OP_ROPE, 8192, 2048, 32, 64, ltx.BF16, "one_wave"),
    (ltx.OP_ROPE_INTERLEAVED, 8192, 2048, 32, 64, ltx.BF16, "one_wave"),
    (ltx.OP_ROPE, 8192, 1152, 16, 72, ltx.BF16, "one_wave"),
    # the general kernel always; the pair-in-lane RoPE never
    (ltx.OP_RMSNORM, 16384, 3076, 0, 0, ltx.BF16, "always"),
    (ltx.OP_ROPE, 8192, 2560, 8, 320, ltx.BF16, "never"),
])
def test_describe_load_priority(op, rows, hidden, heads, head_dim, dtype, want):
    """The launch line states when the kernel raises wave priority for its
    loads; the segmented-row kernel does when its grid fits at once, and the
    two-pass and split kernels carry no such field."""
    name, f = _describe(op, hidden, heads, head_dim, dtype, rows=rows)
    assert f["load_priority"] == want, (name, f)
    name, f = _describe(ltx.OP_RMSNORM, 128, rows=8192)
    assert name == "rmsnorm_short_kernel" and f["load_priority"] == "one_wave", (name, f)
    for args in [(ltx.OP_RMSNORM, 4, 1 << 20), (ltx.OP_RMSNORM, 512, 131072)]:
        assert "load_priority" not in ltx.ltxnorm_describe_launch(*args), args


@pytest.mark.parametrize("dtype,hidden,want", [
    (ltx.BF16, 3072, 6), (ltx.BF16, 2312, 6), (ltx.BF16, 4096, 8), (ltx.F16, 3584, 8), (ltx.F32, 2048, 8),
    (ltx.F32, 1028, 6), (ltx.BF16, 2048, None), (ltx.BF16, 5120, None), (ltx.BF16, 3076, None),
])
def test_describe_one_wave_regroup(dtype, hidden, want):
    """RMSNorm rows of 3 or 4 wavefronts x 2 vectors name the one-wavefront
    form they take when the whole grid is resident at once; other splits,
    the general kernel and the other operations do not."""
    name, f = _describe(ltx.OP_RMSNORM, hidden, dtype=dtype, rows=8192)
    if want is None:
        assert "one_wave_vectors_per_lane" not in f, (name, f)
    else:
        assert name == "rmsnorm_kernel" and f["vectors_per_lane"] == "2", (name, f)
        assert int(f["one_wave_vectors_per_lane"]) == want == 2 * int(f["wavefronts_per_row"]), (name, f)


@pytest.mark.parametrize("op,hidden,heads,head_dim,dtype,want", [
    (ltx.OP_ADALN, 3072, 0, 0, ltx.BF16, 6), (ltx.OP_ADALN, 4096, 0, 0, ltx.BF16, 8),
    (ltx.OP_ADALN, 2048, 0, 0, ltx.F32, 8), (ltx.OP_ADALN, 5120, 0, 0, ltx.BF16, None),
    (ltx.OP_ROPE, 3072, 24, 128, ltx.BF16, 6), (ltx.OP_ROPE, 4096, 32, 128, ltx.BF16, 8),
    (ltx.OP_ROPE, 5120, 40, 128, ltx.BF16, None), (ltx.OP_ROPE, 2048, 32, 64, ltx.BF16, None),
    (ltx.OP_ROPE_INTERLEAVED, 3072, 24, 128, ltx.BF16, 6), (ltx.OP_ROPE_INTERLEAVED, 2560, 20, 128, ltx.BF16, 6),
    (ltx.OP_ROPE_INTERLEAVED, 4096, 32, 128, ltx.BF16, 8),
    # a head of 48 vectors is shared by 3 wavefronts' lanes, not by one's
    (ltx.OP_ROPE_INTERLEAVED, 3072, 8, 384, ltx.BF16, None),
])
def test_describe_one_wave_regroup_fused(op, hidden, heads, head_dim, dtype, want):
    """AdaLN and the fused RoPE kernels name their one-wavefront form for
    the splits that have one (2 wavefronts x 3 or 4 vectors; interleaved
    also 3 or 4 x 2, where a head's vectors divide one wavefront's lanes)."""
    name, f = _describe(op, hidden, heads, head_dim, dtype, rows=8192)
    got = f.get("one_wave_vectors_per_lane")
    if want is None:
        assert got is None, (name, f)
    else:
        assert int(got) == want == int(f["wavefronts_per_row"]) * int(f["vectors_per_lane"]), (name, f)
