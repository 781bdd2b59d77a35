"""Python binding of libltxnorm.so: gfx950 RMSNorm and fused RMSNorm + RoPE.

Argument marshalling only.  Every step of both ops runs in the HIP kernels of
``csrc/ltxnorm.hip`` behind the C ABI declared in ``include/ltxnorm.h``; this
module converts tensors to device pointers and the current torch stream to a
``hipStream_t``.  There is no fallback: if the library is not built, or a
tensor is not on the GPU, calls raise.

The low-level functions keep the C names and argument order:

    ltxnorm_rmsnorm_fwd(out, x, weight, rows, hidden, eps, stream)
    ltxnorm_rmsnorm_rope_fwd(out, x, weight, cos_tab, sin_tab, rows, hidden,
                             heads, head_dim, seq_len, eps, stream)
    ltxnorm_rmsnorm_rope_interleaved_fwd(... same arguments ...)
    ltxnorm_rmsnorm_adaln_fwd(out, x, weight, scale, shift, rows, hidden,
                              rows_per_sample, eps, stream)
    and a ``_dt`` twin of each taking ``dtype`` (BF16, F16 or F32) before stream
    ltxnorm_status_str(status), ltxnorm_version()

Pointer arguments accept a torch tensor, an integer address or None; ``stream``
accepts a ``torch.cuda.Stream``, an integer handle, or None for torch's
current stream.  A non-OK status raises ``LtxnormError``.

``rmsnorm(x, weight=None, eps=1e-6, out=None)``, ``rmsnorm_rope(...)`` and
``rmsnorm_adaln(...)`` are the tensor-level forms (functional, or out-variant
when ``out`` is given); they take bfloat16, float16 or float32 tensors.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libltxnorm.so")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_UNSUPPORTED, ERR_ALIAS, ERR_VALUE, ERR_HIP = range(8)
BF16, F16, F32 = 0, 1, 2
OP_RMSNORM, OP_ROPE, OP_ROPE_INTERLEAVED, OP_ADALN = 0, 1, 2, 3
MAX_HIDDEN = 1 << 24

_lib = None


class LtxnormError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {ltxnorm_status_str(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """The loaded libltxnorm.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                "(or python -m rmsnorm_video_dit_amd._build); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        p, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
        L.ltxnorm_rmsnorm_fwd.argtypes = [p, p, p, i64, i64, f32, p]
        L.ltxnorm_rmsnorm_fwd.restype = ctypes.c_int
        L.ltxnorm_rmsnorm_rope_fwd.argtypes = [p, p, p, p, p, i64, i64, i32, i32, i64, f32, p]
        L.ltxnorm_rmsnorm_rope_fwd.restype = ctypes.c_int
        L.ltxnorm_rmsnorm_rope_interleaved_fwd.argtypes = [p, p, p, p, p, i64, i64, i32, i32, i64,
                                                           f32, p]
        L.ltxnorm_rmsnorm_rope_interleaved_fwd.restype = ctypes.c_int
        L.ltxnorm_rmsnorm_adaln_fwd.argtypes = [p, p, p, p, p, i64, i64, i64, f32, p]
        L.ltxnorm_rmsnorm_adaln_fwd.restype = ctypes.c_int
        c_int = ctypes.c_int
        for name in ("ltxnorm_rmsnorm_fwd", "ltxnorm_rmsnorm_rope_fwd",
                     "ltxnorm_rmsnorm_rope_interleaved_fwd", "ltxnorm_rmsnorm_adaln_fwd"):
            base = getattr(L, name)
            twin = getattr(L, name + "_dt")
            twin.argtypes = list(base.argtypes[:-1]) + [c_int, p]
            twin.restype = ctypes.c_int
        L.ltxnorm_status_str.argtypes = [ctypes.c_int]
        L.ltxnorm_status_str.restype = ctypes.c_char_p
        L.ltxnorm_version.argtypes = []
        L.ltxnorm_version.restype = ctypes.c_int
        L.ltxnorm_describe_launch.argtypes = [c_int, i64, i64, i32, i32, c_int, ctypes.c_char_p,
                                              ctypes.c_size_t]
        L.ltxnorm_describe_launch.restype = ctypes.c_int
        _lib = L
    return _lib


def _addr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def ltxnorm_status_str(status: int) -> str:
    return lib().ltxnorm_status_str(int(status)).decode()


def ltxnorm_version() -> int:
    return lib().ltxnorm_version()


def ltxnorm_describe_launch(op: int, rows: int, hidden: int, heads: int = 0, head_dim: int = 0,
                            dtype: int = BF16) -> str:
    """The kernel and launch shape a call would use (no GPU needed); raises
    LtxnormError with the status the entry point would return for bad shapes."""
    buf = ctypes.create_string_buffer(256)
    st = lib().ltxnorm_describe_launch(int(op), int(rows), int(hidden), int(heads), int(head_dim),
                                       int(dtype), buf, len(buf))
    _raise_if(st, "ltxnorm_describe_launch")
    return buf.value.decode()


def ltxnorm_rmsnorm_fwd_status(out, x, weight, rows, hidden, eps, stream) -> int:
    """Same call, returning the raw status code instead of raising."""
    return lib().ltxnorm_rmsnorm_fwd(_addr(out), _addr(x), _addr(weight), int(rows), int(hidden),
                                     float(eps), _stream(stream))


def ltxnorm_rmsnorm_fwd_dt_status(out, x, weight, rows, hidden, eps, dtype, stream) -> int:
    return lib().ltxnorm_rmsnorm_fwd_dt(_addr(out), _addr(x), _addr(weight), int(rows),
                                        int(hidden), float(eps), int(dtype), _stream(stream))


def ltxnorm_rmsnorm_rope_fwd_dt_status(out, x, weight, cos_tab, sin_tab, rows, hidden, heads,
                                       head_dim, seq_len, eps, dtype, stream) -> int:
    return lib().ltxnorm_rmsnorm_rope_fwd_dt(_addr(out), _addr(x), _addr(weight), _addr(cos_tab),
                                             _addr(sin_tab), int(rows), int(hidden), int(heads),
                                             int(head_dim), int(seq_len), float(eps), int(dtype),
                                             _stream(stream))


def ltxnorm_rmsnorm_rope_interleaved_fwd_dt_status(out, x, weight, cos_tab, sin_tab, rows, hidden,
                                                   heads, head_dim, seq_len, eps, dtype,
                                                   stream) -> int:
    return lib().ltxnorm_rmsnorm_rope_interleaved_fwd_dt(
        _addr(out), _addr(x), _addr(weight), _addr(cos_tab), _addr(sin_tab), int(rows),
        int(hidden), int(heads), int(head_dim), int(seq_len), float(eps), int(dtype),
        _stream(stream))


def ltxnorm_rmsnorm_adaln_fwd_dt_status(out, x, weight, scale, shift, rows, hidden,
                                        rows_per_sample, eps, dtype, stream) -> int:
    return lib().ltxnorm_rmsnorm_adaln_fwd_dt(_addr(out), _addr(x), _addr(weight), _addr(scale),
                                              _addr(shift), int(rows), int(hidden),
                                              int(rows_per_sample), float(eps), int(dtype),
                                              _stream(stream))


def _raise_if(st, where):
    if st != OK:
        raise LtxnormError(st, where)


def ltxnorm_rmsnorm_fwd_dt(out, x, weight, rows, hidden, eps, dtype, stream=None) -> None:
    _raise_if(ltxnorm_rmsnorm_fwd_dt_status(out, x, weight, rows, hidden, eps, dtype, stream),
              "ltxnorm_rmsnorm_fwd_dt")


def ltxnorm_rmsnorm_rope_fwd_dt(out, x, weight, cos_tab, sin_tab, rows, hidden, heads, head_dim,
                                seq_len, eps, dtype, stream=None) -> None:
    _raise_if(ltxnorm_rmsnorm_rope_fwd_dt_status(out, x, weight, cos_tab, sin_tab, rows, hidden,
                                                 heads, head_dim, seq_len, eps, dtype, stream),
              "ltxnorm_rmsnorm_rope_fwd_dt")


def ltxnorm_rmsnorm_rope_interleaved_fwd_dt(out, x, weight, cos_tab, sin_tab, rows, hidden, heads,
                                            head_dim, seq_len, eps, dtype, stream=None) -> None:
    _raise_if(ltxnorm_rmsnorm_rope_interleaved_fwd_dt_status(out, x, weight, cos_tab, sin_tab,
                                                             rows, hidden, heads, head_dim,
                                                             seq_len, eps, dtype, stream),
              "ltxnorm_rmsnorm_rope_interleaved_fwd_dt")


def ltxnorm_rmsnorm_adaln_fwd_dt(out, x, weight, scale, shift, rows, hidden, rows_per_sample, eps,
                                 dtype, stream=None) -> None:
    _raise_if(ltxnorm_rmsnorm_adaln_fwd_dt_status(out, x, weight, scale, shift, rows, hidden,
                                                  rows_per_sample, eps, dtype, stream),
              "ltxnorm_rmsnorm_adaln_fwd_dt")


def ltxnorm_rmsnorm_rope_fwd_status(out, x, weight, cos_tab, sin_tab, rows, hidden, heads,
                                    head_dim, seq_len, eps, stream) -> int:
    return lib().ltxnorm_rmsnorm_rope_fwd(_addr(out), _addr(x), _addr(weight), _addr(cos_tab),
                                          _addr(sin_tab), int(rows), int(hidden), int(heads),
                                          int(head_dim), int(seq_len), float(eps), _stream(stream))


def ltxnorm_rmsnorm_rope_interleaved_fwd_status(out, x, weight, cos_tab, sin_tab, rows, hidden,
                                                heads, head_dim, seq_len, eps, stream) -> int:
    return lib().ltxnorm_rmsnorm_rope_interleaved_fwd(
        _addr(out), _addr(x), _addr(weight), _addr(cos_tab), _addr(sin_tab), int(rows),
        int(hidden), int(heads), int(head_dim), int(seq_len), float(eps), _stream(stream))


def ltxnorm_rmsnorm_adaln_fwd_status(out, x, weight, scale, shift, rows, hidden, rows_per_sample,
                                     eps, stream) -> int:
    return lib().ltxnorm_rmsnorm_adaln_fwd(_addr(out), _addr(x), _addr(weight), _addr(scale),
                                           _addr(shift), int(rows), int(hidden),
                                           int(rows_per_sample), float(eps), _stream(stream))


def ltxnorm_rmsnorm_adaln_fwd(out, x, weight, scale, shift, rows, hidden, rows_per_sample, eps,
                              stream=None) -> None:
    st = ltxnorm_rmsnorm_adaln_fwd_status(out, x, weight, scale, shift, rows, hidden,
                                          rows_per_sample, eps, stream)
    if st != OK:
        raise LtxnormError(st, "ltxnorm_rmsnorm_adaln_fwd")


def ltxnorm_rmsnorm_fwd(out, x, weight, rows, hidden, eps, stream=None) -> None:
    st = ltxnorm_rmsnorm_fwd_status(out, x, weight, rows, hidden, eps, stream)
    if st != OK:
        raise LtxnormError(st, "ltxnorm_rmsnorm_fwd")


def ltxnorm_rmsnorm_rope_fwd(out, x, weight, cos_tab, sin_tab, rows, hidden, heads, head_dim,
                             seq_len, eps, stream=None) -> None:
    st = ltxnorm_rmsnorm_rope_fwd_status(out, x, weight, cos_tab, sin_tab, rows, hidden, heads,
                                         head_dim, seq_len, eps, stream)
    if st != OK:
        raise LtxnormError(st, "ltxnorm_rmsnorm_rope_fwd")


def ltxnorm_rmsnorm_rope_interleaved_fwd(out, x, weight, cos_tab, sin_tab, rows, hidden, heads,
                                         head_dim, seq_len, eps, stream=None) -> None:
    st = ltxnorm_rmsnorm_rope_interleaved_fwd_status(out, x, weight, cos_tab, sin_tab, rows,
                                                     hidden, heads, head_dim, seq_len, eps, stream)
    if st != OK:
        raise LtxnormError(st, "ltxnorm_rmsnorm_rope_interleaved_fwd")


def _dtype_code(t):
    import torch
    codes = {torch.bfloat16: BF16, torch.float16: F16, torch.float32: F32}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}: use bfloat16, float16 or float32")
    return codes[t.dtype]


def _check_act(x, name, like=None):
    if not x.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (no host path exists)")
    _dtype_code(x)
    if like is not None and x.dtype != like.dtype:
        raise TypeError(f"{name} must have the dtype of x ({like.dtype}), got {x.dtype}")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_weight(weight, x):
    """The weight is [hidden] in x's dtype: the kernels read exactly hidden
    values from it, so a shorter tensor is refused here, before any launch."""
    if weight is None:
        return
    _check_act(weight, "weight", x)
    hidden = x.shape[-1] if x.dim() else 0
    if weight.numel() != hidden:
        raise ValueError(f"weight must hold hidden = {hidden} values, got {weight.numel()}")


def rmsnorm(x, weight=None, eps: float = 1e-6, out=None):
    """RMSNorm over the last dimension of ``x`` (bf16, fp16 or fp32; weight
    [H] of the same dtype, or None)."""
    import torch
    _check_act(x, "x")
    _check_weight(weight, x)
    hidden = x.shape[-1]
    if out is None:
        out = torch.empty_like(x)
    else:
        _check_act(out, "out", x)
        if out.shape != x.shape:
            raise ValueError("out must have the shape of x")
    rows = x.numel() // hidden if hidden else 0
    ltxnorm_rmsnorm_fwd_dt(out, x, weight, rows, hidden, eps, _dtype_code(x), None)
    return out


def rmsnorm_rope(x, weight, cos_tab, sin_tab, heads: int, head_dim: int, eps: float = 1e-6,
                 out=None, interleaved: bool = False):
    """RMSNorm over the full last dimension (heads*head_dim), then RoPE per
    head: rotate-half pairs (i, i + d/2), or adjacent pairs (2i, 2i + 1) with
    ``interleaved``; row r uses table row r mod cos_tab.shape[0]."""
    import torch
    _check_act(x, "x")
    _check_weight(weight, x)
    for t, n in ((cos_tab, "cos_tab"), (sin_tab, "sin_tab")):
        if not t.is_cuda or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous float32 GPU tensor")
    if cos_tab.shape != sin_tab.shape or cos_tab.dim() != 2 or cos_tab.shape[1] != head_dim // 2:
        raise ValueError("cos_tab and sin_tab must both be [seq_len, head_dim/2]")
    hidden = x.shape[-1]
    if out is None:
        out = torch.empty_like(x)
    else:
        _check_act(out, "out", x)
        if out.shape != x.shape:
            raise ValueError("out must have the shape of x")
    rows = x.numel() // hidden if hidden else 0
    fn = ltxnorm_rmsnorm_rope_interleaved_fwd_dt if interleaved else ltxnorm_rmsnorm_rope_fwd_dt
    fn(out, x, weight, cos_tab, sin_tab, rows, hidden, heads, head_dim, cos_tab.shape[0], eps,
       _dtype_code(x), None)
    return out


def rmsnorm_adaln(x, weight, scale, shift, eps: float = 1e-6, out=None, rows_per_sample=None):
    """RMSNorm then per-sample modulation: norm(x) * weight * (1 + scale) + shift.

    ``x`` bf16 ``[B, S, H]`` (or ``[rows, H]`` with ``rows_per_sample``);
    ``scale`` and ``shift`` bf16 ``[B, H]`` or None (zeros); row r uses
    sample r // S."""
    import torch
    _check_act(x, "x")
    _check_weight(weight, x)
    for t, n in ((scale, "scale"), (shift, "shift")):
        if t is not None:
            _check_act(t, n, x)
    hidden = x.shape[-1]
    rows = x.numel() // hidden if hidden else 0
    if rows_per_sample is None:
        if x.dim() != 3:
            raise ValueError("give rows_per_sample for x that is not [B, S, H]")
        rows_per_sample = x.shape[1]
    rows_per_sample = int(rows_per_sample)
    if out is None:
        out = torch.empty_like(x)
    else:
        _check_act(out, "out", x)
        if out.shape != x.shape:
            raise ValueError("out must have the shape of x")
    if rows_per_sample >= 1:
        samples = -(-rows // rows_per_sample) if rows else 0
        for t, n in ((scale, "scale"), (shift, "shift")):
            if t is not None and t.numel() != samples * hidden:
                raise ValueError(f"{n} must hold [{samples}, {hidden}] values")
    # rows_per_sample < 1 goes to the library unchanged, which refuses it
    # with LTXNORM_ERR_SHAPE before any launch
    ltxnorm_rmsnorm_adaln_fwd_dt(out, x, weight, scale, shift, rows, hidden, rows_per_sample, eps,
                                 _dtype_code(x), None)
    return out
