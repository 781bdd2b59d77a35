"""CPU oracle for RMSNorm and fused RMSNorm + rotate-half RoPE (bf16 in, double out).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
and the benchmark's CPU-baseline leg may import this package.  It shares no
code with the HIP library ``rmsnorm_video_dit_amd`` and never imports it.

The arithmetic lives in ``oracle.c`` (plain C, IEEE double, built with gcc);
this module only marshals numpy arrays into it.  The input type follows the
numpy dtype: ``uint16`` arrays are bf16 bit patterns, ``float16`` arrays are
IEEE binary16 and ``float32`` arrays IEEE binary32 (the three precisions of
the skill page's "Supported Data Types").

What is computed, and the reading of the pages behind it, is documented at the
top of ``oracle.c``: RMSNorm per the Hugging Face cuda-kernels skill page
(section "Kernel-Specific Guidelines", RMSNorm: layout [..., hidden], eps
default 1e-6, optional weight), and RMSNorm followed by rotate-half RoPE per
head for the ``rms_norm_rope`` op that the LTX-2 ltx-kernels README lists.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

GCC_CMD = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           _SRC, "-o", _LIB, "-lm"]


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc (no HIP headers, no GPU code).

    ``-ffp-contract=off`` keeps every product and sum a separately rounded
    IEEE double operation, exactly as written in the C source.
    """
    cmd = list(GCC_CMD)
    cmd[cmd.index(_SRC)] = src
    cmd[cmd.index(_LIB)] = out
    tmp = out + ".tmp%d" % os.getpid()
    cmd[cmd.index(out)] = tmp
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


BF16, F16, F32 = 0, 1, 2
_NAMES = {"bf16": BF16, "f16": F16, "f32": F32}


def dtype_of(a: np.ndarray) -> int:
    """Oracle type code of an input array: uint16 = bf16 bit patterns,
    float16 = binary16, float32 = binary32."""
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float16:
        return F16
    if a.dtype == np.float32:
        return F32
    raise TypeError(f"unsupported input dtype {a.dtype}: use uint16 (bf16 bits), float16 or float32")


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    i32 = ctypes.c_int32
    f32 = ctypes.c_float
    c_int = ctypes.c_int
    lib.oracle_rmsnorm.argtypes = [p, p, p, i64, i64, f32]
    lib.oracle_rmsnorm.restype = c_int
    lib.oracle_rmsnorm_dt.argtypes = [p, p, p, i64, i64, f32, c_int]
    lib.oracle_rmsnorm_dt.restype = c_int
    rope = [p, p, p, p, p, p, i64, i64, i32, i32, i64, f32]
    lib.oracle_rmsnorm_rope.argtypes = rope
    lib.oracle_rmsnorm_rope.restype = c_int
    lib.oracle_rmsnorm_rope_dt.argtypes = rope + [c_int]
    lib.oracle_rmsnorm_rope_dt.restype = c_int
    lib.oracle_rmsnorm_rope_interleaved.argtypes = rope
    lib.oracle_rmsnorm_rope_interleaved.restype = c_int
    lib.oracle_rmsnorm_rope_interleaved_dt.argtypes = rope + [c_int]
    lib.oracle_rmsnorm_rope_interleaved_dt.restype = c_int
    lib.oracle_rmsnorm_adaln.argtypes = [p, p, p, p, p, p, i64, i64, i64, f32]
    lib.oracle_rmsnorm_adaln.restype = c_int
    lib.oracle_rmsnorm_adaln_dt.argtypes = [p, p, p, p, p, p, i64, i64, i64, f32, c_int]
    lib.oracle_rmsnorm_adaln_dt.restype = c_int
    lib.oracle_round.argtypes = [p, i64, p, p]
    lib.oracle_round.restype = None
    lib.oracle_round_dt.argtypes = [p, i64, p, p, c_int]
    lib.oracle_round_dt.restype = None
    lib.oracle_f16_from_f32.argtypes = [f32]
    lib.oracle_f16_from_f32.restype = ctypes.c_uint16
    lib.oracle_decode.argtypes = [p, i64, c_int, p]
    lib.oracle_decode.restype = None
    lib.oracle_f16_array.argtypes = [p, i64, p]
    lib.oracle_f16_array.restype = None
    lib.oracle_bf16_from_f32.argtypes = [ctypes.c_float]
    lib.oracle_bf16_from_f32.restype = ctypes.c_uint16
    lib.oracle_bf16_array.argtypes = [p, i64, p]
    lib.oracle_bf16_array.restype = None
    return lib


def load(path: str | None = None) -> ctypes.CDLL:
    """Load the built oracle, compiling it first only if nothing is built."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build()
            _lib = _bind(ctypes.CDLL(_LIB))
        return _lib


def _ptr(a: np.ndarray | None):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _same(a, dt, name):
    """Contiguous array of the input type `dt` (None passes through)."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if dtype_of(a) != dt:
        raise TypeError(f"{name} must have the dtype of x, got {a.dtype}")
    return a


class Oracle:
    """numpy front end over one loaded oracle library (the real one, or a
    deliberately broken copy built by the mutation tests)."""

    def __init__(self, lib: ctypes.CDLL | None = None):
        self.lib = lib if lib is not None else load()

    def rmsnorm(self, x, w, eps: float = 1e-6) -> np.ndarray:
        """RMSNorm of ``x[..., H]`` with weight ``w[H]`` of the same type (or
        None); returns the double result with the shape of ``x``."""
        x = np.ascontiguousarray(x)
        dt = dtype_of(x)
        hidden = x.shape[-1]
        rows = x.size // hidden if hidden else 0
        w = _same(w, dt, "w")
        if w is not None:
            assert w.shape == (hidden,)
        y = np.empty(x.shape, dtype=np.float64)
        rc = self.lib.oracle_rmsnorm_dt(_ptr(y), _ptr(x), _ptr(w), rows, hidden,
                                        ctypes.c_float(eps), dt)
        if rc != 0:
            raise ValueError("oracle_rmsnorm rejected its arguments")
        return y

    def rmsnorm_rope(self, x, w, cos_tab, sin_tab, heads: int, head_dim: int,
                     eps: float = 1e-6, with_mag: bool = False, interleaved: bool = False):
        """RMSNorm over the whole row then RoPE per head: rotate-half pairs
        (i, i + d/2), or with ``interleaved`` adjacent pairs (2i, 2i + 1).

        ``x`` bf16 ``[rows, heads*head_dim]`` (any leading shape); tables
        binary32 ``[seq_len, head_dim/2]``; row r uses table row r mod seq_len.
        Returns the double result, and with ``with_mag`` also the per-output
        magnitude sum |a*c| + |b*s| that bounds its cancellation.
        """
        x = np.ascontiguousarray(x)
        dt = dtype_of(x)
        hidden = x.shape[-1]
        rows = x.size // hidden if hidden else 0
        w = _same(w, dt, "w")
        cos_tab = np.ascontiguousarray(cos_tab, dtype=np.float32)
        sin_tab = np.ascontiguousarray(sin_tab, dtype=np.float32)
        if cos_tab.ndim != 2 or cos_tab.shape != sin_tab.shape or cos_tab.shape[1] != head_dim // 2:
            raise ValueError("cos/sin tables must both be [seq_len, head_dim/2]")
        seq_len = cos_tab.shape[0]
        y = np.empty(x.shape, dtype=np.float64)
        mag = np.empty(x.shape, dtype=np.float64) if with_mag else None
        fn = (self.lib.oracle_rmsnorm_rope_interleaved_dt if interleaved
              else self.lib.oracle_rmsnorm_rope_dt)
        rc = fn(_ptr(y), _ptr(mag), _ptr(x), _ptr(w), _ptr(cos_tab), _ptr(sin_tab),
                rows, hidden, heads, head_dim, seq_len, ctypes.c_float(eps), dt)
        if rc != 0:
            raise ValueError("oracle_rmsnorm_rope rejected its arguments")
        return (y, mag) if with_mag else y

    def rmsnorm_adaln(self, x, w, scale, shift, rows_per_sample: int, eps: float = 1e-6,
                      with_mag: bool = False):
        """RMSNorm then per-sample modulation y * (1 + scale[b]) + shift[b],
        b = row // rows_per_sample; scale/shift bf16 [samples, H] or None.
        With ``with_mag`` also returns |y * (1 + scale)| + |shift| per output,
        which bounds the cancellation of the final sum."""
        x = np.ascontiguousarray(x)
        dt = dtype_of(x)
        hidden = x.shape[-1]
        rows = x.size // hidden if hidden else 0
        w = _same(w, dt, "w")
        samples = -(-rows // rows_per_sample) if rows else 0
        for t, n in ((scale, "scale"), (shift, "shift")):
            if t is not None and np.asarray(t).size != samples * hidden:
                raise ValueError(f"{n} must hold [{samples}, {hidden}] values")
        scale = _same(scale, dt, "scale")
        shift = _same(shift, dt, "shift")
        y = np.empty(x.shape, dtype=np.float64)
        mag = np.empty(x.shape, dtype=np.float64) if with_mag else None
        rc = self.lib.oracle_rmsnorm_adaln_dt(_ptr(y), _ptr(mag), _ptr(x), _ptr(w), _ptr(scale),
                                              _ptr(shift), rows, hidden, rows_per_sample,
                                              ctypes.c_float(eps), dt)
        if rc != 0:
            raise ValueError("oracle_rmsnorm_adaln rejected its arguments")
        return (y, mag) if with_mag else y

    def round(self, y: np.ndarray, out_dtype: str = "bf16"):
        """Round double results once to binary32 (ref32) and that to the
        output type, both round-to-nearest-even: bf16 bit patterns (uint16),
        binary16 (float16 array) or binary32 (float32, equal to ref32)."""
        y = np.ascontiguousarray(y, dtype=np.float64)
        dt = _NAMES[out_dtype]
        ref32 = np.empty(y.shape, dtype=np.float32)
        ref = np.empty(y.shape, dtype={BF16: np.uint16, F16: np.uint16, F32: np.float32}[dt])
        self.lib.oracle_round_dt(_ptr(y), y.size, _ptr(ref32), _ptr(ref), dt)
        if dt == F16:
            ref = ref.view(np.float16)
        return ref32, ref

    def decode(self, x: np.ndarray) -> np.ndarray:
        """Values of an input array (bf16 bits, float16 or float32) as doubles."""
        x = np.ascontiguousarray(x)
        out = np.empty(x.shape, dtype=np.float64)
        self.lib.oracle_decode(_ptr(x), x.size, dtype_of(x), _ptr(out))
        return out

    def f16_from_f32(self, f: np.ndarray) -> np.ndarray:
        """Round binary32 values (any bit pattern) to binary16 bit patterns
        (uint16) with the oracle's round-to-nearest-even."""
        f = np.ascontiguousarray(f, dtype=np.float32)
        out = np.empty(f.shape, dtype=np.uint16)
        self.lib.oracle_f16_array(_ptr(f), f.size, _ptr(out))
        return out

    def bf16_from_f32(self, f: np.ndarray) -> np.ndarray:
        """Round binary32 values (any bit pattern, NaNs included) to bf16 bit
        patterns with the oracle's round-to-nearest-even."""
        f = np.ascontiguousarray(f, dtype=np.float32)
        out = np.empty(f.shape, dtype=np.uint16)
        self.lib.oracle_bf16_array(_ptr(f), f.size, _ptr(out))
        return out
