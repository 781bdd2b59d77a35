"""CPU oracle for RMSNorm and fused RMSNorm + rotate-half RoPE (bf16 in, double out).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
and the benchmark's CPU-baseline leg may import this package.  It shares no
code with the HIP library ``rmsnorm_video_dit_amd`` and never imports it.

The arithmetic lives in ``oracle.c`` (plain C, IEEE double, built with gcc);
this module only marshals numpy arrays into it.  bf16 tensors travel as
``numpy.uint16`` bit patterns.

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


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    i32 = ctypes.c_int32
    lib.oracle_rmsnorm.argtypes = [p, p, p, i64, i64, ctypes.c_float]
    lib.oracle_rmsnorm.restype = ctypes.c_int
    lib.oracle_rmsnorm_rope.argtypes = [p, p, p, p, p, p, i64, i64, i32, i32,
                                        i64, ctypes.c_float]
    lib.oracle_rmsnorm_rope.restype = ctypes.c_int
    lib.oracle_rmsnorm_rope_interleaved.argtypes = list(lib.oracle_rmsnorm_rope.argtypes)
    lib.oracle_rmsnorm_rope_interleaved.restype = ctypes.c_int
    lib.oracle_rmsnorm_adaln.argtypes = [p, p, p, p, p, p, i64, i64, i64, ctypes.c_float]
    lib.oracle_rmsnorm_adaln.restype = ctypes.c_int
    lib.oracle_round.argtypes = [p, i64, p, p]
    lib.oracle_round.restype = None
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


def _u16(a, name):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"{name} must hold bf16 bit patterns as uint16, got {a.dtype}")
    return a


class Oracle:
    """numpy front end over one loaded oracle library (the real one, or a
    deliberately broken copy built by the mutation tests)."""

    def __init__(self, lib: ctypes.CDLL | None = None):
        self.lib = lib if lib is not None else load()

    def rmsnorm(self, x, w, eps: float = 1e-6) -> np.ndarray:
        """RMSNorm of bf16 ``x[..., H]`` with bf16 weight ``w[H]`` (or None);
        returns the double result with the shape of ``x``."""
        x = _u16(x, "x")
        hidden = x.shape[-1]
        rows = x.size // hidden if hidden else 0
        if w is not None:
            w = _u16(w, "w")
            assert w.shape == (hidden,)
        y = np.empty(x.shape, dtype=np.float64)
        rc = self.lib.oracle_rmsnorm(_ptr(y), _ptr(x), _ptr(w), rows, hidden,
                                     ctypes.c_float(eps))
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
        x = _u16(x, "x")
        hidden = x.shape[-1]
        rows = x.size // hidden if hidden else 0
        if w is not None:
            w = _u16(w, "w")
        cos_tab = np.ascontiguousarray(cos_tab, dtype=np.float32)
        sin_tab = np.ascontiguousarray(sin_tab, dtype=np.float32)
        if cos_tab.ndim != 2 or cos_tab.shape != sin_tab.shape or cos_tab.shape[1] != head_dim // 2:
            raise ValueError("cos/sin tables must both be [seq_len, head_dim/2]")
        seq_len = cos_tab.shape[0]
        y = np.empty(x.shape, dtype=np.float64)
        mag = np.empty(x.shape, dtype=np.float64) if with_mag else None
        fn = self.lib.oracle_rmsnorm_rope_interleaved if interleaved else self.lib.oracle_rmsnorm_rope
        rc = fn(_ptr(y), _ptr(mag), _ptr(x), _ptr(w), _ptr(cos_tab), _ptr(sin_tab),
                rows, hidden, heads, head_dim, seq_len, ctypes.c_float(eps))
        if rc != 0:
            raise ValueError("oracle_rmsnorm_rope rejected its arguments")
        return (y, mag) if with_mag else y

    def rmsnorm_adaln(self, x, w, scale, shift, rows_per_sample: int, eps: float = 1e-6,
                      with_mag: bool = False):
        """RMSNorm then per-sample modulation y * (1 + scale[b]) + shift[b],
        b = row // rows_per_sample; scale/shift bf16 [samples, H] or None.
        With ``with_mag`` also returns |y * (1 + scale)| + |shift| per output,
        which bounds the cancellation of the final sum."""
        x = _u16(x, "x")
        hidden = x.shape[-1]
        rows = x.size // hidden if hidden else 0
        w = None if w is None else _u16(w, "w")
        samples = -(-rows // rows_per_sample) if rows else 0
        for t, n in ((scale, "scale"), (shift, "shift")):
            if t is not None and np.asarray(t).size != samples * hidden:
                raise ValueError(f"{n} must hold [{samples}, {hidden}] values")
        scale = None if scale is None else _u16(scale, "scale")
        shift = None if shift is None else _u16(shift, "shift")
        y = np.empty(x.shape, dtype=np.float64)
        mag = np.empty(x.shape, dtype=np.float64) if with_mag else None
        rc = self.lib.oracle_rmsnorm_adaln(_ptr(y), _ptr(mag), _ptr(x), _ptr(w), _ptr(scale),
                                           _ptr(shift), rows, hidden, rows_per_sample,
                                           ctypes.c_float(eps))
        if rc != 0:
            raise ValueError("oracle_rmsnorm_adaln rejected its arguments")
        return (y, mag) if with_mag else y

    def round(self, y: np.ndarray):
        """Round double results once to binary32 (ref32) and that to bf16
        (ref16, uint16 bit patterns), both round-to-nearest-even."""
        y = np.ascontiguousarray(y, dtype=np.float64)
        ref32 = np.empty(y.shape, dtype=np.float32)
        ref16 = np.empty(y.shape, dtype=np.uint16)
        self.lib.oracle_round(_ptr(y), y.size, _ptr(ref32), _ptr(ref16))
        return ref32, ref16

    def bf16_from_f32(self, f: np.ndarray) -> np.ndarray:
        """Round binary32 values (any bit pattern, NaNs included) to bf16 bit
        patterns with the oracle's round-to-nearest-even."""
        f = np.ascontiguousarray(f, dtype=np.float32)
        out = np.empty(f.shape, dtype=np.uint16)
        self.lib.oracle_bf16_array(_ptr(f), f.size, _ptr(out))
        return out
