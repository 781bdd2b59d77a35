"""Bandwidth ceiling kernels for the benchmark (``copy.hip``), built into
``libceiling.so`` next to this file.

Not part of the library: these kernels only move bytes (plain and
non-temporal 16-byte copies, non-temporal read-only and write-only streams),
so that the benchmark can report a normalisation kernel's rate as a fraction
of what the same part's HBM gives plain loads and stores of the same bytes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "copy.hip")
LIB = os.path.join(HERE, "libceiling.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-fvisibility=hidden", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

PLAIN, NT_COPY, NT_READ, NT_WRITE = 0, 1, 2, 3
MODES = {"plain_copy": PLAIN, "nt_copy": NT_COPY, "nt_read": NT_READ, "nt_write": NT_WRITE}

_lib = None


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB)
        L.ceiling_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        L.ceiling_copy.restype = ctypes.c_int
        _lib = L
    return _lib


def copy(dst_ptr: int, src_ptr: int, nvec: int, mode: int, per: int, sink_ptr, stream: int) -> None:
    """One pass over ``nvec`` 16-byte vectors (device pointers, a raw
    hipStream_t handle); raises on a launch error."""
    st = lib().ceiling_copy(dst_ptr, src_ptr, int(nvec), int(mode), int(per), sink_ptr, stream)
    if st != 0:
        raise RuntimeError(f"ceiling_copy(mode={mode}, per={per}) failed with status {st}")
