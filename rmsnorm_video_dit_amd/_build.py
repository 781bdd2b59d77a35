"""Build libltxnorm.so for gfx950 with hipcc (cross-compiles without a GPU)."""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
HEADERS = [os.path.join(ROOT, "include", "ltxnorm.h")] + sorted(glob.glob(os.path.join(CSRC, "*.h")))
LIB = os.path.join(PKG, "libltxnorm.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # only the C ABI (marked LTXNORM_API) is exported
    "-fvisibility=hidden",
    # no packed-fp32 VALU forms in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]
NOISE = "'-packed-fp32-ops' is not a recognized feature for this target"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if NOISE not in ln and ln.strip()]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)


def build(out: str = LIB, verbose: bool = False) -> str:
    """Compile every HIP source (in parallel, one translation unit per I/O
    dtype plus the C-ABI layer) and link one shared library (atomic replace)."""
    tag = "%d" % os.getpid()
    objs = [out + "." + os.path.basename(src) + "." + tag + ".o" for src in SOURCES]
    try:
        with cf.ThreadPoolExecutor(max(1, min(len(SOURCES), os.cpu_count() or 1))) as ex:
            jobs = [ex.submit(_run, [HIPCC, *FLAGS, "-c", src, "-o", obj], verbose)
                    for src, obj in zip(SOURCES, objs)]
            for j in jobs:
                j.result()
        tmp = out + ".tmp" + tag
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
        os.replace(tmp, out)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
