"""Build libltxnorm.so for gfx950 with hipcc (cross-compiles without a GPU)."""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import re
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
# the compiler's per-kernel resource report (registers, occupancy, scratch)
RESOURCE_REMARKS = "-Rpass-analysis=kernel-resource-usage"
RESOURCES = os.path.join(PKG, "kernel_resources.txt")
_REMARK = re.compile(r"remark:\s+(Function Name|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|"
                     r"Occupancy \[waves/SIMD\]|LDS Size \[bytes/block\]):\s+(\S+)")


def _resources(text: str) -> list:
    """(kernel, {field: value}) from the compiler's resource remarks."""
    out = []
    for m in _REMARK.finditer(text):
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            out.append((val, {}))
        elif out:
            out[-1][1][key.split(" [")[0]] = val
    return out


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    text = res.stdout + res.stderr
    # compiler output other than the feature notice and the resource remarks
    # (each remark comes with its include chain and a source excerpt)
    msgs = [ln for ln in text.splitlines()
            if ln.strip() and NOISE not in ln and "kernel-resource-usage" not in ln
            and not ln.startswith("In file included from") and not ln.lstrip()[:1].isdigit()
            and not ln.lstrip().startswith("|")]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    return _resources(text)


def build(out: str = LIB, verbose: bool = False) -> str:
    """Compile every HIP source (in parallel, one translation unit per I/O
    dtype plus the C-ABI layer) and link one shared library (atomic replace).
    The compiler's per-kernel resource report goes to kernel_resources.txt;
    a kernel that uses scratch memory fails the build."""
    tag = "%d" % os.getpid()
    objs = [out + "." + os.path.basename(src) + "." + tag + ".o" for src in SOURCES]
    try:
        with cf.ThreadPoolExecutor(max(1, min(len(SOURCES), os.cpu_count() or 1))) as ex:
            jobs = [ex.submit(_run, [HIPCC, *FLAGS, RESOURCE_REMARKS, "-c", src, "-o", obj], verbose)
                    for src, obj in zip(SOURCES, objs)]
            kernels = [k for j in jobs for k in j.result()]
        # No kernel may use private (scratch) memory: a spill or a
        # runtime-indexed array there costs every lane a memory round trip.
        spilled = [name for name, f in kernels if f.get("ScratchSize", "0") != "0"]
        if spilled:
            raise RuntimeError(f"{len(spilled)} kernels use scratch memory, e.g. " + ", ".join(spilled[:5]))
        with open(RESOURCES + ".tmp" + tag, "w") as fh:
            fh.write("# kernel VGPRs AGPRs scratch_bytes_per_lane occupancy_waves_per_simd lds_bytes\n")
            for name, f in sorted(kernels):
                fh.write(f"{name} {f.get('VGPRs')} {f.get('AGPRs')} {f.get('ScratchSize')} "
                         f"{f.get('Occupancy')} {f.get('LDS Size')}\n")
        os.replace(RESOURCES + ".tmp" + tag, RESOURCES)
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
