"""Build the C-ABI check program tests/c_abi/ltxnorm_c_check: the oracle
(oracle/oracle.c, gcc with the oracle's own flags) linked with a C++ driver
that calls libltxnorm.so through include/ltxnorm.h only.  Test
infrastructure: run by the GPU test tests/test_gpu_c_abi.py."""
from __future__ import annotations

import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "ltxnorm_c_check.cpp")
BIN = os.path.join(HERE, "ltxnorm_c_check")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(out: str = BIN) -> str:
    with tempfile.TemporaryDirectory() as tmp:
        obj = os.path.join(tmp, "oracle.o")
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-ffp-contract=off", "-c",
                        os.path.join(ROOT, "oracle", "oracle.c"), "-o", obj], check=True)
        cobj = os.path.join(tmp, "ltxnorm_c_check.o")
        subprocess.run([HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                        "-I", os.path.join(ROOT, "include"), "-c", SRC, "-o", cobj],
                       check=True, capture_output=True, text=True)
        exe = os.path.join(tmp, "ltxnorm_c_check")
        subprocess.run([HIPCC, "--offload-arch=gfx950", cobj, obj,
                        "-L", os.path.join(ROOT, "rmsnorm_video_dit_amd"), "-lltxnorm",
                        "-Wl,-rpath,$ORIGIN/../../rmsnorm_video_dit_amd", "-lm", "-o", exe],
                       check=True, capture_output=True, text=True)
        os.replace(exe, out)
    return out


if __name__ == "__main__":
    print(build())
