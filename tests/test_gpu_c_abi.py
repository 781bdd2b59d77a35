"""The library through its C ABI alone: tests/c_abi/ltxnorm_c_check.cpp
allocates with hipMalloc, launches on a stream of its own and compares every
output element with the oracle, with no Python or PyTorch in the calling
program (RMSNorm on the vector, general and short-row kernels, both RoPE
pairings, AdaLN, fp32 I/O, in place, and the status of rejected calls)."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "ltxnorm_c_check")


def test_c_abi_program():
    assert os.path.exists(BIN), f"{BIN} is missing: run __graft_entry__.build() first"
    print("c-abi program", flush=True)
    res = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(res.stdout, res.stderr, flush=True)
    assert res.returncode == 0 and res.stdout.strip().endswith("ok"), res.stdout + res.stderr
