"""The C ABI's host layer under AddressSanitizer, on the CPU: validation,
ltxnorm_describe_launch over 200,000 random shapes and output-buffer
lengths, and status strings (tests/c_abi/host_asan_check.cpp).  Only the
host pass is instrumented; nothing is launched."""
import os
import subprocess

import pytest

from rmsnorm_video_dit_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CHECK = os.path.join(ROOT, "tests", "c_abi", "host_asan_check.cpp")
ABI = os.path.join(ROOT, "rmsnorm_video_dit_amd", "csrc", "ltxnorm.hip")
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(not os.path.exists(_build.HIPCC), reason="hipcc not installed")
def test_host_layer_under_address_sanitizer(tmp_path):
    obj = str(tmp_path / "abi.o")
    chk = str(tmp_path / "check.o")
    exe = str(tmp_path / "host_asan_check")
    for src, out in ((ABI, obj), (CHECK, chk)):
        r = subprocess.run([_build.HIPCC, *_build.FLAGS, *HOST_ASAN, "-x", "hip", "-c", src, "-o", out],
                           capture_output=True, text=True, timeout=600)
        assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([_build.HIPCC, "--offload-arch=gfx950", *HOST_ASAN, obj, chk, "-o", exe],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "statuses 1 3 5 6 1 2 4 0" in r.stdout, r.stdout
    described = int(r.stdout.split("described ")[1].split()[0])
    assert described > 10000, r.stdout
