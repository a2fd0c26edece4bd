"""The kernels divide by launch constants with a multiply-high and shift
(make_fastdiv / fdiv in csrc/ctconv_internal.h).  This builds a host program
from that header with hipcc and checks it against integer division: every
numerator below 8192 and random ones for every divisor up to 2048, random
divisors and powers of two, and the largest numerators below 2^31."""

import os
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_fastdiv_matches_integer_division():
    src = os.path.join(ROOT, "tests", "native", "fastdiv_check.hip")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "fastdiv_check")
        cmd = [HIPCC, "-O2", "-std=c++17", "--offload-arch=gfx950", "-I",
               os.path.join(ROOT, "include"), "-I",
               os.path.join(ROOT, "vision_upsampler_decoders_amd", "csrc"), src, "-o", exe]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        # the host program makes no GPU call
        r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, r.stdout + r.stderr
        assert r.stdout.strip().startswith("0 of ")
