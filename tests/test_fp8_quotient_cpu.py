"""Host check of the quotient route of the in-wave FP8 row encode (one rounded
reciprocal per row, one remainder correction per element) against correctly
rounded fp32 division, through tests/c/fp8_quotient_check.c: every x in the
binades where the E4M3 byte depends on the last bits, signed zeros and subnormals,
for scales at and above the route's 2^-64 threshold, and 20 million random
(scale, element) pairs.  The same program with the argument "full" checks every
x of each scale (8.8e9 cases; minutes)."""

import os
import shutil
import subprocess

import pytest


def test_fp8_quotient_route_equals_division(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc is not available")
    src = os.path.join(os.path.dirname(__file__), "c", "fp8_quotient_check.c")
    exe = str(tmp_path / "fp8_quotient_check")
    subprocess.run([gcc, "-O2", "-ffp-contract=off", src, "-o", exe, "-lm"], check=True)
    out = subprocess.run([exe, "20000000"], capture_output=True, text=True, timeout=600)
    assert out.returncode == 0 and out.stdout.startswith("ok"), out.stdout
