"""CPU check of the identity the E4M3 cache writer's division relies on.

For FP16 x and a scale b in [2^-110, 2^126] the writer forms the FP32 quotient
from y = RN(1/b) with one FMA correction (Markstein):
    q = RN(x y),  r = fma(-q, b, x),  RN(q + r y) = RN(x / b),
with x's sign copied onto the result.  The C program in tests/division tries
every finite FP16 x against special mantissas at every exponent of the range
and seeded random scales, against IEEE single division, bit for bit."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "division", "reciprocal_division_check.c")


def test_reciprocal_division_matches_ieee(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "reciprocal_division_check")
    # -mfma: fmaf is the fused operation; no contraction anywhere else
    r = subprocess.run([gcc, "-O2", "-mfma", "-ffp-contract=off", SRC, "-o", exe, "-lm",
                        "-lpthread"], capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("cannot build with -mfma here: " + r.stderr[-300:])
    r = subprocess.run([exe, "3000", "4"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "mismatches 0" in r.stdout
