"""Each planted mistake in the oracle (ORC_MUTANT=n in oracle.c) must fail at
least one pin.  The mistakes are the plausible ones: wrong GQA head map, a
dropped k_scale or v_scale, an off-by-one visibility bound, a sign error in
the softmax exponent, a transposed query index, the block table ignored, a
shifted split boundary, a missing combine weight, wrong subnormal or exponent
bias in the E4M3 decode, ties rounded to odd, the selection ignored, and the
sparse visibility bound taken on list positions instead of tokens, and in
the combine of FP32 partials the max read as the sum or the split index
dropped from the numerator.  Each
build runs in its own process, so a crash also counts as caught."""

import os
import subprocess
import sys

import pytest

from oracle import build as obuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MUTANTS = list(range(1, 19))

_RUNNER = r"""
import sys, traceback
sys.path.insert(0, {root!r})
import oracle
from tests import oracle_pins
o = oracle.Oracle({lib!r})
for pin in oracle_pins.ALL_PINS:
    try:
        pin(o)
    except Exception as e:
        print("CAUGHT", pin.__name__, type(e).__name__, str(e)[:120])
        sys.exit(0)
print("NOT CAUGHT")
sys.exit(3)
"""


@pytest.mark.parametrize("mutant", MUTANTS)
def test_planted_mistake_is_caught(mutant, tmp_path):
    lib = str(tmp_path / f"liboracle_m{mutant}.so")
    obuild.build(mutant=mutant, out=lib)
    env = dict(os.environ, ORC_PIN_QUICK="1")
    r = subprocess.run([sys.executable, "-c", _RUNNER.format(root=ROOT, lib=lib)],
                       capture_output=True, text=True, env=env, timeout=300)
    assert "NOT CAUGHT" not in r.stdout, f"mutant {mutant} passed every pin"
    assert r.returncode != 3, r.stdout + r.stderr
