"""Build liboracle.so from oracle.c with gcc (test infrastructure only).

``build()`` makes the normal oracle.  ``build(mutant=n, out=path)`` makes a
copy with planted mistake n (see the ORC_MUTANT switch in oracle.c), used only
by the test that shows the pins catch each planted mistake.
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-D_GNU_SOURCE", "-fPIC", "-shared", "-pthread",
          "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra", "-Werror"]


def build(mutant: int = 0, out: str = LIB, extra_flags=()) -> str:
    cmd = ["gcc", *CFLAGS, *extra_flags, f"-DORC_MUTANT={int(mutant)}", SRC, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build(*(int(a) for a in sys.argv[1:2])))
