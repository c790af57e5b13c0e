"""Build libpaged_attn_e4m3.so (HIP, gfx950) in-tree with hipcc.

All HIP code is compiled with packed-FP32 instruction generation disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``).
"""

from __future__ import annotations

import glob
import hashlib
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpaged_attn_e4m3.so")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


CODEGEN_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]

# sources whose kernels issue direct-to-LDS loads as inline asm
ASM_DMA_SOURCES = ["verify_mfma.hip"]
# sources whose kernels issue wide (more than 8-byte) stores as inline asm
ASM_STORE_SOURCES = ["cache_write.hip"]


def source_files():
    """Every file the library is compiled from, in a fixed order."""
    return (sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.h")))
            + [os.path.join(ROOT, "include", "paged_attn_e4m3.h")])


def source_hash() -> str:
    """First 16 hex digits of a SHA-256 over the library's sources and its
    code-generation flags; compiled into the library as its build id."""
    h = hashlib.sha256()
    for path in source_files():
        with open(path, "rb") as f:
            h.update(os.path.relpath(path, ROOT).encode() + b"\0" + f.read() + b"\0")
    h.update(" ".join(CODEGEN_FLAGS).encode())
    return h.hexdigest()[:16]


def check_hazards(extra_flags=()) -> None:
    """Compile the inline-asm sources to gfx950 assembly and reject the build
    if a direct-to-LDS load lacks the wait states gfx9 requires before it, or
    a wide asm store the wait states a VALU write of its data needs after it."""
    try:
        from . import asm_hazards
    except ImportError:          # run as a script
        import asm_hazards

    def assembly(name):
        src = os.path.join(CSRC, name)
        asm = os.path.join(HERE, name + ".s.tmp")
        cmd = [hipcc(), *CODEGEN_FLAGS, "--cuda-device-only", "-S",
               "-I", os.path.join(ROOT, "include"), "-I", CSRC, *extra_flags, src, "-o", asm]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc -S failed:\n" + r.stdout + r.stderr)
        with open(asm) as f:
            text = f.read()
        os.remove(asm)
        return text

    for name in ASM_DMA_SOURCES:
        found = asm_hazards.check(assembly(name))
        if found:
            lines = "\n".join(f"  {k}: {p}  ->  {t}" for k, p, t in found[:10])
            raise RuntimeError(f"{name}: {len(found)} unprotected hazards before "
                               f"direct-to-LDS loads:\n{lines}")
    for name in ASM_STORE_SOURCES:
        found = asm_hazards.check_stores(assembly(name))
        if found:
            lines = "\n".join(f"  {t}" for t in found[:10])
            raise RuntimeError(f"{name}: {len(found)} asm stores without the wait states "
                               f"after them:\n{lines}")


def build(out: str = LIB, extra_flags=(), verbose: bool = False) -> str:
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    tmp = out + ".tmp"
    cmd = [hipcc(), *CODEGEN_FLAGS, "-fPIC", "-shared",
           "-Wall", "-Werror", "-Wno-unused-function", f'-DPA_BUILD_ID="{source_hash()}"',
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, *extra_flags, *srcs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stdout + r.stderr)
    if verbose:
        print(r.stderr)
    check_hazards(extra_flags)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
