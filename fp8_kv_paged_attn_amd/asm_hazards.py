"""Check gfx950 assembly for hazards around inline-asm memory instructions.

The verify kernel issues its global->LDS loads as inline asm, and LLVM's hazard
recognizer does not look inside inline asm.  gfx9 requires, before such a load:
  * one wait state after an instruction that writes M0 (the LDS destination);
  * five wait states after a VALU instruction (v_readfirstlane, v_readlane,
    v_cmp) that writes an SGPR the load reads as its address base.
Missing the second one lets the load read the SGPR's previous contents as an
address.  ``check(asm_text)`` returns the offending instruction pairs (empty
when clean).

The cache writer's device-scope stores are inline asm too.  After a vector
memory store of more than 8 bytes, a VALU instruction that overwrites the
store's data VGPRs needs two wait states (gfx940 and later), which the
compiler cannot insert after an asm store: the asm carries them.
``check_stores(asm_text)`` returns every such store inside an asm block that is
not followed, in the same block, by an ``s_nop`` of at least two wait states.
``build.py`` runs both checks on every build.
"""

from __future__ import annotations

import re
from typing import List, Set, Tuple


def _sgprs(tok: str) -> Set[int]:
    m = re.match(r"s\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"s(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _instructions(asm: str) -> List[str]:
    out = []
    for line in asm.split("\n"):
        t = line.split(";")[0].strip()
        if not t or t.startswith(".") or t.endswith(":"):
            continue
        out.append(t)
    return out


def check(asm: str) -> List[Tuple[str, str, str]]:
    """(kind, producer, load) for every hazard found in straight-line code
    before each global_load_lds instruction."""
    ins = _instructions(asm)
    found = []
    for i, t in enumerate(ins):
        if not t.startswith("global_load_lds"):
            continue
        ops = [o.strip() for o in t.split(None, 1)[1].split(",")]
        used: Set[int] = set()
        for o in ops[1:]:
            used |= _sgprs(o.split()[0])
        ws = 0
        j = i - 1
        while j >= 0 and ws < 5:
            p = ins[j]
            parts = p.split(None, 1)
            mnem = parts[0]
            dst = parts[1].split(",")[0].strip() if len(parts) > 1 else ""
            if mnem == "s_nop":
                ws += int(parts[1]) + 1
                j -= 1
                continue
            if mnem.startswith("s_branch") or mnem.startswith("s_cbranch") or mnem == "s_endpgm":
                break
            if dst == "m0" and ws < 1:
                found.append(("m0", p, t))
            if mnem.startswith("v_") and (_sgprs(dst) & used):
                found.append(("valu-sgpr", p, t))
            ws += 1
            j -= 1
    return found


_WIDE_STORE = re.compile(r"^(global|buffer|flat)_store_dword(x3|x4)\b")


def check_stores(asm: str) -> List[str]:
    """Inline-asm stores of more than 8 bytes without two wait states after
    them inside their asm block."""
    found = []
    in_asm = False
    pending = None          # a wide asm store still waiting for its s_nop
    for line in asm.split("\n"):
        raw = line.strip()
        if raw.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if raw.startswith(";;#ASMEND"):
            if pending is not None:
                found.append(pending)
                pending = None
            in_asm = False
            continue
        t = raw.split(";")[0].strip()
        if not t or t.startswith(".") or t.endswith(":") or not in_asm:
            continue
        if pending is not None:
            parts = t.split()
            if not (parts[0] == "s_nop" and len(parts) > 1 and int(parts[1], 0) >= 1):
                found.append(pending)
            pending = None
        if _WIDE_STORE.match(t):
            pending = t
    return found
