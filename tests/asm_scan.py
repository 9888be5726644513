"""Scanner for one hazard of gfx950 device assembly that the compiler does not
guard inside inline asm: a VALU instruction that writes an SGPR (or M0) read
by a following vector-memory instruction needs five wait states between
them, and M0 written for an LDS-DMA load needs one (the gfx9-family
manually-inserted wait-state rules).  Test infrastructure: it reads the
``.s`` text hipcc writes with ``--cuda-device-only -S``."""
from __future__ import annotations

import re

_SREG = re.compile(r"^s\[(\d+):(\d+)\]$|^s(\d+)$")
_LABEL = re.compile(r"^(\.?[A-Za-z_$][\w.$]*):")
_BRANCH = re.compile(r"^s_(?:c)?branch\w*\s+(\S+)")
_DMA = re.compile(r"^global_load_lds_dwordx4\s+v\d+,\s*(s\[\d+:\d+\])")


def sregs(op: str) -> set:
    """Scalar register numbers named by one operand ('m0' -> {'m0'})."""
    op = op.strip()
    if op == "m0":
        return {"m0"}
    if op == "vcc":
        return {"vcc"}
    m = _SREG.match(op)
    if not m:
        return set()
    if m.group(3) is not None:
        return {int(m.group(3))}
    return set(range(int(m.group(1)), int(m.group(2)) + 1))


def valu_sgpr_writes(text: str) -> set:
    """Scalar registers a VALU instruction writes (its SGPR destination, or
    the carry / scale SGPR output of the _co, addc, subb and div_scale
    forms); empty for anything else."""
    if not text.startswith("v_"):
        return set()
    mnem, _, rest = text.partition(" ")
    ops = [o.strip() for o in rest.split(",")] if rest else []
    out = set()
    if ops:
        out |= sregs(ops[0])
    if len(ops) > 1 and re.search(r"_co_|_co$|addc|subb|div_scale|mad_u64|mad_i64", mnem):
        out |= sregs(ops[1])
    if mnem.startswith("v_cmp") and mnem.endswith("_e32"):
        out.add("vcc")
    return out


def wait_states(text: str) -> int:
    m = re.match(r"^s_nop\s+(\d+)", text)
    return int(m.group(1)) + 1 if m else 1


def parse(asm: str):
    """(kind, text) items of the device assembly: 'label', 'insn' or 'func'
    (a function boundary)."""
    items = []
    for raw in asm.splitlines():
        line = raw.split(";", 1)[0].strip()
        if not line:
            continue
        if line.startswith(".") and not _LABEL.match(line):
            if line.startswith((".amdhsa_kernel", ".end_amdhsa_kernel", ".size", ".Lfunc_end")):
                items.append(("func", line))
            continue
        m = _LABEL.match(line)
        if m:
            if not m.group(1).startswith(".L"):
                items.append(("func", line))
            items.append(("label", m.group(1)))
            continue
        items.append(("insn", line))
    return items


def scan(asm: str, need: int = 5):
    """Every SGPR-base global_load_lds_dwordx4 and, for each, the VALU
    writes of its base SGPRs or M0 found less than `need` wait states
    before it along any path.  Returns (count, violations)."""
    items = parse(asm)
    sources = {}
    for i, (k, t) in enumerate(items):
        if k == "insn":
            m = _BRANCH.match(t)
            if m:
                sources.setdefault(m.group(1), []).append(i)
    violations = []
    count = 0
    for i, (k, t) in enumerate(items):
        if k != "insn":
            continue
        m = _DMA.match(t)
        if not m:
            continue
        count += 1
        regs = sregs(m.group(1)) | {"m0"}
        seen = set()
        stack = [(i - 1, need)]
        while stack:
            j, left = stack.pop()
            if (j, left) in seen:
                continue
            seen.add((j, left))
            while j >= 0 and left > 0:
                kind, text = items[j]
                if kind == "func":
                    break
                if kind == "label":
                    for b in sources.get(text, []):
                        stack.append((b, left))
                    prev = j - 1
                    if prev >= 0 and items[prev][0] == "insn" and re.match(r"^s_(branch|endpgm|setpc)", items[prev][1]):
                        break
                    j = prev
                    continue
                w = valu_sgpr_writes(text)
                if w & regs:
                    violations.append((t, text, need - left))
                left -= wait_states(text)
                j -= 1
    return count, violations


def sgpr_spills(asm: str) -> dict:
    """Kernel symbol -> .sgpr_spill_count from the code-object metadata."""
    out = {}
    for m in re.finditer(r"\.name:\s+(\S+)\s*\n(?:.*\n)*?\s+\.sgpr_spill_count:\s+(\d+)", asm):
        out[m.group(1)] = int(m.group(2))
    return out
