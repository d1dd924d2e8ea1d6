"""Check of compiled gfx950 assembly: no instruction may touch a register
that an LDS read is still filling.

The kernels issue some LDS reads through inline asm (so that the compiler
does not make them wait for in-flight LDS DMA) and wait for them with
explicit `s_waitcnt lgkmcnt(N)`.  The compiler cannot see that such a read
fills its output register asynchronously: if register pressure makes it copy
that register before the wait, the copy holds stale data.  This walks each
kernel's instructions in layout order, keeps the queue of outstanding LDS
operations (they complete in order, so lgkmcnt(N) retires all but the
newest N), and reports every instruction that reads or writes a register of
an outstanding LDS read.  Branches are followed in layout order only (the
queue carries across labels), which matches straight-line tile code.
"""
from __future__ import annotations

import re

_RANGE = re.compile(r"\b([va])\[(\d+):(\d+)\]")
_SINGLE = re.compile(r"\b([va])(\d+)\b")
_FUNC = re.compile(r"^(_Z\w+):", re.M)


def _regs(text: str) -> set[str]:
    out = set()
    for m in _RANGE.finditer(text):
        out.update(f"{m.group(1)}{r}" for r in range(int(m.group(2)), int(m.group(3)) + 1))
    for m in _SINGLE.finditer(_RANGE.sub("", text)):
        out.add(m.group(1) + m.group(2))
    return out


def kernel_bodies(asm: str) -> dict[str, list[str]]:
    """Instruction lines (comments stripped) of every kernel in `asm`."""
    bodies = {}
    for m in _FUNC.finditer(asm):
        end = asm.find(".Lfunc_end", m.end())
        lines = [l.split(";")[0].strip() for l in asm[m.end() : end].split("\n")]
        bodies[m.group(1)] = [l for l in lines if l and not l.startswith(".") and not l.endswith(":")]
    return bodies


def violations(lines: list[str]) -> list[str]:
    pending: list[tuple[int, set[str]]] = []  # (line, destination registers), oldest first
    found = []
    for i, line in enumerate(lines):
        op, _, rest = line.partition(" ")
        if op == "s_waitcnt":
            m = re.search(r"lgkmcnt\((\d+)\)", rest)
            if m:
                del pending[: max(0, len(pending) - int(m.group(1)))]
            continue
        if op.startswith("s_"):
            continue
        parts = [p.strip() for p in rest.split(",")]
        dst = _regs(parts[0]) if parts and parts[0] else set()
        src = set().union(*(_regs(p) for p in parts[1:])) if len(parts) > 1 else set()
        is_ds = op.startswith("ds_")
        is_store = is_ds and (op.startswith("ds_write") or op.startswith("ds_store"))
        touched = src if "mfma" in op else (src | dst)
        if is_ds and not is_store:
            touched = src  # its destination is the new pending entry
        for j, regs in pending:
            hit = touched & regs
            if hit:
                found.append(f"{line}  <- uses {sorted(hit)} still being filled by: {lines[j]}")
        if is_ds:
            pending.append((i, set() if is_store else dst))
    return found
