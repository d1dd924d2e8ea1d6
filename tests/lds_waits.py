"""Check of compiled gfx950 assembly: no instruction may touch a register
that an LDS read is still filling.

The kernels issue some LDS reads through inline asm (so that the compiler
does not make them wait for in-flight LDS DMA) and wait for them with
explicit `s_waitcnt lgkmcnt(N)`.  The compiler cannot see that such a read
fills its output register asynchronously: if register pressure makes it copy
that register before the wait, the copy holds stale data.

The check splits each kernel into basic blocks and runs a forward dataflow
analysis over its control-flow graph.  The state at a point is the queue of
LDS operations that may still be outstanding, newest last, each with the
registers it fills (LDS operations complete in order, so lgkmcnt(N) retires
all but the newest N).  Where paths meet, queues are merged position by
position from the newest end, keeping every register any path may still be
filling.  Every instruction that reads or writes such a register is
reported.
"""
from __future__ import annotations

import re

_RANGE = re.compile(r"\b([va])\[(\d+):(\d+)\]")
_SINGLE = re.compile(r"\b([va])(\d+)\b")
_FUNC = re.compile(r"^(_Z\w+):", re.M)
_LABEL = re.compile(r"^(\.LBB\w+):")
_BRANCH = re.compile(r"^(s_branch|s_cbranch_\w+)\s+(\.LBB\w+)")


def _regs(text: str) -> set[str]:
    out = set()
    for m in _RANGE.finditer(text):
        out.update(f"{m.group(1)}{r}" for r in range(int(m.group(2)), int(m.group(3)) + 1))
    for m in _SINGLE.finditer(_RANGE.sub("", text)):
        out.add(m.group(1) + m.group(2))
    return out


def kernel_bodies(asm: str) -> dict[str, list[str]]:
    """Lines of every kernel in `asm` (comments stripped): instructions and
    basic-block labels."""
    bodies = {}
    for m in _FUNC.finditer(asm):
        end = asm.find(".Lfunc_end", m.end())
        lines = [l.split(";")[0].strip() for l in asm[m.end() : end].split("\n")]
        bodies[m.group(1)] = [l for l in lines if l and (not l.startswith(".") or _LABEL.match(l))]
    return bodies


def _blocks(lines: list[str]):
    """Basic blocks as (label, instructions, successor labels)."""
    blocks, cur, n = [], None, 0
    for line in lines:
        m = _LABEL.match(line)
        if m or cur is None:
            cur = [m.group(1) if m else f"entry{n}", [], []]
            n += 1
            blocks.append(cur)
            if m:
                continue
        cur[1].append(line)
        b = _BRANCH.match(line)
        if b:
            cur[2].append(b.group(2))
        if b or line.startswith("s_setpc") or line.startswith("s_endpgm"):
            cur = None  # a branch ends the block (a conditional one falls through, below)
    # fall-through edges
    for i, blk in enumerate(blocks[:-1]):
        last = blk[1][-1] if blk[1] else ""
        if not last.startswith("s_branch") and not last.startswith("s_endpgm") and not last.startswith("s_setpc"):
            blk[2].append(blocks[i + 1][0])
    return blocks


# lgkmcnt counts at most 15 operations: a wave cannot have more in flight
_MAX_PENDING = 16


def _merge(a, b):
    """Queues merged from the newest end; each entry a frozenset of registers."""
    n = max(len(a), len(b))
    pa = [frozenset()] * (n - len(a)) + list(a)
    pb = [frozenset()] * (n - len(b)) + list(b)
    return tuple(x | y for x, y in zip(pa, pb))


def _step(state, line, report=None):
    op, _, rest = line.partition(" ")
    if op == "s_waitcnt":
        m = re.search(r"lgkmcnt\((\d+)\)", rest)
        if m:
            k = int(m.group(1))
            state = state[len(state) - k :] if k < len(state) else state
        return state
    if op.startswith("s_"):
        return state
    parts = [p.strip() for p in rest.split(",")]
    dst = _regs(parts[0]) if parts and parts[0] else set()
    src = set().union(*(_regs(p) for p in parts[1:])) if len(parts) > 1 else set()
    is_ds = op.startswith("ds_")
    is_store = is_ds and (op.startswith("ds_write") or op.startswith("ds_store"))
    touched = src if ("mfma" in op or (is_ds and not is_store)) else (src | dst)
    if report is not None:
        pending = set().union(*state) if state else set()
        hit = touched & pending
        if hit:
            report.append(f"{line}  <- uses {sorted(hit)} while an LDS read may still fill them")
    if is_ds:
        state = (state + (frozenset() if is_store else frozenset(dst),))[-_MAX_PENDING:]
    return state


def violations(lines: list[str]) -> list[str]:
    blocks = _blocks(lines)
    index = {b[0]: i for i, b in enumerate(blocks)}
    preds = {i: [] for i in range(len(blocks))}
    for i, b in enumerate(blocks):
        for s in b[2]:
            if s in index:
                preds[index[s]].append(i)
    out_state = [None] * len(blocks)
    changed = True
    while changed:
        changed = False
        for i, b in enumerate(blocks):
            ins = [out_state[p] for p in preds[i] if out_state[p] is not None]
            state = ()
            for s in ins:
                state = _merge(state, s)
            for line in b[1]:
                state = _step(state, line)
            if state != out_state[i]:
                out_state[i] = state
                changed = True
    found = []
    for i, b in enumerate(blocks):
        state = ()
        for s in (out_state[p] for p in preds[i] if out_state[p] is not None):
            state = _merge(state, s)
        for line in b[1]:
            state = _step(state, line, found)
    return found
