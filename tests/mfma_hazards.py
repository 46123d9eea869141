"""Static check of inline-assembly MFMA results in the generated AMD assembly.

Where an MFMA is written as inline assembly, the compiler does not know how
long the matrix core takes to write the result, so it inserts no wait states
after it. The kernels rely on their own schedule for that (an accumulator is
next used by the same MFMA, or after an explicit run of s_nop), but the
register allocator may still place a copy or a spill of an accumulator right
behind the MFMA that writes it, which then reads the old value. This module
finds such places in the assembly the compiler emits for our own sources.

The analysis: instructions are split into basic blocks at labels and after
branches; an MFMA sets, for each register it writes, the number of wait
states still owed (MFMA_WAIT); every instruction pays one wait state, an
``s_nop N`` pays N + 1; states flow along fall-through and branch edges (the
largest debt of any predecessor) until nothing changes. A non-MFMA
instruction that names a register with a debt left, or an MFMA that reads one
as a source other than its own accumulator, is a hazard.

A second check (scan_sgpr_vmem) follows the same flow for scalar registers
written by a vector-ALU instruction (v_readlane and v_readfirstlane, the
compiler's reloads of spilled scalar registers among them): a vector memory
instruction (buffer, global, flat, scratch) must not read such a register
within VMEM_SGPR_WAIT wait states. The compiler keeps that distance for its
own loads, not for the loads written as inline assembly, whose buffer
descriptors are scalar registers.
"""
from __future__ import annotations

import re

# Wait states between a v_mfma_f32_16x16x32_f16 (eight passes) and another
# instruction touching its destination; the kernels' own explicit wait before
# reading accumulators (three s_nop 7) pays 24.
MFMA_WAIT = {"v_mfma_f32_16x16x32_f16": 18}

# Wait states between a vector-ALU write of a scalar register and a vector
# memory instruction that reads it.
VMEM_SGPR_WAIT = 5
_VMEM = ("buffer_", "global_", "flat_", "scratch_")
_SREG = re.compile(r"(?<![\w.])(?:s\[(\d+):(\d+)\]|s(\d+)(?!\w))")

_REG = re.compile(r"(?<![\w.])([va])(?:\[(\d+):(\d+)\]|(\d+)(?!\w))")
_BRANCH = re.compile(r"^s_(cbranch_\w+|branch)\s+(\S+)")


def _regs(text: str) -> set[str]:
    out = set()
    for m in _REG.finditer(text):
        kind = m.group(1)
        if m.group(4) is not None:
            out.add(f"{kind}{m.group(4)}")
        else:
            for r in range(int(m.group(2)), int(m.group(3)) + 1):
                out.add(f"{kind}{r}")
    return out


def functions(asm: str) -> dict[str, list[str]]:
    """Instruction and label lines of every function in a compiler -S listing."""
    out: dict[str, list[str]] = {}
    name = None
    for raw in asm.split("\n"):
        line = raw.split(";")[0].strip()
        if not line:
            continue
        m = re.match(r"^([A-Za-z_][\w.$]*):$", line)
        if m and not line.startswith(".L"):
            name = m.group(1)
            out[name] = []
            continue
        if name is None:
            continue
        if line.startswith(".Lfunc_end"):
            name = None
            continue
        if line.startswith(".") and not line.endswith(":"):
            continue  # directives
        out[name].append(line)
    return out


def _blocks(lines: list[str]):
    """Basic blocks: (label or None, instructions, successor labels, falls through)."""
    blocks = []
    cur_label, cur = None, []

    def close(falls):
        blocks.append([cur_label, cur, [], falls])

    for line in lines:
        if line.endswith(":"):
            if cur or cur_label is not None:
                close(True)
            cur_label, cur = line[:-1], []
            continue
        cur.append(line)
        b = _BRANCH.match(line)
        if b or line.startswith("s_endpgm") or line.startswith("s_setpc"):
            uncond = bool(b and b.group(1) == "branch") or not b
            close(not uncond)
            if b:
                blocks[-1][2].append(b.group(2))
            cur_label, cur = None, []
    if cur or cur_label is not None:
        close(False)
    return blocks


def scan(lines: list[str], wait: dict[str, int] = MFMA_WAIT) -> list[tuple[int, str, str]]:
    """Hazards in one function: (block index, instruction, register)."""
    blocks = _blocks(lines)
    index = {b[0]: i for i, b in enumerate(blocks) if b[0] is not None}
    preds: list[list[int]] = [[] for _ in blocks]
    for i, (_, _, succ, falls) in enumerate(blocks):
        for s in succ:
            if s in index:
                preds[index[s]].append(i)
        if falls and i + 1 < len(blocks):
            preds[i + 1].append(i)
    state_out: list[dict[str, int]] = [dict() for _ in blocks]

    def run(i, state, report):
        state = dict(state)
        for ins in blocks[i][1]:
            op = ins.split()[0]
            regs = _regs(ins[len(op):])
            if op.startswith("v_mfma"):
                parts = [p.strip() for p in ins[len(op):].split(",")]
                dst = _regs(parts[0])
                srcs = set().union(*(_regs(p) for p in parts[1:-1])) if len(parts) > 2 else set()
                accum = _regs(parts[-1]) if len(parts) > 1 else set()
                for r in srcs | (accum - dst):
                    if state.get(r, 0) > 0:
                        report.append((i, ins, r))
                for r in dst:
                    if state.get(r, 0) > 0 and accum != dst:
                        report.append((i, ins, r))
                paid = 1
            else:
                for r in regs:
                    if state.get(r, 0) > 0:
                        report.append((i, ins, r))
                paid = int(ins.split()[1], 0) + 1 if op == "s_nop" else 1
            state = {r: w - paid for r, w in state.items() if w - paid > 0}
            if op in wait:
                parts = [p.strip() for p in ins[len(op):].split(",")]
                for r in _regs(parts[0]):
                    state[r] = wait[op]
        return state

    changed = True
    while changed:
        changed = False
        for i in range(len(blocks)):
            start: dict[str, int] = {}
            for p in preds[i]:
                for r, w in state_out[p].items():
                    if w > start.get(r, 0):
                        start[r] = w
            out = run(i, start, [])
            if out != state_out[i]:
                state_out[i] = out
                changed = True
    report: list[tuple[int, str, str]] = []
    for i in range(len(blocks)):
        start = {}
        for p in preds[i]:
            for r, w in state_out[p].items():
                if w > start.get(r, 0):
                    start[r] = w
        run(i, start, report)
    return report


def _sregs(text: str) -> set[str]:
    out = set()
    for m in _SREG.finditer(text):
        if m.group(3) is not None:
            out.add(f"s{m.group(3)}")
        else:
            for r in range(int(m.group(1)), int(m.group(2)) + 1):
                out.add(f"s{r}")
    return out


def _flow(lines: list[str], step) -> list[tuple[int, str, str]]:
    """Runs step(instruction, state, report) -> state over the basic blocks
    until the states at block ends stop changing (the largest debt of any
    predecessor at a block's start), then once more collecting reports."""
    blocks = _blocks(lines)
    index = {b[0]: i for i, b in enumerate(blocks) if b[0] is not None}
    preds: list[list[int]] = [[] for _ in blocks]
    for i, (_, _, succ, falls) in enumerate(blocks):
        for t in succ:
            if t in index:
                preds[index[t]].append(i)
        if falls and i + 1 < len(blocks):
            preds[i + 1].append(i)
    state_out: list[dict[str, int]] = [dict() for _ in blocks]

    def start(i):
        st: dict[str, int] = {}
        for p in preds[i]:
            for r, w in state_out[p].items():
                if w > st.get(r, 0):
                    st[r] = w
        return st

    def run(i, state, report):
        for ins in blocks[i][1]:
            state = step(i, ins, state, report)
        return state

    changed = True
    while changed:
        changed = False
        for i in range(len(blocks)):
            out = run(i, start(i), [])
            if out != state_out[i]:
                state_out[i] = out
                changed = True
    report: list[tuple[int, str, str]] = []
    for i in range(len(blocks)):
        run(i, start(i), report)
    return report


def scan_sgpr_vmem(lines: list[str], wait: int = VMEM_SGPR_WAIT) -> list[tuple[int, str, str]]:
    """Vector memory instructions reading a scalar register that a vector-ALU
    instruction wrote fewer than `wait` wait states before: (block, instruction,
    register)."""

    def step(i, ins, state, report):
        op = ins.split()[0]
        if op.startswith(_VMEM):
            for r in _sregs(ins[len(op):]):
                if state.get(r, 0) > 0:
                    report.append((i, ins, r))
        paid = int(ins.split()[1], 0) + 1 if op == "s_nop" else 1
        state = {r: w - paid for r, w in state.items() if w - paid > 0}
        if op.startswith("v_") and not op.startswith("v_mfma"):
            dst = ins[len(op):].split(",")[0].strip()
            if _SREG.fullmatch(dst):
                for r in _sregs(dst):
                    state[r] = wait
        return state

    return _flow(lines, step)
