"""Hazard check for the MFMAs that kernels issue as inline asm.

The compiler inserts the wait states that the matrix instructions need
(between a VALU write and an MFMA reading it, and between an MFMA and a
later read of its result) only for MFMAs it selected itself: an inline-asm
MFMA is opaque to its hazard recognizer. A kernel that issues MFMAs as asm
(to keep its accumulators in place in AGPRs) must separate them from every
other access of the same registers by itself, including the register moves
and spills that the register allocator places where it likes.

This module reads the device assembly of a build (``hipcc -S
--cuda-device-only``), builds each kernel's control-flow graph and checks
every path:

* from an asm MFMA forward, no instruction other than another asm MFMA that
  accumulates into exactly the same registers touches its accumulator
  registers within ``AFTER_MFMA`` wait states;
* into an asm MFMA backward, no instruction other than an MFMA writes one of
  its A, B or C registers (or, for the scaled MFMAs, a scale register)
  within ``BEFORE_MFMA`` wait states.

It also flags flat memory instructions in these kernels: a flat access
counts in both vmcnt and lgkmcnt, and their barriers wait for lgkmcnt(0)
(the LDS reads), so a flat store would be drained at the next barrier
instead of overlapping the K loop.

Wait states are counted as the hardware documentation counts them: one per
instruction, N + 1 for ``s_nop N``. The bounds are above what gfx950 asks
for a 16x16x32 MFMA (its result is read back after at most 19 wait states
for the longest MFMAs of the family; a VALU result feeds an MFMA after 2).
"""
from __future__ import annotations

import re
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Set, Tuple

AFTER_MFMA = 32
BEFORE_MFMA = 4

_REG = re.compile(r"^([va])(?:(\d+)|\[(\d+):(\d+)\])$")


def _regs(tok: str) -> Set[Tuple[str, int]]:
    m = _REG.match(tok)
    if not m:
        return set()
    kind = m.group(1)
    if m.group(2) is not None:
        return {(kind, int(m.group(2)))}
    return {(kind, r) for r in range(int(m.group(3)), int(m.group(4)) + 1)}


# instructions whose first operand is not a register they write
_NO_DEST = ("s_", "global_store", "buffer_store", "scratch_store", "ds_write", "ds_store",
            "global_load_lds", "buffer_load_dword off", "v_cmp", "v_cmpx", "global_atomic")


@dataclass
class Insn:
    text: str
    op: str
    asm: bool                      # inside an inline-asm region
    label: Optional[str] = None    # label that starts at this instruction
    writes: Set[Tuple[str, int]] = field(default_factory=set)
    reads: Set[Tuple[str, int]] = field(default_factory=set)

    @property
    def is_mfma(self) -> bool:
        return self.op.startswith("v_mfma")

    def waits(self) -> int:
        if self.op == "s_nop":
            return int(self.text.split()[1], 0) + 1
        return 1


def _parse_insn(line: str, asm: bool) -> Insn:
    body = line.split(";")[0].strip()
    op = body.split()[0]
    ops = [o.strip() for o in body[len(op):].split(",")] if len(body) > len(op) else []
    ops = [o.split()[0] for o in ops if o]
    ins = Insn(text=body, op=op, asm=asm)
    if op.startswith("v_mfma"):
        # every register operand after the destination is read: A, B, C and,
        # for the scaled MFMAs, the two scale registers
        ins.writes = _regs(ops[0])
        for o in ops[1:]:
            ins.reads |= _regs(o)
        return ins
    dest_first = ops and not op.startswith(_NO_DEST) and (
        op.startswith("v_") or op.startswith(("ds_read", "ds_load", "global_load", "buffer_load", "scratch_load")))
    for k, o in enumerate(ops):
        r = _regs(o)
        if k == 0 and dest_first:
            ins.writes |= r
        else:
            ins.reads |= r
    return ins


def kernel_body(asm_text: str, symbol_part: str) -> List[Tuple[str, List[Insn]]]:
    """Instructions of every kernel whose symbol contains ``symbol_part``."""
    out = []
    lines = asm_text.split("\n")
    i = 0
    while i < len(lines):
        line = lines[i]
        m = re.match(r"^([A-Za-z_][\w.$]*):", line)
        if m and symbol_part in m.group(1) and not m.group(1).startswith(".L"):
            name = m.group(1)
            insns: List[Insn] = []
            asm = False
            pending_label = None
            i += 1
            while i < len(lines) and not lines[i].startswith(".Lfunc_end"):
                t = lines[i].strip()
                i += 1
                if not t:
                    continue
                if t.startswith(";;#ASMSTART"):
                    asm = True
                    continue
                if t.startswith(";;#ASMEND"):
                    asm = False
                    continue
                if t.startswith(";") or t.startswith("."):
                    lm = re.match(r"^(\.L[\w$]+):", t)
                    if lm:
                        pending_label = lm.group(1)
                    continue
                ins = _parse_insn(t, asm)
                ins.label = pending_label
                pending_label = None
                insns.append(ins)
            out.append((name, insns))
        else:
            i += 1
    return out


def _cfg(insns: List[Insn]) -> Tuple[List[List[int]], List[List[int]]]:
    where = {ins.label: k for k, ins in enumerate(insns) if ins.label}
    succ: List[List[int]] = [[] for _ in insns]
    for k, ins in enumerate(insns):
        op = ins.op
        target = ins.text.split()[-1] if op.startswith(("s_branch", "s_cbranch")) else None
        if target is not None and target in where:
            succ[k].append(where[target])
        falls = not (op == "s_branch" or op.startswith("s_endpgm") or op.startswith("s_setpc"))
        if falls and k + 1 < len(insns):
            succ[k].append(k + 1)
    pred: List[List[int]] = [[] for _ in insns]
    for k, ss in enumerate(succ):
        for s in ss:
            pred[s].append(k)
    return succ, pred


def check_kernel(insns: List[Insn]) -> List[str]:
    """Violations (empty when every path keeps the bounds)."""
    succ, pred = _cfg(insns)
    bad: List[str] = [f"{x.text!r} is a flat memory access" for x in insns
                      if x.op.startswith(("flat_load", "flat_store", "flat_atomic"))]
    for k, m in enumerate(insns):
        if not (m.is_mfma and m.asm):
            continue
        acc = {r for r in m.writes if r[0] == "a"} or m.writes
        # forward from the MFMA
        seen: Dict[int, int] = {}
        stack = [(s, 0) for s in succ[k]]
        while stack:
            j, w = stack.pop()
            if w >= AFTER_MFMA or seen.get(j, -1) >= AFTER_MFMA - w:
                continue
            seen[j] = AFTER_MFMA - w
            ins = insns[j]
            same = ins.is_mfma and ins.asm and ins.writes == m.writes
            if not same and (ins.reads | ins.writes) & acc:
                bad.append(f"{ins.text!r} touches the result of {m.text!r} {w} wait states after it")
                continue
            stack.extend((s, w + ins.waits()) for s in succ[j])
        # backward into the MFMA
        srcs = m.reads
        seen = {}
        stack = [(p, 0) for p in pred[k]]
        while stack:
            j, w = stack.pop()
            if w >= BEFORE_MFMA or seen.get(j, -1) >= BEFORE_MFMA - w:
                continue
            seen[j] = BEFORE_MFMA - w
            ins = insns[j]
            if not ins.is_mfma and ins.writes & srcs:
                bad.append(f"{ins.text!r} writes an operand of {m.text!r} {w} wait states before it")
                continue
            stack.extend((p, w + ins.waits()) for p in pred[j])
    return bad


def check_asm(asm_text: str, symbol_part: str) -> Dict[str, Tuple[int, List[str]]]:
    """{kernel: (asm MFMAs checked, violations)} for the matching kernels."""
    res = {}
    for name, insns in kernel_body(asm_text, symbol_part):
        n = sum(1 for x in insns if x.is_mfma and x.asm)
        res[name] = (n, check_kernel(insns))
    return res
