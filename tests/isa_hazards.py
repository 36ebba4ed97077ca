"""Checks on the gfx950 assembly of the library's kernels (test helper).

A VGPR written by a matrix instruction (v_mfma_*) may be read by a vector
ALU, LDS or memory instruction, or by another matrix instruction as its A or
B operand, only after enough independent instructions ("wait states"): the
hardware does not interlock that dependency, and the compiler inserts s_nop
instructions to provide it.  On straight-line code the compiler in this
toolchain separates such a read from the 16x16 bf16 products by at least 8
wait states.  It was seen to leave only 2 when the product was the last
instruction before a conditional branch and the read sat in the block where
both paths join; the kernel then read stale values, with no error.
``short_reads`` walks every control-flow path from each matrix instruction
and reports reads of its result closer than ``need`` wait states.
"""
from __future__ import annotations

import re

_VRANGE = re.compile(r"v\[(\d+):(\d+)\]")
_VREG = re.compile(r"v(\d+)$")
_LABEL = re.compile(r"^([.\w]+):$")
_KERNEL = re.compile(r"^(_Z\w+):", re.M)


def vgprs(operand: str) -> set[int]:
    operand = operand.strip()
    m = _VRANGE.match(operand)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = _VREG.match(operand)
    return {int(m.group(1))} if m else set()


def _operands(ins: str) -> list[str]:
    parts = ins.split(None, 1)
    return [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []


def _parse(body: list[str]):
    """Instructions (comments dropped) and label -> instruction index."""
    ins, labels = [], {}
    for line in body:
        t = line.split(";")[0].strip()
        if not t:
            continue
        m = _LABEL.match(t)
        if m:
            labels[m.group(1)] = len(ins)
            continue
        if t.startswith("."):
            continue
        ins.append(t)
    return ins, labels


def _successors(ins, labels, i):
    op = ins[i].split()[0]
    if op == "s_branch":
        return [labels[ins[i].split()[1]]]
    if op.startswith("s_cbranch"):
        return [i + 1, labels[ins[i].split()[1]]]
    if op in ("s_endpgm", "s_setpc_b64", "s_trap"):
        return []
    return [i + 1]


def _wait_states(ins: str) -> int:
    parts = ins.split()
    return int(parts[1], 0) + 1 if parts[0] == "s_nop" else 1


def _reads(ins: str) -> set[int]:
    op = ins.split()[0]
    ops = _operands(ins)
    if op.startswith("v_mfma"):
        # A and B operands; the accumulator (C) chain is not this hazard.
        out = set()
        for o in ops[1:3]:
            out |= vgprs(o)
        return out
    if op.startswith(("v_", "ds_", "global_", "buffer_", "flat_", "scratch_")):
        out = set()
        for o in ops:
            out |= vgprs(o)
        return out
    return set()


def kernels(asm: str) -> list[str]:
    return _KERNEL.findall(asm)


def short_reads(asm: str, kernel: str, need: int = 8):
    """(product, reader, wait states) for every read of a matrix result fewer
    than `need` wait states after the product along some path of `kernel`."""
    start = asm.index(kernel + ":")
    end = asm.index(".Lfunc_end", start)
    ins, labels = _parse(asm[start:end].splitlines()[1:])
    found = []
    for k, t in enumerate(ins):
        if not t.startswith("v_mfma"):
            continue
        dst = vgprs(_operands(t)[0])
        stack = [(n, 0) for n in _successors(ins, labels, k)]
        seen = set()
        while stack:
            n, w = stack.pop()
            if n >= len(ins) or (n, w) in seen:
                continue
            seen.add((n, w))
            u = ins[n]
            if _reads(u) & dst:
                found.append((t, u, w))
                continue
            if u.startswith("v_mfma") and vgprs(_operands(u)[0]) == dst:
                continue  # the next product of an accumulator chain takes over
            w2 = w + _wait_states(u)
            if w2 < need:
                stack.extend((m, w2) for m in _successors(ins, labels, n))
    return found
