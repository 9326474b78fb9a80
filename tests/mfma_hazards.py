"""Static check of gfx950 assembly for MFMA results read too early.

An XDL MFMA writes its destination over several passes, and a VALU, LDS or
memory instruction that reads that destination must wait until the passes
have retired (about 11 wait states for the 8-pass 16x16x32 bf16 MFMA; the
compiler inserts s_nop where the read follows in straight-line code).  The
check walks every path from each MFMA, fall-through and taken branches, and
reports a non-MFMA read of its destination that comes through a taken branch
within 8 issue slots, or within 2 slots on any path (s_nop n counts n + 1).
A dependent MFMA reading the previous result as its accumulator is checked
by the hardware and is not reported.
"""
from __future__ import annotations

import re

_REG = re.compile(r'\b([av])(?:\[(\d+):(\d+)\]|(\d+)(?!\w))')
_LABEL = re.compile(r'^(\.LBB\w+|_Z\w+):')


def _regs(text):
    out = set()
    for m in _REG.finditer(text):
        if m.group(2):
            out |= {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
        else:
            out.add((m.group(1), int(m.group(4))))
    return out


def _is_inst(s):
    return bool(s) and not s.startswith((';', '.')) and not s.endswith(':')


def scan(text, branch_slots=8, any_slots=2, window=11):
    """List of (mfma line, read line, slots, path of branch labels)."""
    lines = text.splitlines()
    labels = {m.group(1): i for i, l in enumerate(lines) for m in [_LABEL.match(l)] if m}
    insts = [i for i, l in enumerate(lines) if _is_inst(l.strip())]
    nxt = {insts[k]: insts[k + 1] for k in range(len(insts) - 1)}
    instset = set(insts)

    def first_after(line):
        for j in range(line + 1, len(lines)):
            if j in instset:
                return j
        return None

    found = []
    for i, l in enumerate(lines):
        s = l.strip()
        if not s.startswith('v_mfma'):
            continue
        dst = _regs(s.split(None, 1)[1].split(',')[0])
        stack, seen = [(nxt.get(i), 0, ())], set()
        while stack:
            j, slots, path = stack.pop()
            if j is None or slots >= window or (j, slots) in seen:
                continue
            seen.add((j, slots))
            t = lines[j].strip().split(';')[0].strip()
            op = t.split()[0] if t else ''
            if op == 's_endpgm':
                continue
            if op == 's_nop':
                stack.append((nxt.get(j), slots + 1 + int(t.split()[1], 0), path))
                continue
            if not op.startswith(('v_mfma', 's_')) and ',' in t:
                operands = t.split(None, 1)[1]
                srcs = operands if op.startswith(('global_store', 'buffer_store', 'ds_write', 'flat_store')) \
                    else ','.join(operands.split(',')[1:])
                if dst & _regs(srcs):
                    if (path and slots < branch_slots) or slots < any_slots:
                        found.append((i + 1, j + 1, slots, path))
                    continue
            if op.startswith('s_cbranch') or op == 's_branch':
                tgt = t.split()[1]
                if tgt in labels:
                    stack.append((first_after(labels[tgt]), slots + 1, path + (tgt,)))
                if op == 's_branch':
                    continue
            stack.append((nxt.get(j), slots + 1, path))
    return found
