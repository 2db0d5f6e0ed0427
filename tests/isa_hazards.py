"""Scan gfx950 assembly (hipcc -save-temps output) for MFMA data hazards the
hardware does not interlock: an instruction reading the result of a
v_mfma_f32_32x32x16_bf16 too soon after it, or a VALU instruction writing one
of its sources just before it.  The compiler inserts the wait states around
the MFMAs it emits itself; the QK MFMAs of the head_dim-512 prefill are
inline assembly, which it cannot see, so their neighbourhood is checked here.

Wait states: each instruction counts one, `s_nop N` counts N + 1.  A read of
an MFMA result fewer than 12 wait states after it is flagged (12 is what the
compiler inserts before a dependent read of this MFMA on gfx950), unless it
is the next MFMA accumulating into exactly the same registers (no wait states
needed); so is a VALU write of an MFMA source fewer than 2 before it.
"""
from __future__ import annotations

import re


def _regs(tok: str) -> set[int]:
    out: set[int] = set()
    for m in re.finditer(r'\bv\[(\d+):(\d+)\]|\bv(\d+)\b', tok):
        if m.group(3):
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def _instrs(lines):
    for i, raw in enumerate(lines):
        t = raw.strip()
        if not t or t.startswith(';') or t.startswith('.') or t.endswith(':'):
            continue
        yield i, t


def find_hazards(text: str, read_window: int = 12, write_window: int = 2) -> list[str]:
    lines = text.splitlines()
    ins = list(_instrs(lines))
    found = []
    for k, (i, t) in enumerate(ins):
        m = re.match(r'v_mfma\S*\s+v\[(\d+):(\d+)\],\s*(\S+),\s*(\S+),\s*(\S+)', t)
        if not m:
            continue
        dst = set(range(int(m.group(1)), int(m.group(2)) + 1))
        ws = 0
        for j, u in ins[k + 1:]:
            if u.startswith('s_nop'):
                ws += int(u.split()[1]) + 1
                if ws >= read_window:
                    break
                continue
            parts = u.split(None, 1)
            op = parts[0]
            args = parts[1].split(',') if len(parts) > 1 else []
            if op.startswith('v_mfma'):
                d2 = _regs(args[0])
                ab = _regs(args[1]) | _regs(args[2])
                c = _regs(args[3]) if len(args) > 3 else set()
                if ab & dst or (c & dst and c != dst):
                    found.append(f"line {j + 1}: MFMA reads the result of line {i + 1} early: {u}")
                if d2 == dst:
                    break
            else:
                stores = op.startswith(('ds_write', 'global_store', 'buffer_store',
                                        'scratch_store', 'flat_store'))
                srcs = _regs(','.join(args if stores else args[1:]))
                dst_w = _regs(args[0]) if (args and op.startswith('v_') and not stores) else set()
                if srcs & dst or dst_w & dst:
                    found.append(f"line {j + 1}: {ws} wait states after the MFMA at line "
                                 f"{i + 1}: {u}")
                    break
            ws += 1
            if ws >= read_window:
                break
    for k, (i, t) in enumerate(ins):
        m = re.match(r'v_mfma\S*\s+(\S+),\s*(\S+),\s*(\S+),\s*(\S+)', t)
        if not m:
            continue
        srcs = _regs(m.group(2)) | _regs(m.group(3)) | _regs(m.group(4))
        ws = 0
        for j, u in reversed(ins[max(0, k - 40):k]):
            if u.startswith('s_nop'):
                ws += int(u.split()[1]) + 1
            else:
                op = u.split()[0]
                if (op.startswith('v_') and not op.startswith(('v_mfma', 'v_readlane',
                                                               'v_readfirstlane', 'v_cmp'))):
                    args = u.split(None, 1)
                    d = _regs(args[1].split(',')[0]) if len(args) > 1 else set()
                    if d & srcs:
                        found.append(f"line {j + 1} writes a source of the MFMA at line {i + 1} "
                                     f"{ws} wait states before it: {u}")
                ws += 1
            if ws >= write_window:
                break
    return found
