"""A static check of compiled kernels (hipcc -S output) for the defect the replay found in
the dK/dV kernel's row search: a lane mask made by a compare inside a loop whose lanes
leave one by one, and used together with EXEC after that loop.

A compare writes 0 for inactive lanes, so such a mask holds only the lanes still in the
loop at its last evaluation; ``s_and_b64 vcc, exec, mask`` after the loop then reads
"false" for every lane that left earlier, and a branch on it can go the wrong way.

Loops come from the compiler's block annotations ("; Loop: Header=BB..", "Loop Header");
a loop counts as lane-by-lane when its blocks narrow EXEC with the loop-exit idiom
``s_andn2_b64 exec, exec, X``.  Loops that every lane leaves together are not flagged:
their compares are made under the EXEC the loop was entered with.
"""
from __future__ import annotations

import re

from . import emulator as E

_BLOCK = re.compile(r"^\s*(?:\.L(BB\d+_\d+):|;\s*%bb\.\d+:)(.*)$")


def _loop_sets(path, name):
    """For each instruction of ``name`` (in parse order), the loop headers around it."""
    out, cur, on = [], frozenset(), False
    with open(path) as fh:
        for raw in fh:
            code = raw.split(";")[0].strip()
            if not on:
                on = code == name + ":"
                continue
            if code.startswith(".Lfunc_end"):
                break
            m = _BLOCK.match(raw)
            if m:
                label, rest = m.group(1), m.group(2)
                hdr = re.search(r"Header=(BB\d+_\d+)", rest)
                cur = {hdr.group(1)} if hdr else set()
                if label and "Loop Header" in rest:
                    cur.add(label)
                cur = frozenset(cur)
                continue
            if not code or code.startswith(".") or code.endswith(":"):
                continue
            out.append(cur)
    return out


def _mask_def(x):
    if x.op.startswith("v_cmp") and x.args and not isinstance(x.args[0], str):
        o = x.args[0]
        if o.kind == "s" and o.n == 2:
            return o.idx
    return None


def _sgprs_written(x):
    """SGPRs an instruction writes (destination operands; carry-out SGPR pairs included)."""
    regs = set()
    if not x.args or isinstance(x.args[0], str):
        return regs
    first = x.args[0]
    if first.kind == "s" and not x.op.startswith(("s_cmp", "s_bitcmp")):  # compares only read theirs
        regs |= set(range(first.idx, first.idx + first.n))
    if x.op.startswith("v_") and len(x.args) > 1 and not isinstance(x.args[1], str) and x.args[1].kind == "s" \
            and ("_co_" in x.op or x.op.startswith(("v_mad_u64", "v_mad_i64", "v_div_scale"))):
        regs |= set(range(x.args[1].idx, x.args[1].idx + x.args[1].n))
    return regs


def _exec_uses(x):
    """SGPR-pair lane masks an instruction combines with EXEC."""
    a = x.args
    if x.op == "s_and_b64" and len(a) == 3:
        if a[1].kind == "exec" and a[2].kind == "s":
            return [a[2].idx]
        if a[2].kind == "exec" and a[1].kind == "s":
            return [a[1].idx]
    if x.op.endswith("saveexec_b64") and a[1].kind == "s":
        return [a[1].idx]
    if x.op == "v_cndmask_b32_e64" and a[3].kind == "s":
        return [a[3].idx]
    return []


def lane_mask_reuse_sites(path, name):
    """(compare line, compare, use line, use) for every flagged site of kernel ``name``."""
    ins, _ = E.parse_function(path, name)
    loops = _loop_sets(path, name)
    if len(loops) != len(ins):
        raise RuntimeError(f"{name}: block annotations do not line up with the instructions")
    lane_by_lane = set()
    for x, lp in zip(ins, loops):
        if x.op == "s_andn2_b64" and x.args[0].kind == "exec" and x.args[1].kind == "exec":
            lane_by_lane |= lp
    sites = []
    for i, x in enumerate(ins):
        for reg in _exec_uses(x):
            j = i - 1
            while j >= 0 and not (_sgprs_written(ins[j]) & {reg, reg + 1}):
                j -= 1
            if j >= 0 and _mask_def(ins[j]) == reg and (loops[j] - loops[i]) & lane_by_lane:
                sites.append((ins[j].line, ins[j].text, x.line, x.text))
    return sites
