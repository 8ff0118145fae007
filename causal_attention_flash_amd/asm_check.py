"""Build-time check of the asynchronous transposing LDS reads (attn_direct.h).

DOffsets::tr_async issues ds_read_b64_tr_b16 as inline assembly, which the
compiler treats as an ordinary instruction whose result exists at once; the data
only arrives after the s_waitcnt lgkmcnt(0) that lds_wait() places.  The code is
correct only if, between such a read and that wait, no instruction reads, writes
or copies the read's destination registers (a copy to an AGPR under register
pressure is the typical way this breaks), no such read takes its address from a
pending destination, and no branch leaves that stretch of code.  Source code
cannot force this; this module checks the compiler's output for it.

check_text(asm) returns a list of violations found in hipcc -S device assembly
(empty: all good); build.py runs it on every source that uses tr_async and
fails the build on any violation.
"""
from __future__ import annotations

import re

_VREG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")
_KERNEL = re.compile(r"^([A-Za-z_.$][\w.$]*):[^\n]*$(.*?)^\.Lfunc_end", re.M | re.S)
_LABEL = re.compile(r"^([.\w$]+):")


def _vregs(text: str) -> set:
    out = set()
    for m in _VREG.finditer(text):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def check_function(name: str, body: str) -> tuple:
    """Scan one function; return (violations, number of asynchronous reads)."""
    lines = body.split("\n")
    labels = {}
    for i, ln in enumerate(lines):
        m = _LABEL.match(ln.strip())
        if m:
            labels[m.group(1)] = i
    bad = []
    pending = {}  # register -> line of the read that writes it
    branches = []  # (line, target) seen while reads are pending
    in_asm = False
    nreads = 0
    for i, ln in enumerate(lines):
        if ";;#ASMSTART" in ln:
            in_asm = True
            continue
        if ";;#ASMEND" in ln:
            in_asm = False
            continue
        t = ln.split(";")[0].strip()
        if not t or _LABEL.match(t):
            continue
        op, _, rest = t.partition(" ")
        if in_asm and op == "ds_read_b64_tr_b16":
            ops = [o.strip() for o in rest.split(",")]
            dst, addr = _vregs(ops[0]), _vregs(ops[1]) if len(ops) > 1 else set()
            if (dst | addr) & set(pending):
                bad.append(f"{name}: line {i}: '{t}' uses a pending destination")
            for r in dst:
                pending[r] = i
            nreads += 1
            continue
        if in_asm and op == "s_waitcnt" and "lgkmcnt(0)" in rest:
            if pending:
                first = min(pending.values())
                for bi, target in branches:
                    if not first < labels.get(target, -1) < i:
                        bad.append(f"{name}: line {bi}: branch to {target} leaves a pending read's range")
            pending.clear()
            branches.clear()
            continue
        if not pending:
            continue
        if op.startswith("s_cbranch") or op == "s_branch" or op.startswith("s_setpc") or op == "s_endpgm":
            target = rest.strip().split()[-1] if rest.strip() else ""
            branches.append((i, target))
            if op == "s_endpgm" or op.startswith("s_setpc"):
                bad.append(f"{name}: line {i}: '{op}' with asynchronous reads pending")
            continue
        hit = _vregs(rest) & set(pending)
        if hit:
            bad.append(f"{name}: line {i}: '{t}' touches pending v{min(hit)}")
    if pending:
        bad.append(f"{name}: asynchronous reads pending at the end of the function")
    return bad, nreads


def check_text(asm: str) -> list:
    """All violations in a device assembly file; [] if none."""
    bad = []
    for m in _KERNEL.finditer(asm):
        if "ds_read_b64_tr_b16" in m.group(2):
            bad += check_function(m.group(1), m.group(2))[0]
    return bad


def count_reads(asm: str) -> int:
    """Number of asynchronous transposing reads the file's functions issue."""
    return sum(check_function(m.group(1), m.group(2))[1] for m in _KERNEL.finditer(asm))
