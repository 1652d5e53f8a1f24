"""Scan gfx950 assembly of libmesa's kernels for MFMA operand hazards.

A multi-pass v_mfma reads its accumulator input (SrcC) over several passes.
When the compiler gives an MFMA a SrcC register range different from its
destination, a later instruction may overwrite those SrcC registers before
the MFMA has read them; the observed result is a corrupted accumulator
component (seen on gfx950 with a 16x16x4 f32 MFMA whose SrcC came from the
MFMA issued just before it, the SrcC registers being rewritten 9 wait states
later).  This check compiles every kernel source to assembly and reports each
MFMA with SrcC != Dst whose SrcC registers are written again by a VALU or
load instruction (a register or a range) before MIN_WAIT_STATES wait states
have passed (one per instruction, N+1 per s_nop N) -- about twice the gap
that was observed to fail.  A later MFMA's own destination is not such a
write: MFMAs run in order and write their results only after their passes.
"""
from __future__ import annotations

import os
import re
import subprocess
import tempfile

from . import build as B

WINDOW = 64
MIN_WAIT_STATES = 16
_MFMA = re.compile(r"\bv_mfma_\S+\s+([av])\[(\d+):(\d+)\],\s*[^,]+,\s*[^,]+,\s*([av])\[(\d+):(\d+)\]")
_WRITE = re.compile(r"^\s*(v_\S+|ds_read\S*|global_load\S*|buffer_load\S*)\s+([av])(?:\[(\d+):(\d+)\]|(\d+)\b)")


def _regs(kind, lo, hi):
    return {(kind, r) for r in range(int(lo), int(hi) + 1)}


def scan_asm(text: str):
    """Returns a list of (line_no, mfma_line, clobber_line) too-close SrcC rewrites."""
    lines = text.splitlines()
    out = []
    for i, line in enumerate(lines):
        m = _MFMA.search(line)
        if not m:
            continue
        dst = _regs(m.group(1), m.group(2), m.group(3))
        src = _regs(m.group(4), m.group(5), m.group(6))
        if dst == src:
            continue
        pending = src - dst
        waits = 0
        for j in range(i + 1, min(i + 1 + WINDOW, len(lines))):
            t = lines[j].strip()
            if not t or t.startswith(";") or t.startswith(".") or t.endswith(":"):
                continue
            nop = re.match(r"s_nop\s+(\d+)", t)
            waits += int(nop.group(1)) + 1 if nop else 1
            if waits > MIN_WAIT_STATES:
                break
            w = _WRITE.match(lines[j])
            if not w or w.group(1).startswith("v_mfma"):
                continue
            kind = w.group(2)
            if w.group(3) is not None:
                wr = _regs(kind, w.group(3), w.group(4))
            else:
                wr = {(kind, int(w.group(5)))}
            if wr & pending:
                out.append((i + 1, line.strip(), lines[j].strip()))
                break
    return out


# Inline asm is opaque to the compiler's hazard recognizer, so the wait
# states that the ISA asks for around VALU instructions written in asm are
# checked here in the built code:
#  - an MFMA that reads (as SrcA, SrcB or SrcC) a VGPR written by a VALU
#    instruction needs VALU_TO_MFMA wait states after that write;
#  - an MFMA's result is not ready for MFMA_RESULT_WINDOW wait states and the
#    compiler makes nothing in asm wait for it, so an asm instruction may not
#    read an MFMA destination written that recently.
VALU_TO_MFMA = 2
MFMA_RESULT_WINDOW = 20
_REG = re.compile(r"\b([av])(?:\[(\d+):(\d+)\]|(\d+)\b)")


def _operand_regs(t: str):
    """(mnemonic, [register set of each comma-separated operand])."""
    parts = t.split(None, 1)
    ops = []
    if len(parts) > 1:
        for op in parts[1].split(","):
            regs = set()
            for m in _REG.finditer(op):
                regs |= _regs(m.group(1), m.group(2), m.group(3)) if m.group(2) else {(m.group(1), int(m.group(4)))}
            ops.append(regs)
    return parts[0], ops


def _instructions(text: str):
    """[(text, in_asm)] of the instructions, with inline-asm membership."""
    out, in_asm = [], False
    for line in text.splitlines():
        t = line.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        t = t.split(";")[0].strip()
        if not t or t.startswith(".") or t.endswith(":"):
            continue
        out.append((t, in_asm))
    return out


def _wait_states(t: str) -> int:
    nop = re.match(r"s_nop\s+(\d+)", t)
    return int(nop.group(1)) + 1 if nop else 1


def scan_inline_asm(text: str):
    """Returns [(asm instruction, offending MFMA)] that break either rule above."""
    ins = _instructions(text)
    out = []
    for i, (t, in_asm) in enumerate(ins):
        if not in_asm or not t.startswith("v_") or t.startswith("v_mfma"):
            continue
        _, ops = _operand_regs(t)
        if not ops:
            continue
        written = ops[0]
        read = set().union(*ops[1:]) if len(ops) > 1 else set()
        waits = 0
        for u, _ in ins[i + 1:]:
            if waits >= VALU_TO_MFMA:
                break
            if u.startswith("v_mfma"):
                _, mops = _operand_regs(u)
                if set().union(*mops[1:]) & written:
                    out.append((t, u))
                    break
            waits += _wait_states(u)
        waits = 0
        for u, _ in reversed(ins[:i]):
            if waits >= MFMA_RESULT_WINDOW or not read:
                break
            _, uops = _operand_regs(u)
            if u.startswith("v_mfma") and uops and uops[0] & read:
                out.append((t, u))
                break
            if uops and (u.startswith("v_") or u.startswith("ds_") or "load" in u):
                read = read - uops[0]
            waits += _wait_states(u)
    return out


def loop_lds_waits(text: str, kernel_prefix: str, min_mfma: int = 100, max_mfma: int = 400):
    """The loops of one kernel that issue between min_mfma and max_mfma MFMAs
    per pass (in the CG kernels, each wave's iteration; the persistent loop
    around the chunks issues more): a list of (MFMAs, full LDS waits
    `s_waitcnt lgkmcnt(0)`) per pass, in code order.  A loop is the code from
    a label to a later branch back to it.  The compiler has at times scheduled
    such a loop to wait on each of its LDS reads right after issuing it, which
    shows as several times the usual count of full waits."""
    lines = text.splitlines()
    starts = [i for i, l in enumerate(lines) if l.startswith(kernel_prefix) and ":" in l]
    if not starts:
        raise ValueError(f"no kernel {kernel_prefix} in the assembly")
    st = starts[0]
    en = next((i for i in range(st + 1, len(lines)) if re.match(r"^_Z\w+:", lines[i])), len(lines))
    body = lines[st:en]
    labels = {}
    for i, l in enumerate(body):
        m = re.match(r"^(\.LBB\S+):", l)
        if m:
            labels[m.group(1)] = i
    out = []
    for i, l in enumerate(body):
        m = re.search(r"\bs_cbranch_\w+\s+(\.LBB\S+)", l)
        if not m or m.group(1) not in labels or labels[m.group(1)] >= i:
            continue
        ins = [x.strip() for x in body[labels[m.group(1)]:i + 1]]
        nm = sum(x.startswith("v_mfma") for x in ins)
        if min_mfma <= nm <= max_mfma:
            out.append((nm, sum(x == "s_waitcnt lgkmcnt(0)" for x in ins)))
    return out


def compile_asm(src: str) -> str:
    """gfx950 assembly of one kernel source, built with its own flags."""
    with tempfile.TemporaryDirectory() as td:
        asm = os.path.join(td, src + ".s")
        cmd = [B.HIPCC, *B.flags_for(src), "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", asm]
        subprocess.run(cmd, check=True, capture_output=True)
        return open(asm).read()


def check_all(sources=None):
    """Compile each kernel source to gfx950 assembly; return {source: hazards},
    the SrcC rewrites of scan_asm followed by the inline-asm findings."""
    sources = sources or [s for s in B.SOURCES if s != "mesa_host.hip"]
    res = {}
    with tempfile.TemporaryDirectory() as td:
        for src in sources:
            asm = os.path.join(td, src + ".s")
            cmd = [B.HIPCC, *B.flags_for(src), "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", asm]
            subprocess.run(cmd, check=True, capture_output=True)
            text = open(asm).read()
            res[src] = scan_asm(text) + scan_inline_asm(text)
    return res


if __name__ == "__main__":
    for src, hz in check_all().items():
        print(src, len(hz))
        for h in hz[:10]:
            print("   ", h)
