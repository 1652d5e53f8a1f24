"""Scan gfx950 assembly of libmesa's kernels for an MFMA accumulator hazard.

A multi-pass v_mfma reads its accumulator input (SrcC) over several passes.
When the compiler gives an MFMA a SrcC register range different from its
destination, a later instruction may overwrite those SrcC registers before
the MFMA has read them; the observed result is a corrupted accumulator
component (seen on gfx950 with a 16x16x4 f32 MFMA whose SrcC came from the
MFMA issued just before it, the SrcC registers being rewritten 9 wait states
later).  This check compiles every kernel source to assembly and reports each
MFMA with SrcC != Dst whose SrcC registers are written again before
MIN_WAIT_STATES wait states have passed (one per instruction, N+1 per
s_nop N) -- about twice the gap that was observed to fail.
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
_WRITE = re.compile(r"^\s*(v_\S+|ds_read\S*|global_load\S*|buffer_load\S*)\s+([av])(?:\[(\d+):(\d+)\]|(\d+))\b")


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
            if not w:
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


def check_all(sources=None):
    """Compile each kernel source to gfx950 assembly; return {source: hazards}."""
    sources = sources or [s for s in B.SOURCES if s != "mesa_host.hip"]
    res = {}
    with tempfile.TemporaryDirectory() as td:
        for src in sources:
            asm = os.path.join(td, src + ".s")
            cmd = [B.HIPCC, *B.flags_for(src), "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", asm]
            subprocess.run(cmd, check=True, capture_output=True)
            res[src] = scan_asm(open(asm).read())
    return res


if __name__ == "__main__":
    for src, hz in check_all().items():
        print(src, len(hz))
        for h in hz[:10]:
            print("   ", h)
