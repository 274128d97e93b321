"""Static check of the gfx950 assembly for inline-asm LDS reads.

Some LDS reads in the kernels are issued through inline asm (so the compiler
does not wait for unrelated global->LDS transfers before them).  The compiler
does not know those instructions write their destination registers later, so
the source code waits for them explicitly (s_waitcnt lgkmcnt(0)) before use.
This check makes sure the compiler did not read or overwrite such a register
in between (for example by inserting a register copy):

  * a ds_read_* inside an ;;#ASMSTART / ;;#ASMEND region marks its destination
    VGPRs pending;
  * s_waitcnt with lgkmcnt(0) clears every pending register;
  * any other instruction that names a pending VGPR is a violation.

The scan follows program order through the text, which is conservative across
branches (a register stays pending until a later lgkmcnt(0) in the text).

    python -m exact_io_aware_49_amd.check_isa [file.s ...]
With no arguments the kernel sources are compiled to assembly first.
"""

from __future__ import annotations

import os
import re
import subprocess
import sys
import tempfile

from . import build as B

REG_RE = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")


def regs_of(operands: str):
    out = set()
    for m in REG_RE.finditer(operands):
        if m.group(1) is not None:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
        else:
            out.add(int(m.group(3)))
    return out


def check_text(text: str, name: str = "<asm>"):
    """Return a list of violation strings for one assembly file."""
    violations = []
    pending = {}  # vgpr -> line number of the asm read
    in_asm = False
    func = None
    for ln, raw in enumerate(text.splitlines(), 1):
        line = raw.split(";", 1)[0].rstrip() if not raw.lstrip().startswith(";;#ASM") else raw.strip()
        if raw.strip().startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if raw.strip().startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not line.strip():
            continue
        if re.match(r"^[A-Za-z_.$][\w.$]*:", line):
            lab = line.split(":")[0]
            if not lab.startswith(".L"):
                func = lab
                pending.clear()
            continue
        parts = line.strip().split(None, 1)
        op = parts[0]
        operands = parts[1] if len(parts) > 1 else ""
        if op.startswith("."):
            continue
        if op == "s_waitcnt":
            if re.search(r"lgkmcnt\(0\)", operands):
                pending.clear()
            continue
        if in_asm and op.startswith("ds_read"):
            dst = operands.split(",", 1)[0]
            for r in regs_of(dst):
                pending[r] = ln
            continue
        if in_asm:
            continue
        touched = regs_of(operands) & set(pending)
        if touched:
            violations.append(f"{name}:{ln}: {func}: '{line.strip()}' uses v{sorted(touched)} "
                              f"loaded by the inline-asm LDS read at line {pending[min(touched)]} "
                              f"before lgkmcnt(0)")
    return violations


def device_asm(src: str, outdir: str) -> str:
    """Compile one source to gfx950 assembly; return its path."""
    out = os.path.join(outdir, os.path.splitext(os.path.basename(src))[0] + ".s")
    cmd = [B.hipcc()] + B.common_flags(False) + B.source_flags(src) + ["--offload-device-only", "-S", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"assembly generation failed: {' '.join(cmd)}\n{r.stderr}")
    return out


def check_sources():
    violations = []
    with tempfile.TemporaryDirectory() as td:
        for src in B.SOURCES:
            if not src.endswith(".hip"):
                continue
            path = device_asm(os.path.join(B.CSRC, src), td)
            with open(path) as f:
                violations += check_text(f.read(), src)
    return violations


def main(argv=None):
    argv = sys.argv[1:] if argv is None else argv
    if argv:
        v = []
        for p in argv:
            with open(p) as f:
                v += check_text(f.read(), p)
    else:
        v = check_sources()
    for x in v:
        print(x)
    print(f"{len(v)} violation(s)")
    return 1 if v else 0


if __name__ == "__main__":
    sys.exit(main())
