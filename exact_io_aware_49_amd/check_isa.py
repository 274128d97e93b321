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

The scan follows the control-flow graph of each function (blocks split at labels
and branches): a register is pending at the start of a block if it is pending at
the end of any predecessor, so a wait on every path is required.

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


BRANCH_RE = re.compile(r"^s_(c?branch\w*|setpc_b64|endpgm\w*)$")


def _functions(text: str):
    """Split assembly text into functions: lists of (line, op, operands, in_asm) and labels."""
    funcs = []
    cur = None
    in_asm = False
    for ln, raw in enumerate(text.splitlines(), 1):
        stripped = raw.strip()
        if stripped.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if stripped.startswith(";;#ASMEND"):
            in_asm = False
            continue
        line = raw.split(";", 1)[0].rstrip()
        if not line.strip():
            continue
        if re.match(r"^[A-Za-z_.$][\w.$]*:", line):
            lab = line.split(":")[0]
            if not lab.startswith(".L"):
                cur = {"name": lab, "insts": [], "labels": {}}
                funcs.append(cur)
            elif cur is not None:
                cur["labels"][lab] = len(cur["insts"])
            continue
        if cur is None:
            continue
        parts = line.strip().split(None, 1)
        op = parts[0]
        if op.startswith("."):
            continue
        cur["insts"].append((ln, op, parts[1] if len(parts) > 1 else "", in_asm))
    return funcs


def _check_function(f, name):
    """Data flow over the function's control-flow graph: a register read by an
    inline-asm ds_read is pending until an s_waitcnt lgkmcnt(0) on every path;
    any other instruction naming a pending register is a violation."""
    insts, labels = f["insts"], f["labels"]
    n = len(insts)
    starts = sorted(set([0] + list(labels.values()) +
                        [i + 1 for i, (_, op, _, _) in enumerate(insts) if BRANCH_RE.match(op)]))
    starts = [b for b in starts if b < n]
    block_of = {}
    blocks = []
    for bi, b in enumerate(starts):
        e = starts[bi + 1] if bi + 1 < len(starts) else n
        blocks.append((b, e))
        block_of[b] = bi
    succs = []
    for bi, (b, e) in enumerate(blocks):
        ln, op, operands, _ = insts[e - 1]
        nxt = [bi + 1] if bi + 1 < len(blocks) else []
        if op == "s_branch" or op.startswith("s_setpc") or op.startswith("s_endpgm"):
            tgt = []
            if op == "s_branch":
                lab = operands.split()[0]
                if lab in labels and labels[lab] in block_of:
                    tgt = [block_of[labels[lab]]]
            succs.append(tgt)
        elif op.startswith("s_cbranch"):
            lab = operands.split()[0]
            tgt = [block_of[labels[lab]]] if lab in labels and labels[lab] in block_of else []
            succs.append(tgt + nxt)
        else:
            succs.append(nxt)
    pend_in = [dict() for _ in blocks]
    violations = {}

    def transfer(bi, pend):
        pend = dict(pend)
        b, e = blocks[bi]
        for ln, op, operands, in_asm in insts[b:e]:
            if op == "s_waitcnt":
                if re.search(r"lgkmcnt\(0\)", operands):
                    pend.clear()
                continue
            if in_asm and op.startswith("ds_read"):
                for r in regs_of(operands.split(",", 1)[0]):
                    pend[r] = ln
                continue
            if in_asm:
                continue
            touched = regs_of(operands) & set(pend)
            if touched:
                violations[ln] = (f"{name}:{ln}: {f['name']}: '{op} {operands}' uses v{sorted(touched)} "
                                  f"loaded by the inline-asm LDS read at line {pend[min(touched)]} "
                                  f"before lgkmcnt(0)")
        return pend

    work = list(range(len(blocks)))
    while work:
        bi = work.pop(0)
        out = transfer(bi, pend_in[bi])
        for sj in succs[bi]:
            merged = dict(pend_in[sj])
            changed = False
            for r, l in out.items():
                if r not in merged:
                    merged[r] = l
                    changed = True
            if changed:
                pend_in[sj] = merged
                if sj not in work:
                    work.append(sj)
    return [violations[k] for k in sorted(violations)]


def check_text(text: str, name: str = "<asm>"):
    """Return a list of violation strings for one assembly file."""
    violations = []
    for f in _functions(text):
        violations += _check_function(f, name)
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
