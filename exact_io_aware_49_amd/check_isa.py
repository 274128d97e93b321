"""Static checks of the gfx950 assembly around inline asm.

1. Inline-asm LDS reads.  Some LDS reads in the kernels are issued through
   inline asm (so the compiler does not wait for unrelated global->LDS
   transfers before them).  The compiler does not know those instructions write
   their destination registers later, so the source code waits for them
   explicitly (s_waitcnt lgkmcnt(0)) before use.  This check makes sure the
   compiler did not read or overwrite such a register in between (for example
   by inserting a register copy):

     * a ds_read_* inside an ;;#ASMSTART / ;;#ASMEND region marks its
       destination VGPRs pending;
     * s_waitcnt with lgkmcnt(0) clears every pending register;
     * any other instruction that names a pending VGPR is a violation.

2. Matrix-core results read by inline asm.  A v_mfma_* writes its destination
   registers several cycles after it issues; the compiler pads a dependent
   instruction with wait states (s_nop) but does not do so for an instruction
   inside inline asm.  An inline-asm instruction that names a register written
   by a v_mfma_* fewer than MFMA_WAIT_STATES wait states earlier (one per
   instruction issued in between, N + 1 for s_nop N) on some path is a
   violation: it can read the register before the result lands.  A
   compiler-generated instruction (other than another v_mfma_*) that names any
   register of the result shows that the compiler has waited for it, which
   clears the whole result.  The destination of an inline-asm load (ds_read_*,
   buffer_load_*, global_load_*) is not counted: the loaded value lands no
   sooner than the LDS latency, long after any matrix-core result.

Both scans follow the control-flow graph of each function (blocks split at
labels and branches) and take the worst case over the paths into a block.

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


# wait states between a v_mfma_* and an instruction that touches its result: the
# largest gfx950 requirement (16-pass XDL operations: 18, plus one of margin)
MFMA_WAIT_STATES = 19
ANYREG_RE = re.compile(r"\b([va])\[(\d+):(\d+)\]|\b([va])(\d+)\b")


def anyregs_of(operands: str):
    """VGPRs and AGPRs named in operands, as ('v', n) / ('a', n)."""
    out = set()
    for m in ANYREG_RE.finditer(operands):
        if m.group(1) is not None:
            out.update((m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1))
        else:
            out.add((m.group(4), int(m.group(5))))
    return out


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


def _cfg(f):
    """Basic blocks (start, end) of a function and their successor lists."""
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
    return blocks, succs


def _solve(blocks, succs, transfer, merge):
    """Forward data flow to a fixed point; merge(old, new) returns (state, changed)."""
    state_in = [dict() for _ in blocks]
    work = list(range(len(blocks)))
    while work:
        bi = work.pop(0)
        out = transfer(bi, state_in[bi])
        for sj in succs[bi]:
            merged, changed = merge(state_in[sj], out)
            if changed:
                state_in[sj] = merged
                if sj not in work:
                    work.append(sj)


def _merge_union(old, new):
    merged = dict(old)
    changed = False
    for r, v in new.items():
        if r not in merged:
            merged[r] = v
            changed = True
    return merged, changed


def _merge_max(old, new):
    """States map register -> (wait states owed, id of the v_mfma); keep the larger debt."""
    merged = dict(old)
    changed = False
    for r, v in new.items():
        if v[0] > merged.get(r, (0, None))[0]:
            merged[r] = v
            changed = True
    return merged, changed


def _check_function(f, name):
    """Inline-asm LDS reads: a register written by an inline-asm ds_read is
    pending until an s_waitcnt lgkmcnt(0) on every path; any other instruction
    naming a pending register is a violation."""
    insts = f["insts"]
    blocks, succs = _cfg(f)
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

    _solve(blocks, succs, transfer, _merge_union)
    return [violations[k] for k in sorted(violations)]


def _wait_states(op: str, operands: str) -> int:
    if op == "s_nop":
        try:
            return int(operands.split()[0], 0) + 1
        except (ValueError, IndexError):
            return 1
    return 1


def _check_mfma_hazards(f, name):
    """Matrix-core results read by inline asm: state = registers written by a
    v_mfma_* with the wait states still owed (worst case over paths)."""
    insts = f["insts"]
    blocks, succs = _cfg(f)
    violations = {}

    def transfer(bi, owed):
        owed = dict(owed)
        b, e = blocks[bi]
        for ln, op, operands, in_asm in insts[b:e]:
            if owed:
                named = operands
                if in_asm and re.match(r"^(ds_read|buffer_load|global_load)", op):
                    named = operands.split(",", 1)[1] if "," in operands else ""
                hit = anyregs_of(named) & set(owed)
                if hit and in_asm:
                    r = min(hit)
                    violations[ln] = (f"{name}:{ln}: {f['name']}: inline asm '{op} {operands}' touches "
                                      f"{r[0]}{r[1]} with {owed[r][0]} of {MFMA_WAIT_STATES} wait states after "
                                      f"the v_mfma at line {owed[r][1]} that writes it still to go")
                elif hit and not op.startswith("v_mfma"):
                    done = {owed[r][1] for r in hit}
                    owed = {r: v for r, v in owed.items() if v[1] not in done}
            ws = _wait_states(op, operands)
            owed = {r: (v[0] - ws, v[1]) for r, v in owed.items() if v[0] - ws > 0}
            if op.startswith("v_mfma"):
                dst = operands.split(",", 1)[0]
                for r in anyregs_of(dst):
                    owed[r] = (MFMA_WAIT_STATES, ln)
        return owed

    _solve(blocks, succs, transfer, _merge_max)
    return [violations[k] for k in sorted(violations)]


def check_text(text: str, name: str = "<asm>"):
    """Return a list of violation strings for one assembly file."""
    violations = []
    for f in _functions(text):
        violations += _check_function(f, name)
        violations += _check_mfma_hazards(f, name)
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
