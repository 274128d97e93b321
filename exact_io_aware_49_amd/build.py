"""Build libfa.so for gfx950 with hipcc (in-tree, next to this file).

    python -m exact_io_aware_49_amd.build [--jobs N] [--debug]

Each translation unit under csrc/ is compiled separately (in parallel), then
linked into exact_io_aware_49_amd/libfa.so.  Only the C ABI of include/fa.h is
exported (everything else is built with hidden visibility).
"""

from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfa.so")
ARCH = "gfx950"

SOURCES = ["fa_api.cpp", "fa_fwd_bf16.hip", "fa_fwd_bf16_r64.hip", "fa_fwd_f32.hip", "fa_bwd_bf16.hip", "fa_decode.hip", "fa_fwd_fp8.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def common_flags(debug: bool):
    flags = [
        f"--offload-arch={ARCH}",
        "-std=c++17",
        "-fPIC",
        "-fvisibility=hidden",
        "-I", INCLUDE,
        "-I", CSRC,
        # packed fp32 VALU forms are kept out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
    ]
    flags += ["-O1", "-g"] if debug else ["-O3"]
    return flags


# Per-source code-generation flags.  The decode kernel and the 64-row forward
# run one wave per SIMD, where the compiler otherwise keeps matrix results in
# AGPRs and copies them to VGPRs for the vector code on every key tile; the
# VGPR form of the MFMA instructions removes those copies (same results; decode
# 2-8% faster, the 64-row forward 1%).
SOURCE_FLAGS = {
    "fa_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "fa_fwd_bf16_r64.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def source_flags(src: str):
    return list(SOURCE_FLAGS.get(os.path.basename(src), []))


def compile_one(src: str, debug: bool) -> str:
    os.makedirs(BUILD, exist_ok=True)
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + common_flags(debug) + source_flags(src) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 4, debug: bool = False, verbose: bool = True, check: bool = True) -> str:
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: compile_one(s, debug), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if check:
        from .check_isa import check_sources
        bad = check_sources()
        if bad:
            os.remove(LIB)
            raise RuntimeError("inline-asm LDS register hazards in the generated code:\n" + "\n".join(bad))
    if verbose:
        print(f"built {LIB}")
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--debug", action="store_true")
    a = ap.parse_args(argv)
    build(a.jobs, a.debug)


if __name__ == "__main__":
    sys.exit(main())
