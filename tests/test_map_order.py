"""Host check of the workgroup orders of fa_map.h (the real header, compiled for the host by hipcc):
one workgroup per (head, row block), heads kept on one XCD, heaviest causal blocks first, and the
snake order for resident grids (tests/map_check.cpp states the properties)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_io_aware_49_amd", "csrc")


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


def test_block_orders_are_one_to_one_and_heaviest_first(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "map_check")
    subprocess.run([hipcc, "-std=c++17", "-O1", "-I", CSRC, os.path.join(ROOT, "tests", "map_check.cpp"), "-o", exe],
                   check=True, capture_output=True, timeout=300)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-2000:]
    assert r.stdout.strip().startswith("ok"), r.stdout
