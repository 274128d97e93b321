"""Helpers shared by the GPU parity tests: device upload and the tolerance gates.

Tolerances: float32 paths, max |gpu - ref| <= 1e-5; bf16 paths, per output
tensor, max |gpu - ref| <= 2e-2 AND ||gpu - ref||_2 / ||ref||_2 <= 1e-2,
against the float64 oracle evaluated on the exact (bf16-rounded) inputs.
"""

import sys

import numpy as np
import pytest
import torch

TOL_F32_ABS = 1e-5
TOL_BF16_ABS = 2e-2
TOL_BF16_REL = 1e-2


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray, dtype: str):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to("cuda").to(torch.bfloat16 if dtype == "bf16" else torch.float32).contiguous()


def host(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def f32(x: float) -> float:
    """The float32 value the kernel receives for a Python float argument."""
    return float(np.float32(x))


def errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    diff = np.abs(got - ref)
    mx = float(diff.max()) if diff.size else 0.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref)) / den if den > 0 else float(np.linalg.norm(got - ref))
    return mx, rel


# Every bf16 tensor gated here is also checked with allclose(atol=2e-2, rtol=1e-2)
# (elementwise |gpu - ref| <= 2e-2 + 1e-2 |ref|).  That is reported, not gated: the
# test session prints the count and names (tests/conftest.py).
ALLCLOSE = {"pass": 0, "fail": []}


def assert_close(name, got, ref, dtype, lse=False, magnitude_scaled=False):
    """Gate one output tensor.  `magnitude_scaled` (stress inputs only, never the
    named workloads) multiplies the absolute bound by max(1, max|ref|), because a
    bf16 output of magnitude M cannot be closer than M * 2^-9 to the exact value."""
    mx, rel = errors(got, ref)
    if not np.all(np.isfinite(got)):
        raise AssertionError(f"{name}: non-finite values")
    if dtype != "f32":
        if np.allclose(np.asarray(got, np.float64), np.asarray(ref, np.float64), atol=TOL_BF16_ABS, rtol=TOL_BF16_REL):
            ALLCLOSE["pass"] += 1
        else:
            ALLCLOSE["fail"].append(name)
    if dtype == "f32":
        assert mx <= TOL_F32_ABS, f"{name}: max abs err {mx:.3e} > {TOL_F32_ABS}"
    else:
        tol = TOL_BF16_ABS * (max(1.0, float(np.abs(ref).max())) if magnitude_scaled else 1.0)
        assert mx <= tol, f"{name}: max abs err {mx:.3e} > {tol:.3e}"
        if not lse:
            assert rel <= TOL_BF16_REL, f"{name}: rel L2 err {rel:.3e} > {TOL_BF16_REL}"
    return mx, rel
