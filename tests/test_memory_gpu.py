"""Attention memory stays linear in N (German page "FlashAttention (DE)", section
"Komplexität und Optimalität": O(N) instead of O(N^2); Dutch page, section
"Voorbeeld": standard attention's table grows 4x per doubling, FlashAttention's
memory linearly).

For B=1, H=32, d=128 (bf16, causal) and N = 2K..32K the test checks that a
forward call allocates nothing beyond the caller's tensors (Q, K, V, O, lse =
32,896 * N bytes) and that a backward call needs exactly fa_bwd_workspace_size
= 2 * 32 * N * 4 bytes on top of its own tensors.  Device free memory is read with
hipMemGetInfo (torch.cuda.mem_get_info) around the calls.  An N x N bf16 score
table for the same heads would be 64 * N^2 bytes (64 GiB at N = 32768).
"""

import numpy as np
import pytest
import torch

import exact_io_aware_49_amd as fa
from gpu_common import need_gpu, say

pytestmark = pytest.mark.gpu


def test_memory_is_linear_in_n():
    need_gpu()
    H, d = 32, 128
    rows = []
    for N in (2048, 4096, 8192, 16384, 32768):
        say(f"[memory] N={N}")
        g = torch.Generator(device="cuda").manual_seed(N)
        q, k, v, do = (torch.randn((1, H, N, d), device="cuda", generator=g).to(torch.bfloat16) for _ in range(4))
        o = torch.empty_like(q)
        lse = torch.empty((1, H, N), dtype=torch.float32, device="cuda")
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        need = fa.fa_bwd_workspace_size(1, H, N, d, fa.FA_DTYPE_BF16)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        sh = torch.cuda.current_stream().cuda_stream
        args_f = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), 1, H, N, d, 1,
                  d ** -0.5, fa.FA_DTYPE_BF16, sh)
        args_b = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                  dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), need, 1, H, N, d, 1, d ** -0.5,
                  fa.FA_DTYPE_BF16, sh)
        assert fa.fa_fwd(*args_f) == 0 and fa.fa_bwd(*args_b) == 0  # warm-up (code objects load)
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        base_alloc = torch.cuda.memory_allocated()
        free0, _ = torch.cuda.mem_get_info()
        assert fa.fa_fwd(*args_f) == 0
        torch.cuda.synchronize()
        free1, _ = torch.cuda.mem_get_info()
        assert fa.fa_bwd(*args_b) == 0
        torch.cuda.synchronize()
        free2, _ = torch.cuda.mem_get_info()
        assert torch.cuda.max_memory_allocated() == base_alloc
        assert free0 - free1 == 0, f"forward changed free device memory by {free0 - free1} bytes"
        assert free1 - free2 == 0, f"backward changed free device memory by {free1 - free2} bytes"
        assert need == 2 * 32 * N * 4
        fwd_bytes = sum(t.numel() * t.element_size() for t in (q, k, v, o, lse))
        assert fwd_bytes == 32896 * N
        rows.append((N, fwd_bytes, fwd_bytes + 4 * q.numel() * 2 + need, 64 * N * N))
        del q, k, v, do, o, lse, dq, dk, dv, ws
        torch.cuda.empty_cache()
    ns = np.array([r[0] for r in rows], dtype=np.float64)
    fwd = np.array([r[1] for r in rows], dtype=np.float64)
    slope, icpt = np.polyfit(ns, fwd, 1)
    assert abs(icpt) < 1e-3 * fwd[0] and np.allclose(fwd, slope * ns, rtol=1e-12)
    for N, fb, tb, naive in rows:
        say(f"   N={N:6d}  forward tensors {fb / 2**20:8.1f} MiB  fwd+bwd {tb / 2**20:8.1f} MiB  "
            f"naive bf16 score table {naive / 2**30:6.1f} GiB")
