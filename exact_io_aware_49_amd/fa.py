"""Thin ctypes binding of libfa.so (include/fa.h).

The functions `fa_fwd`, `fa_bwd`, `fa_bwd_workspace_size`, their shared-K/V-head
forms `fa_fwd_gqa`, `fa_bwd_gqa`, `fa_bwd_gqa_workspace_size`, and
`fa_status_string` and `fa_version` mirror the C ABI one to one: they take raw device pointers
(ints), sizes and a stream handle, and return the status code.  `forward` and
`backward` are the torch-facing conveniences: they check devices, dtypes and
shapes, allocate outputs (and the backward workspace) with torch on the
tensors' device, pass pointers and torch's current stream, and raise
RuntimeError on any non-zero status.  All attention arithmetic happens in the
HIP kernels; if libfa.so is missing or cannot load, every call raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_DTYPE_F32 = 0
FA_DTYPE_BF16 = 1

STATUS_NAMES = {
    0: "FA_OK",
    1: "FA_ERR_NULL_POINTER",
    2: "FA_ERR_BAD_SHAPE",
    3: "FA_ERR_UNSUPPORTED_HEAD_DIM",
    4: "FA_ERR_UNSUPPORTED_DTYPE",
    5: "FA_ERR_BAD_SCALE",
    6: "FA_ERR_MISALIGNED",
    7: "FA_ERR_WORKSPACE_TOO_SMALL",
    8: "FA_ERR_HIP",
    9: "FA_ERR_BAD_ARGUMENT",
    10: "FA_ERR_SCRATCH_TOO_SMALL",
}

_lib = None


def load_library(path: str = LIB_PATH):
    """Load libfa.so once; raise RuntimeError if it is missing or broken."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"libfa.so not found at {path}; build it with `python -m exact_io_aware_49_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.fa_fwd.restype = i
    lib.fa_bwd_workspace_size.argtypes = [i, i, i, i, i]
    lib.fa_bwd_workspace_size.restype = sz
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, f, i, vp]
    lib.fa_bwd.restype = i
    lib.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.fa_bwd_noalloc.restype = i
    lib.fa_bwd_noalloc_scratch_bytes.argtypes = []
    lib.fa_bwd_noalloc_scratch_bytes.restype = sz
    lib.fa_fwd_gqa.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
    lib.fa_fwd_gqa.restype = i
    lib.fa_bwd_gqa_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.fa_bwd_gqa_workspace_size.restype = sz
    lib.fa_bwd_gqa.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, f, i, vp]
    lib.fa_bwd_gqa.restype = i
    lib.fa_decode_workspace_size.argtypes = [i, i, i, i, i, i, i]
    lib.fa_decode_workspace_size.restype = sz
    lib.fa_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, i, f, i, vp]
    lib.fa_decode.restype = i
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, f, f, f, vp, vp, i, i, i, i, i, i, f, vp]
    lib.fa_fwd_fp8.restype = i
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_version.argtypes = []
    lib.fa_version.restype = i
    _lib = lib
    return lib


# ----------------------------------------------------------------- raw C ABI mirror

def fa_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, dtype, stream) -> int:
    return load_library().fa_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, dtype, stream)


def fa_bwd_workspace_size(B, H, N, d, dtype) -> int:
    return load_library().fa_bwd_workspace_size(B, H, N, d, dtype)


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, N, d, causal, scale, dtype,
           stream) -> int:
    return load_library().fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, N, d,
                                 causal, scale, dtype, stream)


def fa_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, causal, scale, dtype, stream) -> int:
    return load_library().fa_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, causal, scale, dtype,
                                         stream)


def fa_bwd_noalloc_scratch_bytes() -> int:
    return load_library().fa_bwd_noalloc_scratch_bytes()


def fa_fwd_gqa(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, dtype, stream) -> int:
    return load_library().fa_fwd_gqa(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, dtype, stream)


def fa_bwd_gqa_workspace_size(B, Hq, Hkv, N, d, dtype) -> int:
    return load_library().fa_bwd_gqa_workspace_size(B, Hq, Hkv, N, d, dtype)


def fa_bwd_gqa(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv, N, d, causal, scale,
               dtype, stream) -> int:
    return load_library().fa_bwd_gqa(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv,
                                     N, d, causal, scale, dtype, stream)


def fa_decode_workspace_size(B, Hq, Hkv, Nq, Nk, d, dtype) -> int:
    return load_library().fa_decode_workspace_size(B, Hq, Hkv, Nq, Nk, d, dtype)


def fa_decode(q, k, v, kv_lens, o, lse, workspace, workspace_bytes, B, Hq, Hkv, Nq, Nk, d, causal, scale, dtype,
              stream) -> int:
    return load_library().fa_decode(q, k, v, kv_lens, o, lse, workspace, workspace_bytes, B, Hq, Hkv, Nq, Nk, d,
                                    causal, scale, dtype, stream)


def fa_fwd_fp8(q, k, v, q_scale, k_scale, v_scale, o, lse, B, Hq, Hkv, N, d, causal, scale, stream) -> int:
    return load_library().fa_fwd_fp8(q, k, v, q_scale, k_scale, v_scale, o, lse, B, Hq, Hkv, N, d, causal, scale,
                                     stream)


def fa_status_string(status: int) -> str:
    return load_library().fa_status_string(status).decode()


def fa_version() -> int:
    return load_library().fa_version()


# ----------------------------------------------------------------- torch conveniences

_DTYPES = {torch.float32: FA_DTYPE_F32, torch.bfloat16: FA_DTYPE_BF16}


def _check(status: int):
    if status != 0:
        raise RuntimeError(fa_status_string(status))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise RuntimeError(f"unsupported dtype {t.dtype}; use torch.float32 or torch.bfloat16")
    return _DTYPES[t.dtype]


def _check_tensors(*ts):
    ref = ts[0]
    if not ref.is_cuda:
        raise RuntimeError("tensors must be on a GPU device")
    for t in ts:
        if t.device != ref.device:
            raise RuntimeError("all tensors must be on the same device")
        if not t.is_contiguous():
            raise RuntimeError("tensors must be contiguous [B, H, N, d]")


def _stream_handle(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def default_scale(d: int) -> float:
    """1/sqrt(d), the scale of the attention equation."""
    return float(d) ** -0.5


def _kv_heads(q, k, v):
    """Number of K/V heads: k and v are [B, Hkv, N, d] with Hkv dividing q's head count."""
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise RuntimeError("q [B, Hq, N, d] and k, v [B, Hkv, N, d] must share dtype")
    B, H, N, d = q.shape
    hkv = k.shape[1]
    if (k.shape[0], k.shape[2], k.shape[3]) != (B, N, d) or hkv < 1 or H % hkv != 0:
        raise RuntimeError("k, v must be [B, Hkv, N, d] with Hkv dividing the query head count")
    return hkv


def forward(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None):
    """Exact attention forward on the GPU.  q: [B, Hq, N, d], k, v: [B, Hkv, N, d] (bf16 or fp32),
    Hkv dividing Hq (query head h uses K/V head h // (Hq / Hkv); Hkv = Hq is plain multi-head).

    Returns (o, lse): o like q, lse float32 [B, Hq, N].
    """
    load_library()
    _check_tensors(q, k, v)
    hkv = _kv_heads(q, k, v)
    B, H, N, d = q.shape
    scale = default_scale(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else out
    lse_t = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_tensors(q, o, lse_t)
    if o.shape != q.shape or o.dtype != q.dtype or lse_t.shape != (B, H, N) or lse_t.dtype != torch.float32:
        raise RuntimeError("out / lse have the wrong shape or dtype")
    _check(fa_fwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse_t.data_ptr(), B, H, hkv, N,
                      d, int(bool(causal)), scale, _dtype_code(q), _stream_handle(q.device)))
    return o, lse_t


def backward(q, k, v, o, do, lse, causal: bool = False, scale: float | None = None, workspace=None):
    """Exact attention backward with recomputation.  Returns (dq like q, dk and dv like k)."""
    load_library()
    _check_tensors(q, k, v, o, do, lse)
    hkv = _kv_heads(q, k, v)
    for t in (o, do):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise RuntimeError("o and do must match q [B, Hq, N, d]")
    B, H, N, d = q.shape
    if lse.shape != (B, H, N) or lse.dtype != torch.float32:
        raise RuntimeError("lse must be float32 [B, H, N]")
    scale = default_scale(d) if scale is None else float(scale)
    code = _dtype_code(q)
    need = fa_bwd_gqa_workspace_size(B, H, hkv, N, d, code)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    _check(fa_bwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                      dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(), workspace.numel(),
                      B, H, hkv, N, d, int(bool(causal)), scale, code, _stream_handle(q.device)))
    return dq, dk, dv


def decode(q, k, v, kv_lens=None, causal: bool = False, scale: float | None = None, workspace=None):
    """Attention of Nq new query rows against a key/value cache (bf16).

    q: [B, Hq, Nq, d]; k, v: [B, Hkv, Nk, d] (cache capacity Nk, Hkv dividing Hq);
    kv_lens: int32 [B] device tensor of valid cache rows per sequence, or None (all Nk).
    Query i of sequence b sits at position kv_lens[b] - Nq + i.  Returns (o like q,
    lse float32 [B, Hq, Nq]).
    """
    load_library()
    _check_tensors(q, k, v)
    if q.dtype != torch.bfloat16 or k.dtype != q.dtype or v.dtype != q.dtype:
        raise RuntimeError("decode takes bfloat16 q, k, v")
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or k.shape[0] != q.shape[0] or k.shape[3] != q.shape[3]:
        raise RuntimeError("q must be [B, Hq, Nq, d] and k, v [B, Hkv, Nk, d]")
    B, H, nq, d = q.shape
    hkv, nk = k.shape[1], k.shape[2]
    lens_ptr = 0
    if kv_lens is not None:
        _check_tensors(q, kv_lens)
        if kv_lens.dtype != torch.int32 or kv_lens.shape != (B,):
            raise RuntimeError("kv_lens must be an int32 tensor of shape [B]")
        lens_ptr = kv_lens.data_ptr()
    scale = default_scale(d) if scale is None else float(scale)
    need = fa_decode_workspace_size(B, H, hkv, nq, nk, d, FA_DTYPE_BF16)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, nq), dtype=torch.float32, device=q.device)
    _check(fa_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), lens_ptr or None, o.data_ptr(), lse.data_ptr(),
                     workspace.data_ptr(), workspace.numel(), B, H, hkv, nq, nk, d, int(bool(causal)), scale,
                     FA_DTYPE_BF16, _stream_handle(q.device)))
    return o, lse


def forward_fp8(q, k, v, q_scale: float, k_scale: float, v_scale: float, causal: bool = False,
                scale: float | None = None):
    """Exact attention forward on FP8 (E4M3) inputs.

    q: [B, Hq, N, d], k, v: [B, Hkv, N, d] uint8 tensors of E4M3 codes (or torch.float8_e4m3fn,
    viewed as bytes); the value of a code is e4m3(code) * its tensor's scale.  Returns (o bf16
    [B, Hq, N, d], lse float32 [B, Hq, N]).
    """
    load_library()
    q, k, v = (t.view(torch.uint8) if t.dtype != torch.uint8 else t for t in (q, k, v))
    _check_tensors(q, k, v)
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise RuntimeError("q must be [B, Hq, N, d] and k, v [B, Hkv, N, d]")
    B, H, N, d = q.shape
    hkv = k.shape[1]
    if (k.shape[0], k.shape[2], k.shape[3]) != (B, N, d) or hkv < 1 or H % hkv != 0:
        raise RuntimeError("k, v must be [B, Hkv, N, d] with Hkv dividing the query head count")
    scale = default_scale(d) if scale is None else float(scale)
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check(fa_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), float(q_scale), float(k_scale), float(v_scale),
                      o.data_ptr(), lse.data_ptr(), B, H, hkv, N, d, int(bool(causal)), scale,
                      _stream_handle(q.device)))
    return o, lse
