"""Seeded synthetic inputs and the workload table.

This module is shared by the GPU path's tests/benchmark and by the oracle's
tests.  It holds no attention arithmetic: it only draws numbers and rounds
float32 values to bfloat16 (round to nearest, ties to even), the storage
format the bf16 workloads hand to the kernels.

Inputs are i.i.d. N(0, 1), drawn with numpy's PCG64 generator in the order
Q, K, V, dO, each as a C-ordered [B, H, N, d] float32 array.  The pages'
benchmarks ran on models and datasets (GPT-2, BERT-large, Long-Range Arena)
that are not reproduced here; the workloads below borrow only their shapes:
GPT-2-small self-attention (12 heads of 64, sequence 1K), a long-sequence
encoder in the 1K-4K range, and a 32K-token long context.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str          # "fwd" or "bwd"
    B: int
    H: int
    N: int
    d: int
    causal: bool
    dtype: str         # "f32" or "bf16"
    scale: float
    seed: int
    note: str

    @property
    def shape(self):
        return (self.B, self.H, self.N, self.d)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("fwd_f32_b1h2n128d64", "fwd", 1, 2, 128, 64, False, "f32", 1.0 / math.sqrt(64), 1,
                 "small fp32 forward, non-causal"),
        Workload("fwd_gpt2_causal_b8h12n1024d64", "fwd", 8, 12, 1024, 64, True, "bf16",
                 1.0 / math.sqrt(64), 2, "GPT-2-small-shaped causal self-attention"),
        Workload("fwd_encoder_b4h16n4096d128", "fwd", 4, 16, 4096, 128, False, "bf16",
                 1.0 / math.sqrt(128), 3, "long-sequence encoder, non-causal"),
        Workload("fwd_longctx_causal_b1h32n32768d128", "fwd", 1, 32, 32768, 128, True, "bf16",
                 1.0 / math.sqrt(128), 4, "32K-token causal long context"),
        Workload("bwd_causal_b4h16n2048d64", "bwd", 4, 16, 2048, 64, True, "bf16",
                 1.0 / math.sqrt(64), 5, "causal backward with recomputation"),
    ]
}


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); return float32.

    NaN stays NaN (quiet), +-Inf stays +-Inf, finite values beyond the bf16
    range round to +-Inf as round-to-nearest-even prescribes.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    r = r.astype(np.uint32)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = (x.view(np.uint32)[nan] | np.uint32(0x00400000)) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(x_bf16_valued: np.ndarray) -> np.ndarray:
    """The uint16 storage of float32 values that are already bf16-representable."""
    u = np.ascontiguousarray(x_bf16_valued, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """float32 -> OCP E4M3 codes (uint8), round to nearest even, saturating at +-448.

    Used only to make FP8 test inputs: a value is first rounded to the E4M3 grid
    (3 mantissa bits for normals, steps of 2^-9 below 2^-6) and then encoded.
    """
    x = np.asarray(x, dtype=np.float64)
    sign = (np.signbit(x)).astype(np.uint8) << 7
    a = np.minimum(np.abs(x), 448.0)
    # exponent of the grid step: normals have step 2^(e-3), subnormals 2^-9
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    step = np.exp2(e - 3.0)
    q = np.round(a / step) * step            # numpy rounds halves to even
    q = np.minimum(q, 448.0)
    e2 = np.floor(np.log2(np.maximum(q, 2.0 ** -6)))
    normal = q >= 2.0 ** -6
    mant = np.where(normal, np.round((q / np.exp2(e2) - 1.0) * 8.0), np.round(q / 2.0 ** -9))
    exp_field = np.where(normal, e2 + 7.0, 0.0)
    code = (exp_field.astype(np.int64) << 3) | mant.astype(np.int64)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def gen_fp8(shape, seed: int, kv_shape=None):
    """Q, K, V as E4M3 codes with per-tensor scales: N(0,1) float32 (PCG64, Q, K, V in
    that order; K and V of kv_shape when given), each divided by scale = max|x| / 448 and
    encoded.  Returns ([q8, k8, v8], [q_scale, k_scale, v_scale])."""
    rng = np.random.Generator(np.random.PCG64(seed))
    codes, scales = [], []
    kv_shape = shape if kv_shape is None else kv_shape
    for shp in (shape, kv_shape, kv_shape):
        a = rng.standard_normal(size=tuple(shp), dtype=np.float32)
        sc = float(np.float32(np.abs(a).max() / 448.0))
        codes.append(e4m3_encode(a / sc))
        scales.append(sc)
    return codes, scales


def gen_tensors(shape, dtype: str, seed: int, count: int):
    """`count` arrays of `shape`, i.i.d. N(0,1) float32 from PCG64(seed), in draw order.

    For dtype "bf16" each array is rounded to bf16 values (still stored as float32).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for _ in range(count):
        a = rng.standard_normal(size=tuple(shape), dtype=np.float32)
        if dtype == "bf16":
            a = bf16_round(a)
        out.append(a)
    return out


def gen_qkv(shape, dtype: str, seed: int, with_do: bool = False):
    """Q, K, V (and dO) for one workload, drawn in that order."""
    return gen_tensors(shape, dtype, seed, 4 if with_do else 3)


def gen_gqa(B: int, hq: int, hkv: int, N: int, d: int, dtype: str, seed: int, with_do: bool = False):
    """Q [B,hq,N,d], K and V [B,hkv,N,d] (and dO [B,hq,N,d]), drawn in that order.

    The inputs of attention with hq query heads sharing hkv key/value heads.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    shapes = [(B, hq, N, d), (B, hkv, N, d), (B, hkv, N, d)] + ([(B, hq, N, d)] if with_do else [])
    out = []
    for shp in shapes:
        a = rng.standard_normal(size=shp, dtype=np.float32)
        if dtype == "bf16":
            a = bf16_round(a)
        out.append(a)
    return out


# Shared K/V head shapes used by the parity tests: a grouped-query layout with
# 8 query heads per K/V head (32 query heads of 128 over 4 K/V heads, 2K tokens)
# and multi-query attention (one K/V head).
GQA_CASES = {
    "gqa_causal_b2hq32hkv4n2048d128": dict(B=2, hq=32, hkv=4, N=2048, d=128, causal=True, seed=31),
    "mqa_b2hq16hkv1n1024d64": dict(B=2, hq=16, hkv=1, N=1024, d=64, causal=False, seed=32),
}


def gen_decode(B: int, hq: int, hkv: int, nq: int, nk: int, d: int, seed: int, min_len: int | None = None):
    """Inputs of attention against a key/value cache, bf16-valued: Q [B,hq,nq,d], K and V
    [B,hkv,nk,d] (cache capacity nk), drawn in that order, then per-batch cache lengths
    (int32 [B]) uniform in [min_len, nk] (all nk when min_len is None)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for shp in [(B, hq, nq, d), (B, hkv, nk, d), (B, hkv, nk, d)]:
        out.append(bf16_round(rng.standard_normal(size=shp, dtype=np.float32)))
    if min_len is None:
        lens = np.full(B, nk, dtype=np.int32)
    else:
        lens = rng.integers(min_len, nk + 1, size=B).astype(np.int32)
    return out + [lens]


# Decode shapes (new query rows against a key/value cache) used by the parity
# tests and the benchmark: one new token per sequence with 4 query heads per
# K/V head and ragged cache lengths (a 32-head, 8-K/V-head decoder at 8K
# context), and four speculative tokens per sequence, causal, over a 4K cache.
DECODE_CASES = {
    "decode_b16hq32hkv8nk8192d128": dict(B=16, hq=32, hkv=8, nq=1, nk=8192, d=128, causal=False, min_len=4096,
                                         seed=51),
    "decode_spec4_causal_b8hq16hkv16nk4096d64": dict(B=8, hq=16, hkv=16, nq=4, nk=4096, d=64, causal=True,
                                                     min_len=None, seed=52),
}


# FP8 (E4M3) forward shapes: the 16-head, 4K-token, head-dim-128 encoder layer
# at batch 4 (16K tokens per batch), and a causal grouped-query decoder layer
# (32 query heads over 8 K/V heads, head dim 64, 2K tokens).
FP8_CASES = {
    "fp8_fwd_b4h16n4096d128": dict(B=4, hq=16, hkv=16, N=4096, d=128, causal=False, seed=61),
    "fp8_fwd_gqa_causal_b2hq32hkv8n2048d64": dict(B=2, hq=32, hkv=8, N=2048, d=64, causal=True, seed=62),
}


def fp8_case_inputs(c: dict):
    return gen_fp8((c["B"], c["hq"], c["N"], c["d"]), c["seed"], (c["B"], c["hkv"], c["N"], c["d"]))


def workload_inputs(w: Workload):
    """Inputs of a named workload: Q, K, V (and dO for a backward workload)."""
    return gen_qkv(w.shape, w.dtype, w.seed, with_do=(w.kind == "bwd"))
