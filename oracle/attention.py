"""Naive float64 attention and its gradients -- TEST INFRASTRUCTURE ONLY.

The forward follows the attention equation of "FlashAttention (DE)",
section "Problematik der Standard-Attention":

    Attention(Q, K, V) = softmax(Q K^T / sqrt(d_k)) V

computed the way that section describes the standard implementation: the
whole N x N score matrix S is formed, each row is normalised by a two-pass
softmax (row maximum, then exponentials and their sum), and the normalised
matrix P multiplies V.  The scale 1/sqrt(d_k) is an argument (`scale`) so the
caller can pass exactly the value the GPU receives.

What the forward additionally returns, the per-row log-sum-exp
lse_i = ln sum_j exp(S_ij), is the "small normalisation value" kept for the
backward pass in the Dutch glossary page "FlashAttention", section
"Hoe werkt het?", bullet "Herberekening".  The pages give no formula for it;
the natural log of the row's exponential sum of the scaled scores is the
plain reading.

Masking is named among the fused steps in "FlashAttention (DE)", section
"Zusammenfassen von Operationen in einem CUDA-Kernel", without a definition.
The reading used here is the causal mask: query i sees key j iff j <= i
(query and key positions both start at 0; N_q = N_k).  Masked scores are -inf
and get probability exactly 0.

The backward is the calculus of the attention equation for the scalar loss
L = sum(dO * O); the pages give no backward equations:

    dV = P^T dO,  dP = dO V^T,  D_i = sum_j P_ij dP_ij,
    dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.

All arithmetic is numpy float64 on the exact values the GPU receives (inputs
are upcast, never rounded further).  Work is done one (batch, head) pair at a
time; the row-chunked forward keeps whole rows of S (every key), so it is the
same arithmetic with bounded memory.

Multi-query attention (named as a FlashAttention-2 capability in
"FlashAttention (DE)", section "Evolution und Weiterentwicklungen") lets
several query heads share one key/value head.  The pages give no definition;
the reading used here is contiguous groups: with Hq query heads and Hkv K/V
heads (Hkv divides Hq), query head h reads K/V head h // (Hq / Hkv).  Hkv = 1
is multi-query attention and Hkv = Hq ordinary multi-head attention.  Each
query head's output is the attention equation above with its group's K and V;
a shared K/V head's gradient is the sum of the gradients over the query heads
that read it (the chain rule for a shared input).

Layout: q, dO are [B, Hq, N, d]; k, v are [B, Hkv, N, d]; lse is [B, Hq, N].
"""

from __future__ import annotations

import numpy as np


def scores(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """S = scale * q k^T for one head: q [Nq, d], k [Nk, d] -> [Nq, Nk] float64.

    The product inside the softmax of the attention equation
    ("FlashAttention (DE)", section "Problematik der Standard-Attention").
    """
    q64 = np.asarray(q, dtype=np.float64)
    k64 = np.asarray(k, dtype=np.float64)
    return float(scale) * (q64 @ k64.T)


def causal_mask(s: np.ndarray, row_ids: np.ndarray) -> np.ndarray:
    """Return a copy of S with S[r, j] = -inf wherever key j > query row_ids[r].

    Causal reading of the masking step named in "FlashAttention (DE)",
    section "Zusammenfassen von Operationen in einem CUDA-Kernel".
    `row_ids` are the absolute query positions of the rows of S.
    """
    out = np.array(s, dtype=np.float64, copy=True)
    cols = np.arange(out.shape[1])
    hidden = cols[None, :] > np.asarray(row_ids)[:, None]
    out[hidden] = -np.inf
    return out


def softmax_rows(s: np.ndarray):
    """Two-pass softmax over each whole row of S.

    Returns (P, m, l) with m_i = max_j S_ij, l_i = sum_j exp(S_ij - m_i) and
    P_ij = exp(S_ij - m_i) / l_i.  A row that is entirely -inf (cannot occur
    for the causal mask with N_q = N_k) gets P = 0, m = -inf, l = 0.
    """
    s = np.asarray(s, dtype=np.float64)
    m = np.max(s, axis=1)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    e = np.exp(s - m_safe[:, None])
    e[~finite, :] = 0.0
    l = np.sum(e, axis=1)
    p = np.zeros_like(e)
    p[finite] = e[finite] / l[finite, None]
    return p, m, l


def _lse(m: np.ndarray, l: np.ndarray) -> np.ndarray:
    """lse_i = m_i + ln l_i (-inf for an empty row)."""
    out = np.full(m.shape, -np.inf)
    ok = l > 0
    out[ok] = m[ok] + np.log(l[ok])
    return out


def kv_head(h: int, hq: int, hkv: int) -> int:
    """The K/V head read by query head h when hq query heads share hkv K/V heads.

    Contiguous groups of hq / hkv query heads per K/V head (reading of the
    multi-query attention named in "FlashAttention (DE)", section
    "Evolution und Weiterentwicklungen").
    """
    if hkv < 1 or hq % hkv != 0:
        raise ValueError(f"{hq} query heads cannot share {hkv} K/V heads")
    return h // (hq // hkv)


def group_sum(g, hkv: int) -> np.ndarray:
    """Sum per-query-head gradients [B, Hq, N, d] over each K/V head's group -> [B, Hkv, N, d].

    A K/V head read by several query heads receives the sum of their
    gradients (chain rule for a shared input).
    """
    g = np.asarray(g, dtype=np.float64)
    B, hq, n, d = g.shape
    if hkv < 1 or hq % hkv != 0:
        raise ValueError(f"{hq} query heads cannot share {hkv} K/V heads")
    return g.reshape(B, hkv, hq // hkv, n, d).sum(axis=2)


def _head_forward(q, k, v, causal: bool, scale: float, row_ids):
    s = scores(q, k, scale)
    if causal:
        s = causal_mask(s, row_ids)
    p, m, l = softmax_rows(s)
    o = p @ np.asarray(v, dtype=np.float64)
    return o, _lse(m, l)


def attention_forward(q, k, v, causal: bool, scale: float, row_chunk: int | None = None):
    """Exact attention forward.  q: [B, Hq, N, d], k, v: [B, Hkv, N, d] -> (O [B,Hq,N,d], lse [B,Hq,N]).

    With `row_chunk`, query rows are processed `row_chunk` at a time; each
    chunk still sees every key, so the result is the same definition.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, H, N, d = q.shape
    hkv = k.shape[1]
    if k.shape != (B, hkv, k.shape[2], d) or v.shape[:3] != k.shape[:3] or hkv < 1 or H % hkv != 0:
        raise ValueError("q, k, v shapes do not match")
    o = np.empty((B, H, N, v.shape[3]), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    step = N if row_chunk is None else max(1, int(row_chunk))
    for b in range(B):
        for h in range(H):
            for r0 in range(0, N, step):
                r1 = min(N, r0 + step)
                rows = np.arange(r0, r1)
                hk = kv_head(h, H, hkv)
                o[b, h, r0:r1], lse[b, h, r0:r1] = _head_forward(
                    q[b, h, r0:r1], k[b, hk], v[b, hk], causal, scale, rows)
    return o, lse


def attention_forward_rows(q, k, v, causal: bool, scale: float, b: int, h: int, rows):
    """Forward for selected query rows of one (b, h): -> (O rows [R, d], lse rows [R]).

    Each output row depends only on its own row of S, so this is the same
    definition evaluated at a sample of rows (used for spot checks at sizes
    where the full matrix would not fit in host memory).
    """
    rows = np.asarray(rows, dtype=np.int64)
    q = np.asarray(q)
    k = np.asarray(k)
    hk = kv_head(h, q.shape[1], k.shape[1])
    return _head_forward(q[b, h][rows], k[b, hk], np.asarray(v)[b, hk], causal, scale, rows)


def attention_probs(q, k, causal: bool, scale: float) -> np.ndarray:
    """The full probability matrix P [B, H, N, N] (small inputs only)."""
    q = np.asarray(q)
    k = np.asarray(k)
    B, H, N, _ = q.shape
    p = np.empty((B, H, N, k.shape[2]), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            s = scores(q[b, h], k[b, kv_head(h, H, k.shape[1])], scale)
            if causal:
                s = causal_mask(s, np.arange(N))
            p[b, h] = softmax_rows(s)[0]
    return p


def attention_backward_from_probs(p, q, k, v, do, scale: float):
    """Gradients of L = sum(dO * O) for one head, given that head's P.

    dV = P^T dO; dP = dO V^T; D_i = sum_j P_ij dP_ij; dS = P (dP - D);
    dQ = scale dS K; dK = scale dS^T Q.  All float64.
    """
    p = np.asarray(p, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    dv = p.T @ do
    dp = do @ v.T
    dsum = np.sum(p * dp, axis=1)
    ds = p * (dp - dsum[:, None])
    dq = float(scale) * (ds @ k)
    dk = float(scale) * (ds.T @ q)
    return dq, dk, dv


def attention_backward(q, k, v, do, causal: bool, scale: float):
    """Exact attention backward: -> (dQ [B,Hq,N,d], dK [B,Hkv,N,d], dV [B,Hkv,N,d]) float64.

    P is formed from its definition (full S, two-pass softmax) for each query
    head; nothing from a forward pass on the GPU is used.  Per-query-head dK
    and dV are summed over each K/V head's group.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    do = np.asarray(do)
    B, H, N, d = q.shape
    hkv = k.shape[1]
    dq = np.empty((B, H, N, d), dtype=np.float64)
    dk = np.empty((B, H, k.shape[2], d), dtype=np.float64)
    dv = np.empty((B, H, k.shape[2], v.shape[3]), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            hk = kv_head(h, H, hkv)
            s = scores(q[b, h], k[b, hk], scale)
            if causal:
                s = causal_mask(s, np.arange(N))
            p = softmax_rows(s)[0]
            dq[b, h], dk[b, h], dv[b, h] = attention_backward_from_probs(
                p, q[b, h], k[b, hk], v[b, hk], do[b, h], scale)
    return dq, group_sum(dk, hkv), group_sum(dv, hkv)


def decode_positions(length: int, nq: int) -> np.ndarray:
    """Positions of nq new query rows appended to a cache of `length` rows: length - nq + i.

    Reading of attention over a key/value cache in streaming generation
    ("FlashAttention (DE)", section "Evolution und Weiterentwicklungen",
    subsection "Spezialisierte Lösungen", FlashInfer): the new queries are the
    last nq positions of the sequence whose keys and values the cache holds.
    """
    return int(length) - int(nq) + np.arange(int(nq))


def attention_decode(q, k, v, kv_lens, causal: bool, scale: float):
    """Attention of Nq query rows against a key/value cache.

    q: [B, Hq, Nq, d]; k, v: [B, Hkv, Nk, d] with Nk the cache capacity;
    kv_lens: per-batch count L_b of valid cache rows (None = Nk for every
    batch).  Query i of batch b sits at position L_b - Nq + i; it sees cache
    rows j < L_b, and with `causal` only j <= L_b - Nq + i.  Query heads share
    K/V heads as in attention_forward.  A query that sees no row gets O = 0 and
    lse = -inf.  Returns (O [B,Hq,Nq,d], lse [B,Hq,Nq]) float64.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, H, nq, d = q.shape
    hkv, nk = k.shape[1], k.shape[2]
    lens = [nk] * B if kv_lens is None else [int(x) for x in np.asarray(kv_lens).reshape(-1)]
    if len(lens) != B or any(x < 0 or x > nk for x in lens):
        raise ValueError("kv_lens must hold B values in [0, Nk]")
    o = np.zeros((B, H, nq, v.shape[3]), dtype=np.float64)
    lse = np.full((B, H, nq), -np.inf, dtype=np.float64)
    for b in range(B):
        length = lens[b]
        if length == 0:
            continue
        for h in range(H):
            hk = kv_head(h, H, hkv)
            s = scores(q[b, h], k[b, hk, :length], scale)
            if causal:
                s = causal_mask(s, decode_positions(length, nq))
            p, m, l = softmax_rows(s)
            o[b, h] = p @ np.asarray(v[b, hk, :length], dtype=np.float64)
            lse[b, h] = _lse(m, l)
    return o, lse


def e4m3_to_float(codes) -> np.ndarray:
    """Decode 8-bit floating point codes in the OCP E4M3 format to float64.

    FP8 inputs are named for FlashAttention-3 in "FlashAttention (DE)",
    section "Evolution und Weiterentwicklungen", subsection
    "FlashAttention-3 (2024)"; the pages do not fix a format.  The reading
    here is the OCP 8-bit floating point E4M3 format: sign bit, 4 exponent
    bits with bias 7, 3 mantissa bits; exponent field 0 encodes subnormals
    m * 2^-9; there are no infinities; S.1111.111 is NaN; the largest finite
    magnitude is 448.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    out = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def attention_forward_fp8(q8, k8, v8, q_scale: float, k_scale: float, v_scale: float, causal: bool,
                          scale: float):
    """Exact attention of FP8 inputs: the real inputs are the decoded E4M3 codes times their
    per-tensor scale factors (Q = e4m3(q8) * q_scale, and so on); the rest is attention_forward.
    Returns (O, lse) float64.
    """
    q = e4m3_to_float(q8) * float(q_scale)
    k = e4m3_to_float(k8) * float(k_scale)
    v = e4m3_to_float(v8) * float(v_scale)
    return attention_forward(q, k, v, causal, scale)
