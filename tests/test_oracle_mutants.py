"""Plant plausible mistakes in the oracle (on the CPU) and check the pins catch each one.

A pin battery that passes on a wrong oracle proves nothing, so every mutant
below -- a dropped scale, a transposed operand, a sign error, an off-by-one
mask, a missing log, a dropped gradient term, a wrong query-head to K/V-head
mapping, a missing sum over a shared K/V head's group -- must make at least
one pin fail.
"""

import numpy as np
import pytest

import oracle.attention as A
import pins

_orig_scores = A.scores
_orig_mask = A.causal_mask
_orig_softmax = A.softmax_rows
_orig_lse = A._lse
_orig_bwd = A.attention_backward_from_probs


def m_no_scale(q, k, scale):
    return _orig_scores(q, k, 1.0)


def m_transposed_scores(q, k, scale):
    return float(scale) * (np.asarray(k, np.float64) @ np.asarray(q, np.float64).T)


def m_sqrt_scale(q, k, scale):
    return _orig_scores(q, k, float(scale) ** 0.5)


def m_mask_diagonal(s, row_ids):
    out = np.array(s, dtype=np.float64, copy=True)
    cols = np.arange(out.shape[1])
    out[cols[None, :] >= np.asarray(row_ids)[:, None] + 1] = -np.inf
    out[cols[None, :] == np.asarray(row_ids)[:, None]] = -np.inf  # hides the diagonal too
    return out


def m_mask_lower(s, row_ids):
    out = np.array(s, dtype=np.float64, copy=True)
    cols = np.arange(out.shape[1])
    out[cols[None, :] < np.asarray(row_ids)[:, None]] = -np.inf  # wrong triangle
    return out


def m_softmax_sign(s):
    p, m, l = _orig_softmax(-np.asarray(s))
    return p, -m, l


def m_softmax_columns(s):
    s = np.asarray(s, dtype=np.float64)
    e = np.exp(s - np.max(s))
    e[np.isinf(s)] = 0.0
    col = e.sum(axis=0, keepdims=True)
    col[col == 0] = 1.0
    return e / col, np.max(s, axis=1), e.sum(axis=1)


def m_lse_missing_log(m, l):
    return m + l


def m_lse_missing_max(m, l):
    return np.log(np.where(l > 0, l, 1.0))


def m_bwd_drop_D(p, q, k, v, do, scale):
    p = np.asarray(p, np.float64)
    dp = np.asarray(do, np.float64) @ np.asarray(v, np.float64).T
    ds = p * dp
    dv = p.T @ np.asarray(do, np.float64)
    return scale * ds @ np.asarray(k, np.float64), scale * ds.T @ np.asarray(q, np.float64), dv


def m_bwd_no_transpose_dk(p, q, k, v, do, scale):
    dq, dk, dv = _orig_bwd(p, q, k, v, do, scale)
    p = np.asarray(p, np.float64)
    dp = np.asarray(do, np.float64) @ np.asarray(v, np.float64).T
    ds = p * (dp - np.sum(p * dp, axis=1)[:, None])
    return dq, scale * ds @ np.asarray(q, np.float64), dv


def m_bwd_no_scale_dq(p, q, k, v, do, scale):
    dq, dk, dv = _orig_bwd(p, q, k, v, do, scale)
    return dq / scale, dk, dv


def m_bwd_dv_untransposed(p, q, k, v, do, scale):
    dq, dk, dv = _orig_bwd(p, q, k, v, do, scale)
    return dq, dk, np.asarray(p, np.float64) @ np.asarray(do, np.float64)


def m_kv_head_modulo(h, hq, hkv):
    if hkv < 1 or hq % hkv != 0:
        raise ValueError("bad grouping")
    return h % hkv  # interleaved instead of contiguous groups


def m_group_first(g, hkv):
    g = np.asarray(g, np.float64)
    B, hq, n, d = g.shape
    return g.reshape(B, hkv, hq // hkv, n, d)[:, :, 0]  # first head of the group only


def m_group_mean(g, hkv):
    g = np.asarray(g, np.float64)
    B, hq, n, d = g.shape
    return g.reshape(B, hkv, hq // hkv, n, d).mean(axis=2)


def m_decode_top_left(length, nq):
    return np.arange(int(nq))  # queries aligned to the start of the cache


def m_decode_off_by_one(length, nq):
    return int(length) - int(nq) + 1 + np.arange(int(nq))


_orig_e4m3 = A.e4m3_to_float


def m_e4m3_bias8(codes):
    return _orig_e4m3(codes) / 2.0  # exponent bias 8 instead of 7


def m_e4m3_no_subnormals(codes):
    c = np.asarray(codes, np.uint8)
    v = _orig_e4m3(c)
    return np.where(((c >> 3) & 15) == 0, 0.0, v)


MUTANTS = [
    ("scores", m_no_scale),
    ("scores", m_transposed_scores),
    ("scores", m_sqrt_scale),
    ("causal_mask", m_mask_diagonal),
    ("causal_mask", m_mask_lower),
    ("softmax_rows", m_softmax_sign),
    ("softmax_rows", m_softmax_columns),
    ("_lse", m_lse_missing_log),
    ("_lse", m_lse_missing_max),
    ("attention_backward_from_probs", m_bwd_drop_D),
    ("attention_backward_from_probs", m_bwd_no_transpose_dk),
    ("attention_backward_from_probs", m_bwd_no_scale_dq),
    ("attention_backward_from_probs", m_bwd_dv_untransposed),
    ("kv_head", m_kv_head_modulo),
    ("group_sum", m_group_first),
    ("group_sum", m_group_mean),
    ("decode_positions", m_decode_top_left),
    ("decode_positions", m_decode_off_by_one),
    ("e4m3_to_float", m_e4m3_bias8),
    ("e4m3_to_float", m_e4m3_no_subnormals),
]


@pytest.mark.parametrize("target,mutant", MUTANTS, ids=[m.__name__ for _, m in MUTANTS])
def test_mutant_is_caught(monkeypatch, target, mutant):
    monkeypatch.setattr(A, target, mutant)
    failures = pins.run_all_pins()
    assert failures, f"no pin caught the planted mistake {mutant.__name__}"
