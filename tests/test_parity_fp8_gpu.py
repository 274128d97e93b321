"""GPU parity of the FP8 (E4M3) forward against the float64 oracle.

The oracle is exact attention of the decoded inputs (code * per-tensor scale).
The kernel rounds each probability p_ij to E4M3 before the P V product and sums
the same rounded values into the row sum l_i, so its output is the exact
weighted mean of the rows of V under perturbed weights p~_ij = p_ij (1 + e_ij):
    o~_i - o_i = sum_j (p~_ij - p_ij) (v_j - o_i) / sum_j p~_ij.
Round-to-nearest E4M3 keeps |p~ - p| <= 2^-4 p for p >= 2^-6 (normal range)
and <= 2^-10 below it.  The kernel's p are relative to a running reference at
or below the row maximum, so the largest p of a row is at least 1 and the row
sum l >= 1 / w_max (w the exact softmax weights).  Hence, to first order,
    |o~_ic - o_ic| <= sum_j a_ij |v_jc - o_ic|,  a_ij = max(2^-4 w_ij, 2^-10 w_max,i)
    |lse~_i - lse_i| <= -ln(1 - sum_j a_ij).
The gates are these bounds times 1.1 / (1 - 2^-4) (the perturbed row sum in
the denominator, and slack for second-order terms), plus 2^-8 |o| for the
bf16 rounding of the output.  A wrong key order, scale or mask breaks them by
orders of magnitude.
"""

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_49_amd import inputs
import exact_io_aware_49_amd as fa
from gpu_common import f32, host, need_gpu, say

pytestmark = pytest.mark.gpu

def _codes(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to("cuda")


def run_fp8(q8, k8, v8, sc, causal, scale):
    o, lse = fa.forward_fp8(_codes(q8), _codes(k8), _codes(v8), sc[0], sc[1], sc[2], causal=causal, scale=scale)
    torch.cuda.synchronize()
    return host(o), host(lse)


def _decoded(q8, k8, v8, sc):
    return (oracle.e4m3_to_float(q8) * f32(sc[0]), oracle.e4m3_to_float(k8) * f32(sc[1]),
            oracle.e4m3_to_float(v8) * f32(sc[2]))


def _gate(tag, o, lse, ro, rl, w, vh):
    """o, ro: [R, d]; lse, rl: [R]; w: exact weights [R, Nk]; vh: the head's V [Nk, d]."""
    if not (np.all(np.isfinite(o)) and np.all(np.isfinite(lse))):
        raise AssertionError(f"{tag}: non-finite output")
    slack = 1.1 / (1.0 - 2.0 ** -4)
    a = np.maximum(2.0 ** -4 * w, 2.0 ** -10 * w.max(axis=1, keepdims=True))
    a = np.where(w > 0, a, 0.0)  # masked keys have p = 0 exactly
    worst = 0.0
    for r0 in range(0, o.shape[0], 16):
        sl = slice(r0, r0 + 16)
        spread = np.einsum("rj,rjc->rc", a[sl], np.abs(vh[None, :, :] - ro[sl, None, :]))
        bound = slack * spread + 2.0 ** -8 * np.abs(ro[sl]) + 1e-6
        err = np.abs(o[sl] - ro[sl])
        worst = max(worst, float((err / bound).max()))
        if not np.all(err <= bound):
            i = np.unravel_index(np.argmax(err / bound), err.shape)
            raise AssertionError(f"{tag}: O row {r0 + i[0]} col {i[1]} err {err[i]:.3e} > bound {bound[i]:.3e}")
    beta = np.minimum(slack * a.sum(axis=1), 0.5)
    lb = -np.log1p(-beta) + 1e-6
    el = np.abs(lse - rl)
    if not np.all(el <= lb):
        i = int(np.argmax(el / lb))
        raise AssertionError(f"{tag}: lse row {i} err {el[i]:.3e} > bound {lb[i]:.3e}")
    rel = float(np.linalg.norm(o - ro) / max(np.linalg.norm(ro), 1e-30))
    return worst, float(el.max()), rel


def _weights(qh, kh, rl, rows, causal, scale):
    s = (qh[rows] @ kh.T) * scale
    if causal:
        s = np.where(np.arange(kh.shape[0])[None, :] > np.asarray(rows)[:, None], -np.inf, s)
    return np.exp(s - rl[:, None])


def check_fp8(q8, k8, v8, sc, causal, tag, heads=None, rows_per_head=None, seed=0):
    """Full check of the listed heads (all when None), or of sampled rows of them."""
    need_gpu()
    B, H, N, d = q8.shape
    hkv = k8.shape[1]
    scale = f32(d ** -0.5)
    say(f"[fp8] {tag} q={q8.shape} kv={k8.shape} causal={causal} scales={sc}")
    o, lse = run_fp8(q8, k8, v8, sc, causal, scale)
    q, k, v = _decoded(q8, k8, v8, sc)
    rng = np.random.Generator(np.random.PCG64(7000 + seed))
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    worst = [0.0, 0.0, 0.0]
    for b, h in heads:
        hk = h // (H // hkv)
        if rows_per_head is None:
            rows = np.arange(N)
        else:
            rows = set(range(0, 3)) | set(range(N - 3, N)) | set(range(127, 130))
            rows |= set(int(x) for x in rng.integers(0, N, rows_per_head))
            rows = np.array(sorted(r for r in rows if 0 <= r < N))
        ro, rl = oracle.attention_forward_rows(q, k, v, causal, scale, b, h, rows)
        w = _weights(q[b, h], k[b, hk], rl, rows, causal, scale)
        e = _gate(f"{tag} [{b},{h}]", o[b, h, rows], lse[b, h, rows], ro, rl, w, v[b, hk])
        worst = [max(x, y) for x, y in zip(worst, e)]
    say(f"   worst O err/bound {worst[0]:.3f}  lse max err {worst[1]:.2e}  O rel L2 {worst[2]:.2e}")
    return worst


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_sweep(d, causal):
    # ragged N over several query blocks and key tiles, two query heads per K/V head
    (q8, k8, v8), sc = inputs.gen_fp8((2, 4, 333, d), 900 + d + causal, (2, 2, 333, d))
    worst = check_fp8(q8, k8, v8, sc, causal, f"sweep d{d} causal{int(causal)}")
    assert worst[2] < 0.05


@pytest.mark.parametrize("d", [64, 128, 256])
def test_fp8_mqa(d):
    # multi-query: eight query heads over one K/V head, ragged N, causal and not
    (q8, k8, v8), sc = inputs.gen_fp8((2, 8, 301, d), 960 + d, (2, 1, 301, d))
    for causal in (False, True):
        check_fp8(q8, k8, v8, sc, causal, f"mqa d{d} causal{int(causal)}", heads=[(0, 0), (0, 7), (1, 3)])


@pytest.mark.parametrize("N", [1, 63, 64, 65, 128, 129, 200])
def test_fp8_small_and_ragged(N):
    (q8, k8, v8), sc = inputs.gen_fp8((1, 2, N, 128), 950 + N, (1, 1, N, 128))
    check_fp8(q8, k8, v8, sc, True, f"ragged N{N}")
    check_fp8(q8, k8, v8, sc, False, f"ragged N{N}")


@pytest.mark.parametrize("name", list(inputs.FP8_CASES))
def test_fp8_cases(name):
    c = inputs.FP8_CASES[name]
    (q8, k8, v8), sc = inputs.fp8_case_inputs(c)
    heads = [(0, 0), (1, c["hq"] - 1), (c["B"] - 1, c["hq"] // 2)]
    check_fp8(q8, k8, v8, sc, c["causal"], name, heads=heads, rows_per_head=40, seed=c["seed"])


def test_fp8_zero_queries_average_v():
    # Q = 0: every visible key has p = 1 exactly (an E4M3 value), so o is the mean of
    # the visible rows of V, up to float32 summation and the bf16 output rounding
    need_gpu()
    N, d = 300, 64
    (_, k8, v8), sc = inputs.gen_fp8((1, 1, N, d), 991)
    q8 = np.zeros((1, 1, N, d), dtype=np.uint8)
    for causal in (False, True):
        o, lse = run_fp8(q8, k8, v8, sc, causal, f32(d ** -0.5))
        v = oracle.e4m3_to_float(v8)[0, 0] * f32(sc[2])
        cnt = np.arange(1, N + 1)[:, None] if causal else np.full((N, 1), N)
        ref = (np.cumsum(v, axis=0) / cnt) if causal else np.broadcast_to(v.mean(axis=0), (N, d))
        assert np.abs(o[0, 0] - ref).max() <= 2.0 ** -8 * np.abs(ref).max() + 1e-6
        assert np.abs(lse[0, 0] - np.log(cnt[:, 0])).max() <= 1e-5


def test_fp8_peaky_and_growing_scores():
    # Large q_scale makes each row nearly one-hot, and keys whose scores grow along the
    # sequence force the running maximum to move in almost every tile
    need_gpu()
    N, d = 520, 128
    (q8, k8, v8), sc = inputs.gen_fp8((1, 2, N, d), 992)
    check_fp8(q8, k8, v8, (sc[0] * 8.0, sc[1], sc[2]), False, "peaky")
    # every query row is |q row 0|; key j is that direction times ramp_j, so the scores
    # climb to about 85 (natural log units) along the keys
    ramp = np.linspace(0.05, 1.0, N)[None, None, :, None]
    qf = np.abs(oracle.e4m3_to_float(q8[:, :, :1, :]))
    k_ramp = inputs.e4m3_encode(np.broadcast_to(qf / qf.max(), (1, 2, N, d)) * ramp * 448.0)
    q_ramp = np.broadcast_to(q8[:, :, :1, :] & 0x7F, (1, 2, N, d)).copy()
    for causal in (False, True):
        check_fp8(q_ramp, k_ramp, v8, (sc[0], 0.05, sc[2]), causal, f"growing causal{int(causal)}")
