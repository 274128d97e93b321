"""The oracle's pins: checks that tie oracle/ to something other than itself.

Each pin returns a list of failure strings (empty = pass), so the same battery
serves two purposes: tests/test_oracle.py asserts that every pin passes on the
real oracle, and tests/test_oracle_mutants.py plants plausible mistakes in the
oracle (on the CPU) and asserts that at least one pin then fails.

The pins use the attention equation of "FlashAttention (DE)", section
"Problematik der Standard-Attention", its exactness claim (section
"Online-Softmax-Berechnung": the result is exact), and the mathematics of the
softmax (rows of P sum to one, invariance to a per-row shift of the scores).
The pages print no worked numeric example, so the stored fixture
(golden/rational_case.json) is a hand-derived closed form.

All oracle functions are looked up on the module at call time, so a
monkeypatched step is what runs.
"""

from __future__ import annotations

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np

import oracle.attention as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fail_if(cond, msg, out):
    if cond:
        out.append(msg)


def _maxdiff(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.shape != b.shape:
        return float("inf")
    with np.errstate(invalid="ignore"):
        d = np.abs(a - b)
    d[np.isnan(d)] = np.inf
    # equal infinities compare as equal
    same_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    d[same_inf] = 0.0
    return float(d.max()) if d.size else 0.0


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# --------------------------------------------------------------------------- golden

def load_rational_case():
    with open(os.path.join(GOLDEN, "rational_case.json")) as f:
        g = json.load(f)
    fr = lambda s: float(Fraction(s))  # noqa: E731
    ln2, ln3 = math.log(2.0), math.log(3.0)
    q = np.array([[fr(x) for x in row] for row in g["Q"]])
    k = np.array([[fr(c2) * ln2 + fr(c3) * ln3 for (c2, c3) in row]
                  for row in g["K_log_coeffs"]["K"]])
    v = np.array([[fr(x) for x in row] for row in g["V"]])
    do = np.array([[fr(x) for x in row] for row in g["dO"]])
    cases = {}
    for key in ("noncausal", "causal"):
        c = g[key]
        cases[key] = {
            "P": np.array([[fr(x) for x in r] for r in c["P"]]),
            "O": np.array([[fr(x) for x in r] for r in c["O"]]),
            "lse": np.array([math.log(fr(x)) for x in c["lse_exp"]]),
            "dV": np.array([[fr(x) for x in r] for r in c["dV"]]),
            "dQ": np.array([[fr(c2) * ln2 + fr(c3) * ln3 for (c2, c3) in r]
                            for r in c["dQ_log_coeffs"]]),
            "dK": np.array([[fr(x) for x in r] for r in c["dK"]]),
        }
    return fr(g["scale"]), q, k, v, do, cases


def pin_golden_rational():
    out = []
    scale, q, k, v, do, cases = load_rational_case()
    Q, K, V, dO = (x[None, None] for x in (q, k, v, do))
    for key, causal in (("noncausal", False), ("causal", True)):
        c = cases[key]
        o, lse = A.attention_forward(Q, K, V, causal, scale)
        p = A.attention_probs(Q, K, causal, scale)
        dq, dk, dv = A.attention_backward(Q, K, V, dO, causal, scale)
        for name, got, want in (("O", o[0, 0], c["O"]), ("lse", lse[0, 0], c["lse"]),
                                ("P", p[0, 0], c["P"]), ("dQ", dq[0, 0], c["dQ"]),
                                ("dK", dk[0, 0], c["dK"]), ("dV", dv[0, 0], c["dV"])):
            err = _maxdiff(got, want)
            _fail_if(not err <= 1e-12, f"golden {key} {name}: max err {err:.3e}", out)
    return out


# --------------------------------------------------------------------------- invariants

def pin_rows_sum_to_one():
    out = []
    r = _rng(11)
    for causal in (False, True):
        q = r.standard_normal((2, 2, 37, 8))
        k = r.standard_normal((2, 2, 37, 8))
        p = A.attention_probs(q, k, causal, 0.7)
        err = float(np.abs(p.sum(-1) - 1.0).max())
        _fail_if(not err <= 1e-14, f"rows of P (causal={causal}) sum err {err:.3e}", out)
        _fail_if(not (p >= 0).all(), f"P has negative entries (causal={causal})", out)
        if causal:
            upper = np.triu(np.ones((37, 37), dtype=bool), 1)
            _fail_if(not (p[..., upper] == 0).all(), "causal P not zero above the diagonal", out)
    return out


def pin_identical_keys_mean():
    out = []
    r = _rng(12)
    N, d = 16, 4
    q = r.standard_normal((1, 1, N, d))
    k = np.repeat(r.standard_normal((1, 1, 1, d)), N, axis=2)
    v = r.standard_normal((1, 1, N, d))
    o, _ = A.attention_forward(q, k, v, False, 0.5)
    err = _maxdiff(o[0, 0], np.repeat(v[0, 0].mean(0, keepdims=True), N, axis=0))
    _fail_if(not err <= 1e-13, f"identical keys, non-causal: err {err:.3e}", out)
    o, _ = A.attention_forward(q, k, v, True, 0.5)
    want = np.cumsum(v[0, 0], axis=0) / np.arange(1, N + 1)[:, None]
    err = _maxdiff(o[0, 0], want)
    _fail_if(not err <= 1e-13, f"identical keys, causal prefix mean: err {err:.3e}", out)
    return out


def pin_dominant_score():
    out = []
    r = _rng(13)
    N, d, jstar = 10, 6, 7
    u = np.zeros(d)
    u[0] = 1.0
    a = 12.0
    k = r.standard_normal((N, d))
    k[:, 0] = 0.0                   # every other key is orthogonal to u
    k[jstar] = a * u
    q = np.tile(a * u, (N, 1))      # s * q.k* = 0.5 * 144 = 72 nats above the rest
    v = r.standard_normal((N, d))
    o, _ = A.attention_forward(q[None, None], k[None, None], v[None, None], False, 0.5)
    err = _maxdiff(o[0, 0], np.tile(v[jstar], (N, 1)))
    _fail_if(not err <= 1e-12, f"dominant score: err {err:.3e}", out)
    return out


def pin_causal_row0_and_n1():
    out = []
    r = _rng(14)
    q, k, v = (r.standard_normal((2, 3, 9, 5)) for _ in range(3))
    s = 0.3
    o, lse = A.attention_forward(q, k, v, True, s)
    _fail_if(not np.array_equal(o[:, :, 0], v[:, :, 0]), "causal row 0 is not exactly V[0]", out)
    want = s * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0])
    err = _maxdiff(lse[:, :, 0], want)
    _fail_if(not err <= 1e-15, f"causal lse_0 err {err:.3e}", out)
    q1, k1, v1 = (x[:, :, :1] for x in (q, k, v))
    for causal in (False, True):
        o1, lse1 = A.attention_forward(q1, k1, v1, causal, s)
        _fail_if(not np.array_equal(o1, v1), f"N=1 (causal={causal}): O != V", out)
        err = _maxdiff(lse1[..., 0], s * np.sum(q1[..., 0, :] * k1[..., 0, :], -1))
        _fail_if(not err <= 1e-15, f"N=1 lse err {err:.3e}", out)
    return out


def pin_shift_invariance():
    out = []
    r = _rng(15)
    q, k, v = (r.standard_normal((1, 2, 20, 6)) for _ in range(3))
    u = r.standard_normal(6)
    s = 0.4
    for causal in (False, True):
        o, lse = A.attention_forward(q, k, v, causal, s)
        o2, lse2 = A.attention_forward(q, k + u, v, causal, s)
        err = _maxdiff(o, o2)
        _fail_if(not err <= 1e-12, f"shift: O changed by {err:.3e} (causal={causal})", out)
        err = _maxdiff(lse2 - lse, s * (q @ u))
        _fail_if(not err <= 1e-12, f"shift: lse shift err {err:.3e} (causal={causal})", out)
    return out


def pin_permutation():
    out = []
    r = _rng(16)
    q, k, v = (r.standard_normal((1, 1, 15, 4)) for _ in range(3))
    s = 0.6
    o, lse = A.attention_forward(q, k, v, False, s)
    perm = r.permutation(15)
    o2, lse2 = A.attention_forward(q, k[:, :, perm], v[:, :, perm], False, s)
    err = max(_maxdiff(o, o2), _maxdiff(lse, lse2))
    _fail_if(not err <= 1e-13, f"key/value permutation changed the result by {err:.3e}", out)
    o3, lse3 = A.attention_forward(q[:, :, perm], k, v, False, s)
    err = max(_maxdiff(o3, o[:, :, perm]), _maxdiff(lse3, lse[:, :, perm]))
    _fail_if(not err <= 1e-13, f"query permutation not equivariant: {err:.3e}", out)
    return out


# --------------------------------------------------------------------------- brute force

def brute_forward(q, k, v, causal, scale):
    """Pure-Python attention for one head (lists of lists), math.exp / math.fsum only."""
    n, dv = len(q), len(v[0])
    o, lse = [], []
    for i in range(n):
        visible = [j for j in range(len(k)) if (not causal or j <= i)]
        sc = [scale * math.fsum(q[i][c] * k[j][c] for c in range(len(q[i]))) for j in visible]
        mx = max(sc)
        w = [math.exp(x - mx) for x in sc]
        tot = math.fsum(w)
        o.append([math.fsum(w[t] * v[j][c] for t, j in enumerate(visible)) / tot for c in range(dv)])
        lse.append(mx + math.log(tot))
    return o, lse


def pin_brute_force_forward():
    out = []
    r = _rng(17)
    for n, d in itertools.product((1, 2, 5, 8), (1, 3, 4)):
        q, k, v = (r.standard_normal((n, d)) for _ in range(3))
        for causal in (False, True):
            bo, bl = brute_forward(q.tolist(), k.tolist(), v.tolist(), causal, 0.9)
            o, lse = A.attention_forward(q[None, None], k[None, None], v[None, None], causal, 0.9)
            err = max(_maxdiff(o[0, 0], bo), _maxdiff(lse[0, 0], bl))
            _fail_if(not err <= 1e-14, f"brute force n={n} d={d} causal={causal}: {err:.3e}", out)
    return out


def pin_finite_differences():
    """Central differences of L = sum(dO * O) through the pure-Python forward."""
    out = []
    r = _rng(18)
    h = 1e-6
    for n, d, causal in itertools.product((1, 3, 5, 8), (2, 4), (False, True)):
        q, k, v, do = (r.standard_normal((n, d)) for _ in range(4))
        s = 0.8

        def loss(qq, kk, vv):
            o, _ = brute_forward(qq.tolist(), kk.tolist(), vv.tolist(), causal, s)
            return math.fsum(o[i][c] * do[i][c] for i in range(n) for c in range(d))

        dq, dk, dv = A.attention_backward(q[None, None], k[None, None], v[None, None],
                                          do[None, None], causal, s)
        for name, x, g in (("dQ", q, dq[0, 0]), ("dK", k, dk[0, 0]), ("dV", v, dv[0, 0])):
            num = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                xp = x.copy()
                xm = x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = [q, k, v]
                args_m = [q, k, v]
                which = {"dQ": 0, "dK": 1, "dV": 2}[name]
                args_p[which] = xp
                args_m[which] = xm
                num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
            scale_ref = max(1.0, float(np.abs(num).max()))
            err = float(np.abs(num - g).max()) / scale_ref
            _fail_if(not err <= 1e-6,
                     f"finite differences {name} n={n} d={d} causal={causal}: rel {err:.3e}", out)
    return out


# --------------------------------------------------------------------------- shared K/V heads

def _gqa_cases():
    # (Hq, Hkv): multi-query, two groups, plain multi-head
    return ((3, 1), (4, 2), (2, 2))


def pin_gqa_brute_force():
    """Query head h of Hq attends with K/V head floor(h * Hkv / Hq) (contiguous groups);
    checked head by head against the pure-Python forward."""
    out = []
    r = _rng(21)
    for (hq, hkv), n, causal in itertools.product(_gqa_cases(), (1, 4, 7), (False, True)):
        d = 3
        q = r.standard_normal((1, hq, n, d))
        k, v = (r.standard_normal((1, hkv, n, d)) for _ in range(2))
        o, lse = A.attention_forward(q, k, v, causal, 0.7)
        for h in range(hq):
            g = (h * hkv) // hq
            bo, bl = brute_forward(q[0, h].tolist(), k[0, g].tolist(), v[0, g].tolist(), causal, 0.7)
            err = max(_maxdiff(o[0, h], bo), _maxdiff(lse[0, h], bl))
            _fail_if(not err <= 1e-14, f"shared K/V brute force Hq={hq} Hkv={hkv} n={n} h={h}: {err:.3e}", out)
    return out


def pin_gqa_finite_differences():
    """Central differences of L = sum over query heads of sum(dO * O) with respect to the
    shared K and V entries, through the pure-Python forward."""
    out = []
    r = _rng(22)
    h = 1e-6
    for (hq, hkv), causal in itertools.product(((3, 1), (4, 2)), (False, True)):
        n, d, s = 4, 2, 0.8
        q, do = (r.standard_normal((1, hq, n, d)) for _ in range(2))
        k, v = (r.standard_normal((1, hkv, n, d)) for _ in range(2))

        def loss(kk, vv):
            tot = []
            for qh in range(hq):
                g = (qh * hkv) // hq
                o, _ = brute_forward(q[0, qh].tolist(), kk[0, g].tolist(), vv[0, g].tolist(), causal, s)
                tot += [o[i][c] * do[0, qh, i, c] for i in range(n) for c in range(d)]
            return math.fsum(tot)

        _, dk, dv = A.attention_backward(q, k, v, do, causal, s)
        for name, x, gr in (("dK", k, dk), ("dV", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                xp = x.copy()
                xm = x.copy()
                xp[idx] += h
                xm[idx] -= h
                num[idx] = ((loss(xp, v) - loss(xm, v)) if name == "dK" else (loss(k, xp) - loss(k, xm))) / (2 * h)
            scale_ref = max(1.0, float(np.abs(num).max()))
            err = float(np.abs(num - np.asarray(gr)).max()) / scale_ref if np.shape(gr) == x.shape else float("inf")
            _fail_if(not err <= 1e-6, f"shared K/V finite differences {name} Hq={hq} Hkv={hkv} "
                                      f"causal={causal}: rel {err:.3e}", out)
    return out


# --------------------------------------------------------------------------- key/value cache (decode)

def brute_decode(q, k, v, length, causal, scale):
    """Pure-Python attention of the rows of q against the first `length` rows of k, v, the
    queries being the last len(q) positions (query i at length - len(q) + i)."""
    nq, dv = len(q), len(v[0])
    o, lse = [], []
    for i in range(nq):
        pos = length - nq + i
        vis = [j for j in range(length) if (not causal or j <= pos)]
        if not vis:
            o.append([0.0] * dv)
            lse.append(-math.inf)
            continue
        sc = [scale * math.fsum(q[i][c] * k[j][c] for c in range(len(q[i]))) for j in vis]
        mx = max(sc)
        w = [math.exp(x - mx) for x in sc]
        tot = math.fsum(w)
        o.append([math.fsum(w[t] * v[j][c] for t, j in enumerate(vis)) / tot for c in range(dv)])
        lse.append(mx + math.log(tot))
    return o, lse


def pin_decode_brute_force():
    """Per-batch cache lengths, last-positions alignment, shared K/V heads: against the
    pure-Python loop, head by head."""
    out = []
    r = _rng(23)
    for (hq, hkv), nq, causal in itertools.product(((2, 1), (2, 2)), (1, 3), (False, True)):
        B, nk, d = 3, 9, 3
        lens = [9, 4, 2]  # 2 < nq = 3: the first query of that batch sees nothing when causal
        q = r.standard_normal((B, hq, nq, d))
        k, v = (r.standard_normal((B, hkv, nk, d)) for _ in range(2))
        o, lse = A.attention_decode(q, k, v, np.array(lens), causal, 0.6)
        for b in range(B):
            for h in range(hq):
                g = (h * hkv) // hq
                bo, bl = brute_decode(q[b, h].tolist(), k[b, g].tolist(), v[b, g].tolist(), lens[b], causal, 0.6)
                err = max(_maxdiff(o[b, h], bo), _maxdiff(lse[b, h], bl))
                _fail_if(not err <= 1e-14, f"decode brute force Hq={hq} Hkv={hkv} nq={nq} causal={causal} "
                                           f"b={b} h={h}: {err:.3e}", out)
    return out


def pin_decode_reduces_to_forward():
    """A full cache with as many queries as rows is ordinary (causal) attention."""
    out = []
    r = _rng(24)
    for causal in (False, True):
        q, k, v = (r.standard_normal((2, 2, 6, 4)) for _ in range(3))
        o, lse = A.attention_decode(q, k, v, None, causal, 0.5)
        of, lf = A.attention_forward(q, k, v, causal, 0.5)
        err = max(_maxdiff(o, of), _maxdiff(lse, lf))
        _fail_if(not err <= 1e-14, f"decode with Nq = Nk != forward (causal={causal}): {err:.3e}", out)
    return out


# --------------------------------------------------------------------------- FP8 inputs

def pin_e4m3_codes():
    """Values of the OCP E4M3 format (bias 7, 3 mantissa bits, subnormal step 2^-9, largest
    finite 448, S.1111.111 NaN, no infinities), code by code."""
    out = []
    table = {0x00: 0.0, 0x38: 1.0, 0xB8: -1.0, 0x40: 2.0, 0x3C: 1.5, 0x30: 0.5, 0x08: 2.0 ** -6,
             0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x0F: 1.875 * 2.0 ** -6, 0x7E: 448.0, 0xFE: -448.0,
             0x77: 240.0, 0x78: 256.0, 0x4E: 7.0}
    dec = A.e4m3_to_float(np.array(list(table), dtype=np.uint8))
    for (code, want), got in zip(table.items(), dec):
        _fail_if(not got == want, f"e4m3 code 0x{code:02x}: {got} != {want}", out)
    _fail_if(not np.isnan(A.e4m3_to_float(np.array([0x7F, 0xFF], np.uint8))).all(), "e4m3 NaN codes", out)
    allv = A.e4m3_to_float(np.arange(0x00, 0x7F, dtype=np.uint8))
    _fail_if(not np.all(np.diff(allv) > 0), "e4m3 positive codes not strictly increasing", out)
    # spacing: 2^-9 among the subnormals and in the first binade, doubling with each binade
    d = np.diff(allv)
    want = np.array([2.0 ** -9 if i < 8 else 2.0 ** ((i >> 3) - 10) for i in range(len(d))])
    _fail_if(not np.allclose(d, want, rtol=0, atol=0), "e4m3 spacing", out)
    return out


def pin_e4m3_matches_torch():
    """Every E4M3 code decodes to the value torch's float8_e4m3fn gives it (a library routine
    written independently of the oracle)."""
    import torch
    out = []
    codes = np.arange(256, dtype=np.uint8)
    ours = A.e4m3_to_float(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    bad = np.nonzero(~same)[0]
    _fail_if(bad.size != 0, f"e4m3 codes differing from torch: {[hex(int(b)) for b in bad[:8]]}", out)
    return out


def pin_fp8_forward_is_forward_of_decoded():
    """The FP8 forward equals the plain forward of the decoded, scaled inputs (brute force)."""
    out = []
    r = _rng(25)
    codes = [r.integers(0, 0x7F, size=(1, 1, 5, 3)).astype(np.uint8) | (r.integers(0, 2, size=(1, 1, 5, 3)).astype(np.uint8) << 7) for _ in range(3)]
    scales = [0.01, 0.02, 0.5]
    o, lse = A.attention_forward_fp8(*codes, *scales, True, 0.7)
    vals = []
    for c, sc in zip(codes, scales):
        vals.append([[math.copysign(1.0, -1.0 if (x & 0x80) else 1.0) *
                      ((x & 7) * 2.0 ** -9 if ((x >> 3) & 15) == 0 else (1 + (x & 7) / 8) * 2.0 ** (((x >> 3) & 15) - 7)) * sc
                      for x in row] for row in c[0, 0].tolist()])
    bo, bl = brute_forward(vals[0], vals[1], vals[2], True, 0.7)
    err = max(_maxdiff(o[0, 0], bo), _maxdiff(lse[0, 0], bl))
    _fail_if(not err <= 1e-14, f"fp8 forward vs brute force: {err:.3e}", out)
    return out


# --------------------------------------------------------------------------- library routines

def pin_torch_float64():
    import torch
    out = []
    r = _rng(19)
    for causal in (False, True):
        q, k, v, do = (r.standard_normal((2, 3, 24, 8)) for _ in range(4))
        s = 0.35
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        sc = s * (tq @ tk.transpose(-1, -2))
        if causal:
            sc = sc.masked_fill(torch.ones(24, 24, dtype=torch.bool).triu(1), float("-inf"))
        to = torch.softmax(sc, dim=-1) @ tv
        tl = torch.logsumexp(sc, dim=-1)
        (to * torch.tensor(do)).sum().backward()
        o, lse = A.attention_forward(q, k, v, causal, s)
        err = max(_maxdiff(o, to.detach().numpy()), _maxdiff(lse, tl.detach().numpy()))
        _fail_if(not err <= 1e-12, f"torch float64 forward (causal={causal}): {err:.3e}", out)
        sdpa = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(q), torch.tensor(k), torch.tensor(v), is_causal=causal, scale=s)
        err = _maxdiff(o, sdpa.numpy())
        _fail_if(not err <= 1e-12, f"torch SDPA float64 (causal={causal}): {err:.3e}", out)
        dq, dk, dv = A.attention_backward(q, k, v, do, causal, s)
        err = max(_maxdiff(dq, tq.grad.numpy()), _maxdiff(dk, tk.grad.numpy()),
                  _maxdiff(dv, tv.grad.numpy()))
        _fail_if(not err <= 1e-12, f"torch autograd gradients (causal={causal}): {err:.3e}", out)
    return out


# --------------------------------------------------------------------------- gradient identities

def pin_gradient_identities():
    out = []
    r = _rng(20)
    N = 13
    q, k, v, do = (r.standard_normal((1, 2, N, 5)) for _ in range(4))
    s = 0.45
    for causal in (False, True):
        dq, dk, dv = A.attention_backward(q, k, v, do, causal, s)
        err = float(np.abs(dk.sum(axis=2)).max())
        _fail_if(not err <= 1e-12, f"sum_j dK_j != 0 (causal={causal}): {err:.3e}", out)
        err = _maxdiff(dv.sum(axis=2), do.sum(axis=2))
        _fail_if(not err <= 1e-12, f"sum_j dV_j != sum_i dO_i (causal={causal}): {err:.3e}", out)
        if causal:
            _fail_if(not float(np.abs(dq[:, :, 0]).max()) <= 1e-15, "causal dQ_0 != 0", out)
            p = A.attention_probs(q, k, True, s)
            want = p[:, :, N - 1, N - 1][..., None] * do[:, :, N - 1]
            err = _maxdiff(dv[:, :, N - 1], want)
            _fail_if(not err <= 1e-13, f"causal dV_(N-1) closed form: {err:.3e}", out)
    return out


def pin_row_chunking():
    out = []
    r = _rng(21)
    q, k, v = (r.standard_normal((1, 2, 50, 4)) for _ in range(3))
    for causal in (False, True):
        o, lse = A.attention_forward(q, k, v, causal, 0.5)
        o2, lse2 = A.attention_forward(q, k, v, causal, 0.5, row_chunk=7)
        err = max(_maxdiff(o, o2), _maxdiff(lse, lse2))
        _fail_if(not err <= 1e-14, f"row-chunked forward differs (causal={causal}): {err:.3e}", out)
        rows = np.array([0, 3, 17, 49])
        o3, lse3 = A.attention_forward_rows(q, k, v, causal, 0.5, 0, 1, rows)
        err = max(_maxdiff(o3, o[0, 1, rows]), _maxdiff(lse3, lse[0, 1, rows]))
        _fail_if(not err <= 1e-14, f"row-sampled forward differs (causal={causal}): {err:.3e}", out)
    return out


ALL_PINS = [
    pin_golden_rational,
    pin_rows_sum_to_one,
    pin_identical_keys_mean,
    pin_dominant_score,
    pin_causal_row0_and_n1,
    pin_shift_invariance,
    pin_permutation,
    pin_brute_force_forward,
    pin_finite_differences,
    pin_torch_float64,
    pin_gradient_identities,
    pin_row_chunking,
    pin_gqa_brute_force,
    pin_gqa_finite_differences,
    pin_decode_brute_force,
    pin_decode_reduces_to_forward,
    pin_e4m3_codes,
    pin_e4m3_matches_torch,
    pin_fp8_forward_is_forward_of_decoded,
]


def run_all_pins():
    failures = []
    for pin in ALL_PINS:
        try:
            failures += pin()
        except Exception as e:  # a mutant may also crash a pin: that counts as caught
            failures.append(f"{pin.__name__} raised {type(e).__name__}: {e}")
    return failures
