"""GPU parity: the HIP kernels (through the C ABI) against the float64 oracle.

Every case draws seeded inputs, runs the GPU path, and compares against the
oracle on the same (bf16-rounded) values.  The five named workloads run at their
full sizes; where the oracle cannot evaluate every output in seconds it checks
whole heads for a subset and sampled rows (each an exact oracle evaluation of
that row) everywhere else.  Small sweeps cover ragged lengths, N = 1, both head
dims, both masks and both dtypes.
"""

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_49_amd import inputs
import exact_io_aware_49_amd as fa
from gpu_common import assert_close, dev, f32, host, need_gpu, say

pytestmark = pytest.mark.gpu


def run_fwd(q, k, v, causal, scale, dtype):
    qd, kd, vd = dev(q, dtype), dev(k, dtype), dev(v, dtype)
    o, lse = fa.forward(qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return host(o), host(lse)


def check_fwd_full(q, k, v, causal, scale, dtype, tag, stress=False):
    say(f"[fwd] {tag} shape={q.shape} causal={causal} dtype={dtype}")
    o, lse = run_fwd(q, k, v, causal, scale, dtype)
    ro, rl = oracle.attention_forward(q, k, v, causal, f32(scale))
    eo = assert_close(f"{tag} O", o, ro, dtype, magnitude_scaled=stress)
    el = assert_close(f"{tag} lse", lse, rl, dtype, lse=True, magnitude_scaled=stress)
    say(f"   O max/rel {eo[0]:.2e}/{eo[1]:.2e}  lse max {el[0]:.2e}")


# ------------------------------------------------------------------ named workloads

def test_workload_fwd_f32_small():
    need_gpu()
    w = inputs.WORKLOADS["fwd_f32_b1h2n128d64"]
    q, k, v = inputs.workload_inputs(w)
    check_fwd_full(q, k, v, w.causal, w.scale, w.dtype, w.name)


def test_workload_fwd_gpt2_causal():
    need_gpu()
    w = inputs.WORKLOADS["fwd_gpt2_causal_b8h12n1024d64"]
    q, k, v = inputs.workload_inputs(w)
    check_fwd_full(q, k, v, w.causal, w.scale, w.dtype, w.name)


def _sampled_rows(N, rng, n_rand):
    rows = set(range(0, 4)) | set(range(N - 4, N)) | set(range(127, 130))
    rows |= set(int(x) for x in rng.integers(0, N, n_rand))
    return np.array(sorted(r for r in rows if 0 <= r < N))


def check_fwd_sampled(w, full_heads, n_rand):
    need_gpu()
    q, k, v = inputs.workload_inputs(w)
    say(f"[fwd] {w.name} (full heads {full_heads}, sampled rows elsewhere)")
    o, lse = run_fwd(q, k, v, w.causal, w.scale, w.dtype)
    s = f32(w.scale)
    rng = np.random.Generator(np.random.PCG64(1000 + w.seed))
    B, H, N, d = w.shape
    worst = [0.0, 0.0]
    for b in range(B):
        for h in range(H):
            if (b, h) in full_heads:
                ro, rl = oracle.attention_forward(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1],
                                                  v[b:b + 1, h:h + 1], w.causal, s)
                e = assert_close(f"{w.name} O[{b},{h}]", o[b, h], ro[0, 0], w.dtype)
                assert_close(f"{w.name} lse[{b},{h}]", lse[b, h], rl[0, 0], w.dtype, lse=True)
            else:
                rows = _sampled_rows(N, rng, n_rand)
                ro, rl = oracle.attention_forward_rows(q, k, v, w.causal, s, b, h, rows)
                e = assert_close(f"{w.name} O[{b},{h}] rows", o[b, h, rows], ro, w.dtype)
                assert_close(f"{w.name} lse[{b},{h}] rows", lse[b, h, rows], rl, w.dtype, lse=True)
            worst = [max(worst[0], e[0]), max(worst[1], e[1])]
    say(f"   worst O max/rel {worst[0]:.2e}/{worst[1]:.2e}")


def test_workload_fwd_encoder():
    check_fwd_sampled(inputs.WORKLOADS["fwd_encoder_b4h16n4096d128"], {(0, 0), (1, 7), (3, 15)}, 48)


def test_workload_fwd_longctx_causal():
    """The 32K causal forward: heads 0 and 31 in full; on every head the first, a middle
    and the last 256-row query block (one workgroup's rows each; the last one holds the
    causal diagonal of the longest rows) plus sampled rows elsewhere."""
    need_gpu()
    w = inputs.WORKLOADS["fwd_longctx_causal_b1h32n32768d128"]
    q, k, v = inputs.workload_inputs(w)
    B, H, N, d = w.shape
    say(f"[fwd] {w.name}: full heads 0 and {H - 1}; blocks 0, {N // 512}, {N // 256 - 1} of 256 rows on every head")
    o, lse = run_fwd(q, k, v, w.causal, w.scale, w.dtype)
    s = f32(w.scale)
    worst_o, worst_l = [0.0, 0.0], 0.0
    for h in (0, H - 1):
        ro, rl = oracle.attention_forward(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], w.causal, s, row_chunk=512)
        e = assert_close(f"{w.name} O[0,{h}]", o[0, h], ro[0, 0], w.dtype)
        el = assert_close(f"{w.name} lse[0,{h}]", lse[0, h], rl[0, 0], w.dtype, lse=True)
        worst_o = [max(worst_o[0], e[0]), max(worst_o[1], e[1])]
        worst_l = max(worst_l, el[0])
        say(f"   head {h} in full: O max/rel {e[0]:.2e}/{e[1]:.2e}  lse max {el[0]:.2e}")
    rng = np.random.Generator(np.random.PCG64(1000 + w.seed))
    blocks = (0, N // 512, N // 256 - 1)
    for h in range(H):
        rows = set(_sampled_rows(N, rng, 8).tolist())
        for blk in blocks:
            rows |= set(range(256 * blk, 256 * blk + 256))
        rows = np.array(sorted(rows))
        ro, rl = oracle.attention_forward_rows(q, k, v, w.causal, s, 0, h, rows)
        e = assert_close(f"{w.name} O[0,{h}] blocks+rows", o[0, h, rows], ro, w.dtype)
        el = assert_close(f"{w.name} lse[0,{h}] blocks+rows", lse[0, h, rows], rl, w.dtype, lse=True)
        worst_o = [max(worst_o[0], e[0]), max(worst_o[1], e[1])]
        worst_l = max(worst_l, el[0])
    say(f"   worst O max/rel {worst_o[0]:.2e}/{worst_o[1]:.2e}  worst lse max {worst_l:.2e}")


# ------------------------------------------------------------------ the two named C entry points, called raw

def _raw_fwd(qd, kd, vd, causal, scale, dtype_code):
    B, H, N, d = qd.shape
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=qd.device)
    rc = fa.fa_fwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d,
                   int(causal), scale, dtype_code, torch.cuda.current_stream().cuda_stream)
    assert rc == 0, fa.fa_status_string(rc)
    return o, lse


def test_c_abi_fa_fwd_fp32_and_gpt2_workloads():
    """fa_fwd itself (raw device pointers through ctypes) on the float32 workload
    (B1 H2 N128 d64, 1e-5) and the GPT-2-shape causal bf16 workload, every output
    element against the oracle."""
    need_gpu()
    for name, code in (("fwd_f32_b1h2n128d64", fa.FA_DTYPE_F32), ("fwd_gpt2_causal_b8h12n1024d64", fa.FA_DTYPE_BF16)):
        w = inputs.WORKLOADS[name]
        say(f"[fa_fwd raw] {w.name}")
        q, k, v = inputs.workload_inputs(w)
        o, lse = _raw_fwd(dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype), w.causal, w.scale, code)
        torch.cuda.synchronize()
        ro, rl = oracle.attention_forward(q, k, v, w.causal, f32(w.scale))
        eo = assert_close(f"{w.name} O", host(o), ro, w.dtype)
        el = assert_close(f"{w.name} lse", host(lse), rl, w.dtype, lse=True)
        say(f"   O max/rel {eo[0]:.2e}/{eo[1]:.2e}  lse max {el[0]:.2e}")


def test_c_abi_fa_bwd_causal_workload():
    """fa_fwd then fa_bwd (raw pointers, caller-allocated workspace of
    fa_bwd_workspace_size bytes) on the causal backward workload B4 H16 N2048 d64:
    six heads in full against the oracle's gradients, identities on all heads."""
    need_gpu()
    w = inputs.WORKLOADS["bwd_causal_b4h16n2048d64"]
    q, k, v, do = inputs.workload_inputs(w)
    B, H, N, d = w.shape
    say(f"[fa_bwd raw] {w.name}")
    qd, kd, vd, dod = (dev(x, "bf16") for x in (q, k, v, do))
    o, lse = _raw_fwd(qd, kd, vd, w.causal, w.scale, fa.FA_DTYPE_BF16)
    need = fa.fa_bwd_workspace_size(B, H, N, d, fa.FA_DTYPE_BF16)
    assert need == 2 * B * H * N * 4
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    rc = fa.fa_bwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), dod.data_ptr(), lse.data_ptr(),
                   dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), need, B, H, N, d, int(w.causal),
                   w.scale, fa.FA_DTYPE_BF16, torch.cuda.current_stream().cuda_stream)
    assert rc == 0, fa.fa_status_string(rc)
    torch.cuda.synchronize()
    gq, gk, gv = host(dq), host(dk), host(dv)
    s = f32(w.scale)
    worst = {}
    for (b, h) in [(0, 0), (0, 15), (1, 3), (2, 8), (3, 0), (3, 15)]:
        sl = (slice(b, b + 1), slice(h, h + 1))
        rq, rk, rv = oracle.attention_backward(q[sl], k[sl], v[sl], do[sl], w.causal, s)
        for name, got, ref in (("dQ", gq[b, h], rq[0, 0]), ("dK", gk[b, h], rk[0, 0]), ("dV", gv[b, h], rv[0, 0])):
            e = assert_close(f"{w.name} {name}[{b},{h}]", got, ref, "bf16")
            worst[name] = max(worst.get(name, (0, 0)), e)
    assert np.abs(gk.sum(axis=2)).max() < 0.5
    assert np.abs(gv.sum(axis=2) - do.astype(np.float64).sum(axis=2)).max() < 0.5
    say("   worst " + "  ".join(f"{n} max/rel {e[0]:.2e}/{e[1]:.2e}" for n, e in worst.items()))


def run_bwd(q, k, v, do, causal, scale, dtype="bf16"):
    qd, kd, vd, dod = (dev(x, dtype) for x in (q, k, v, do))
    o, lse = fa.forward(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv = fa.backward(qd, kd, vd, o, dod, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return host(dq), host(dk), host(dv)


def check_bwd_heads(q, k, v, do, causal, scale, heads, tag, stress=False):
    say(f"[bwd] {tag} shape={q.shape} causal={causal} heads checked={len(heads)}")
    dq, dk, dv = run_bwd(q, k, v, do, causal, scale)
    s = f32(scale)
    worst = {}
    for (b, h) in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        rq, rk, rv = oracle.attention_backward(q[sl], k[sl], v[sl], do[sl], causal, s)
        for name, got, ref in (("dQ", dq[b, h], rq[0, 0]), ("dK", dk[b, h], rk[0, 0]), ("dV", dv[b, h], rv[0, 0])):
            e = assert_close(f"{tag} {name}[{b},{h}]", got, ref, "bf16", magnitude_scaled=stress)
            worst[name] = max(worst.get(name, (0, 0)), e)
    say("   worst " + "  ".join(f"{n} max/rel {e[0]:.2e}/{e[1]:.2e}" for n, e in worst.items()))
    return dq, dk, dv


def test_workload_bwd_causal():
    need_gpu()
    w = inputs.WORKLOADS["bwd_causal_b4h16n2048d64"]
    q, k, v, do = inputs.workload_inputs(w)
    heads = [(0, 0), (0, 15), (1, 3), (2, 8), (3, 0), (3, 15)]
    dq, dk, dv = check_bwd_heads(q, k, v, do, w.causal, w.scale, heads, w.name)
    # every head: gradient identities of the exact result (sum_j dK_j = 0, sum_j dV_j = sum_i dO_i)
    assert np.abs(dk.sum(axis=2)).max() < 0.5
    assert np.abs(dv.sum(axis=2) - do.astype(np.float64).sum(axis=2)).max() < 0.5


def test_bwd_causal_resident_grid_orders():
    """Causal backward launches whose dQ and dK/dV grids are resident at once take the snake
    dispatch order.  The GPT-2 shape (B8 H12 N1024 d64: three full rounds in both kernels) on every
    head against the oracle; two full rounds and a partial one (B8 H10 N1024 d64) and d = 32
    (B8 H12 N1024) on a spread of heads, gradient identities on all."""
    need_gpu()
    cases = [((8, 12, 1024, 64), None), ((8, 10, 1024, 64), 16), ((8, 12, 1024, 32), 16)]
    for i, ((B, H, N, d), nheads) in enumerate(cases):
        q, k, v, do = inputs.gen_qkv((B, H, N, d), "bf16", 2400 + 13 * i, with_do=True)
        allh = [(b, h) for b in range(B) for h in range(H)]
        heads = allh if nheads is None else allh[:: max(1, len(allh) // nheads)]
        dq, dk, dv = check_bwd_heads(q, k, v, do, True, d ** -0.5, heads, f"resident causal grid B={B} H={H} d={d}")
        assert np.abs(dk.sum(axis=2)).max() < 0.5
        assert np.abs(dv.sum(axis=2) - do.astype(np.float64).sum(axis=2)).max() < 0.5


def test_bwd_encoder_shape():
    """The backward at the non-causal d=128 encoder shape (the benchmark's step): two heads in
    full against the oracle, the gradient identities of the exact result on all 64."""
    need_gpu()
    w = inputs.WORKLOADS["fwd_encoder_b4h16n4096d128"]
    q, k, v, do = inputs.gen_qkv(w.shape, "bf16", w.seed, with_do=True)
    dq, dk, dv = check_bwd_heads(q, k, v, do, False, w.scale, [(0, 0), (3, 15)], "bwd_encoder_b4h16n4096d128")
    assert np.abs(dk.sum(axis=2)).max() < 0.5
    assert np.abs(dv.sum(axis=2) - do.astype(np.float64).sum(axis=2)).max() < 0.5


# ------------------------------------------------------------------ decode (key/value cache)

def _decode_check(q, k, v, lens, causal, tag):
    """fa.decode against the oracle on every output.  Rows that see no cache row must be
    exactly O = 0, lse = -inf; the rest use the bf16 bounds."""
    d = q.shape[3]
    say(f"[decode] {tag} q={q.shape} cache={k.shape} causal={causal} lens={None if lens is None else lens.tolist()[:8]}")
    ld = None if lens is None else torch.from_numpy(np.ascontiguousarray(lens, dtype=np.int32)).to("cuda")
    o, lse = fa.decode(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), ld, causal=causal)
    torch.cuda.synchronize()
    o, lse = host(o), host(lse)
    ro, rl = oracle.attention_decode(q, k, v, lens, causal, f32(d ** -0.5))
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(lse), empty), f"{tag}: rows without visible keys differ"
    assert np.all(o[empty] == 0.0), f"{tag}: a row without visible keys has O != 0"
    eo = assert_close(f"{tag} O", o, ro, "bf16")
    if (~empty).any():
        el = assert_close(f"{tag} lse", lse[~empty], rl[~empty], "bf16", lse=True)
        say(f"   O max/rel {eo[0]:.2e}/{eo[1]:.2e}  lse max {el[0]:.2e}  empty rows {int(empty.sum())}")


@pytest.mark.parametrize("name", list(inputs.DECODE_CASES))
def test_decode_cases(name):
    need_gpu()
    c = inputs.DECODE_CASES[name]
    q, k, v, lens = inputs.gen_decode(c["B"], c["hq"], c["hkv"], c["nq"], c["nk"], c["d"], c["seed"], c["min_len"])
    _decode_check(q, k, v, lens, c["causal"], name)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_decode_sweep(d, causal):
    """Ragged cache lengths (including 0 and fewer rows than queries), 1..40 query rows,
    shared K/V heads, caches that end inside a tile."""
    need_gpu()
    for i, (hq, hkv, nq, nk) in enumerate([(1, 1, 1, 1), (4, 2, 1, 33), (4, 2, 3, 300), (2, 1, 40, 1000),
                                            (8, 8, 2, 70), (6, 2, 17, 513)]):
        rng = np.random.Generator(np.random.PCG64(1400 + i + d))
        lens = rng.integers(0, nk + 1, size=3).astype(np.int32)
        lens[0] = nk
        q, k, v, _ = inputs.gen_decode(3, hq, hkv, nq, nk, d, 1500 + 7 * i + d)
        _decode_check(q, k, v, lens, causal, f"decode sweep Hq={hq} Hkv={hkv} Nq={nq} Nk={nk}")
    q, k, v, _ = inputs.gen_decode(2, 2, 1, 5, 200, d, 1600 + d)
    _decode_check(q, k, v, None, causal, "decode full cache")


def test_decode_long_sequences():
    """Few long sequences, so each (sequence, K/V head) is split over many waves and the merge
    combines hundreds of partials: one 64K-row cache, and two ragged causal ones."""
    need_gpu()
    q, k, v, _ = inputs.gen_decode(1, 8, 1, 1, 65536, 128, 1700)
    _decode_check(q, k, v, None, False, "decode one 64K cache")
    q, k, v, _ = inputs.gen_decode(2, 4, 1, 2, 30000, 64, 1701)
    _decode_check(q, k, v, np.array([30000, 17], dtype=np.int32), True, "decode 30000 + 17 rows, causal")


def test_decode_many_sequences():
    """More than 64 sequences: the kernel reads the cache lengths 64 sequences at a time while
    it sizes the tile list, finds each wave's first tile and moves from sequence to sequence.
    Ragged lengths with empty caches among them; a run of empty sequences across a 64-boundary."""
    need_gpu()
    for i, (B, hq, hkv, nq, nk, d, causal) in enumerate([(150, 8, 2, 1, 512, 128, False),
                                                          (97, 4, 4, 3, 300, 64, True),
                                                          (200, 2, 1, 1, 40, 64, False)]):
        rng = np.random.Generator(np.random.PCG64(1750 + i))
        lens = rng.integers(0, nk + 1, size=B).astype(np.int32)
        lens[rng.random(B) < 0.1] = 0
        lens[60:70] = 0
        lens[B - 1] = nk
        q, k, v, _ = inputs.gen_decode(B, hq, hkv, nq, nk, d, 1760 + i)
        _decode_check(q, k, v, lens, causal, f"decode B={B} Hq={hq} Hkv={hkv} Nq={nq} Nk={nk} d={d}")


def test_decode_cache_rows_past_length_not_read():
    """Cache rows at or past each sequence's length hold NaN: the output is bitwise the one with
    finite rows there (those rows are never read), for lengths that end inside a tile."""
    need_gpu()
    for d, causal in [(128, False), (64, True)]:
        q, k, v, _ = inputs.gen_decode(4, 8, 2, 3, 2000, d, 1710 + d)
        lens = np.array([2000, 1001, 37, 0], dtype=np.int32)
        _decode_check(q, k, v, lens, causal, f"decode ragged d={d}")
        ld = torch.from_numpy(lens).to("cuda")
        qd, kd, vd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
        o1, l1 = fa.decode(qd, kd, vd, ld, causal=causal)
        kn, vn = kd.clone(), vd.clone()
        for b, n in enumerate(lens.tolist()):
            kn[b, :, n:] = float("nan")
            vn[b, :, n:] = float("nan")
        o2, l2 = fa.decode(qd, kn, vn, ld, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"d={d}: output depends on rows past the length"


def test_decode_bitwise_repeatable():
    """Two calls on the 8K-cache decode workload give bitwise equal results."""
    need_gpu()
    c = inputs.DECODE_CASES["decode_b16hq32hkv8nk8192d128"]
    q, k, v, lens = inputs.gen_decode(c["B"], c["hq"], c["hkv"], c["nq"], c["nk"], c["d"], c["seed"], c["min_len"])
    qd, kd, vd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    ld = torch.from_numpy(np.ascontiguousarray(lens, dtype=np.int32)).to("cuda")
    outs = [fa.decode(qd, kd, vd, ld) for _ in range(3)]
    torch.cuda.synchronize()
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])


# ------------------------------------------------------------------ head dim 256 (forward)

@pytest.mark.parametrize("causal", [False, True])
def test_fwd_d256_sweep(causal):
    """Head dim 256, bf16 forward: ragged lengths against the oracle on every output."""
    need_gpu()
    for i, N in enumerate([1, 17, 64, 100, 129, 300]):
        q, k, v = inputs.gen_qkv((1 + i % 2, 1 + i % 3, N, 256), "bf16", 1300 + 7 * i)
        check_fwd_full(q, k, v, causal, 256 ** -0.5, "bf16", f"d256 sweep N={N}")


def test_fwd_d256_heads():
    """Head dim 256 at B=2 H=8 N=2048, causal, with query heads sharing K/V heads (4 per K/V
    head): whole heads of batch 0 against the oracle."""
    need_gpu()
    B, hq, hkv, N, d = 2, 8, 2, 2048, 256
    q, k, v = inputs.gen_gqa(B, hq, hkv, N, d, "bf16", 41)
    say(f"[fwd] d256 B={B} Hq={hq} Hkv={hkv} N={N} causal")
    o, lse = fa.forward(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), causal=True)
    torch.cuda.synchronize()
    o, lse = host(o), host(lse)
    ro, rl = oracle.attention_forward(q[:1], k[:1], v[:1], True, f32(d ** -0.5))
    eo = assert_close("d256 O", o[:1], ro, "bf16")
    el = assert_close("d256 lse", lse[:1], rl, "bf16", lse=True)
    say(f"   O max/rel {eo[0]:.2e}/{eo[1]:.2e}  lse max {el[0]:.2e}")


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_d256(causal):
    """Head dim 256, bf16 backward (dQ kernel at one wave per SIMD; dV and dK from two
    launches of the key-owner kernel): ragged lengths, then B=1 H=4 N=1024 on every head."""
    need_gpu()
    for i, N in enumerate([1, 17, 64, 100, 129, 300]):
        q, k, v, do = inputs.gen_qkv((1 + i % 2, 1 + i % 3, N, 256), "bf16", 1400 + 7 * i, with_do=True)
        heads = [(b, h) for b in range(q.shape[0]) for h in range(q.shape[1])]
        check_bwd_heads(q, k, v, do, causal, 256 ** -0.5, heads, f"d256 sweep N={N}")
    q, k, v, do = inputs.gen_qkv((1, 4, 1024, 256), "bf16", 1450 + causal, with_do=True)
    check_bwd_heads(q, k, v, do, causal, 256 ** -0.5, [(0, h) for h in range(4)], "d256 B1 H4 N1024")


@pytest.mark.parametrize("d", [32, 96])
@pytest.mark.parametrize("causal", [False, True])
def test_head_dims_32_96(d, causal):
    """Head dims 32 (64-byte rows) and 96 (rows padded to 128 columns in LDS), bf16:
    ragged forward sweep, backward on ragged lengths, then B=2 H=4 N=1024 on every head."""
    need_gpu()
    for i, N in enumerate(SWEEP_N):
        q, k, v = inputs.gen_qkv((1 + i % 2, 1 + i % 3, N, d), "bf16", 1500 + 7 * i + d)
        check_fwd_full(q, k, v, causal, d ** -0.5, "bf16", f"d{d} sweep N={N}")
    for i, N in enumerate([1, 65, 129, 300]):
        q, k, v, do = inputs.gen_qkv((1, 2, N, d), "bf16", 1600 + 7 * i + d, with_do=True)
        check_bwd_heads(q, k, v, do, causal, d ** -0.5, [(0, 0), (0, 1)], f"d{d} bwd N={N}")
    q, k, v, do = inputs.gen_qkv((2, 4, 1024, d), "bf16", 1650 + d + causal, with_do=True)
    check_fwd_full(q, k, v, causal, d ** -0.5, "bf16", f"d{d} B2 H4 N1024")
    check_bwd_heads(q, k, v, do, causal, d ** -0.5, [(b, h) for b in range(2) for h in range(4)],
                    f"d{d} B2 H4 N1024")


def test_max_head_slab_d256():
    """The largest head slab the ABI accepts (N*d*2 bytes just under 2^31: d = 256,
    N = 2^22 - 64, causal), so 32-bit buffer offsets reach their limit.  The oracle
    cannot hold these rows, so the inputs are built with a known answer: every key
    row is the same vector, every visible key then has the same score, and
    O_i = mean(V_0..V_i), lse_i = s q_i.k + ln(i + 1) exactly.  Checked on sampled
    rows (first, around powers of two, last) against float64 prefix sums."""
    need_gpu()
    N, d = (1 << 22) - 64, 256
    assert N * d * 2 < (1 << 31) and (N + 64) * d * 2 >= (1 << 31)
    g = torch.Generator(device="cuda").manual_seed(77)
    q = torch.randn((1, 1, N, d), device="cuda", generator=g).to(torch.bfloat16)
    krow = torch.randn((d,), device="cuda", generator=g).to(torch.bfloat16)
    k = krow.expand(1, 1, N, d).contiguous()
    v = torch.randn((1, 1, N, d), device="cuda", generator=g).to(torch.bfloat16)
    scale = d ** -0.5
    say(f"[fwd] max head slab N={N} d={d} causal ({N * d * 2} bytes per tensor)")
    o, lse = fa.forward(q, k, v, causal=True, scale=scale)
    torch.cuda.synchronize()
    rows = sorted({0, 1, 2, 63, 64, 65, 4095, 4096, (1 << 20) - 1, 1 << 20, (1 << 21) + 5, N - 65, N - 2, N - 1})
    # float64 prefix sums of V at the sampled rows, accumulated in chunks of 2^20 rows
    pref = {}
    run = torch.zeros(d, dtype=torch.float64, device="cuda")
    step = 1 << 20
    for c0 in range(0, N, step):
        blk = v[0, 0, c0:c0 + step].double()
        cs = torch.cumsum(blk, dim=0) + run
        for r in rows:
            if c0 <= r < c0 + step:
                pref[r] = cs[r - c0].clone()
        run = cs[-1].clone()
        del blk, cs
    s = f32(scale)
    got_o = host(o[0, 0, rows])
    got_l = host(lse[0, 0, rows])
    ref_o = np.stack([(pref[r] / (r + 1)).cpu().numpy() for r in rows])
    qk = (q[0, 0, rows].double() @ krow.double()).cpu().numpy()
    ref_l = s * qk + np.log(np.asarray(rows, dtype=np.float64) + 1.0)
    eo = assert_close("max slab O rows", got_o, ref_o, "bf16")
    el = assert_close("max slab lse rows", got_l, ref_l, "bf16", lse=True)
    say(f"   O max/rel {eo[0]:.2e}/{eo[1]:.2e}  lse max {el[0]:.2e}")


# ------------------------------------------------------------------ shared K/V heads

def _gqa_check(case_name, heads_b0):
    """Forward and backward of one shared-K/V-head case, checked on batch 0 for the
    K/V heads in `heads_b0` (every query head of each such group).

    dK and dV of a shared head are sums over its query heads, so they grow with
    the group (|dK| reaches ~10 at 8 query heads per K/V head, against ~1 for one
    head), and storing a value of magnitude M in bf16 alone costs up to M * 2^-9.
    Their absolute bound is therefore scaled by max(1, max|ref|); the relative L2
    bound (1e-2) is unchanged.  O, lse and dQ keep the plain bounds."""
    c = inputs.GQA_CASES[case_name]
    B, hq, hkv, N, d, causal = c["B"], c["hq"], c["hkv"], c["N"], c["d"], c["causal"]
    g = hq // hkv
    q, k, v, do = inputs.gen_gqa(B, hq, hkv, N, d, "bf16", c["seed"], with_do=True)
    say(f"[gqa] {case_name} B={B} Hq={hq} Hkv={hkv} N={N} d={d} causal={causal} K/V heads checked={heads_b0}")
    qd, kd, vd, dod = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), dev(do, "bf16")
    scale = d ** -0.5
    o, lse = fa.forward(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv = fa.backward(qd, kd, vd, o, dod, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o, lse, dq, dk, dv = (host(t) for t in (o, lse, dq, dk, dv))
    assert dk.shape == (B, hkv, N, d) and dq.shape == (B, hq, N, d)
    s = f32(scale)
    for hk in heads_b0:
        qs = slice(hk * g, (hk + 1) * g)
        sq = (slice(0, 1), qs)
        sk = (slice(0, 1), slice(hk, hk + 1))
        ro, rl = oracle.attention_forward(q[sq], k[sk], v[sk], causal, s)
        rq, rk, rv = oracle.attention_backward(q[sq], k[sk], v[sk], do[sq], causal, s)
        worst = {}
        for name, got, ref, is_lse in (("O", o[sq], ro, False), ("lse", lse[sq], rl, True), ("dQ", dq[sq], rq, False),
                                       ("dK", dk[sk], rk, False), ("dV", dv[sk], rv, False)):
            worst[name] = assert_close(f"{case_name} {name} kv head {hk}", got, ref, "bf16", lse=is_lse,
                                       magnitude_scaled=name in ("dK", "dV"))
            worst[name] = worst[name] + (float(np.abs(ref).max()),)
        say("   kv head %d: " % hk + "  ".join(f"{n} max/rel {e[0]:.2e}/{e[1]:.2e} (max|ref| {e[2]:.2f})"
                                               for n, e in worst.items()))
    # every K/V head: the gradient identities of the exact result
    assert np.abs(dk.sum(axis=2)).max() < 0.5
    dosum = do.astype(np.float64).reshape(B, hkv, g, N, d).sum(axis=(2, 3))
    assert np.abs(dv.sum(axis=2) - dosum).max() < 0.5


def test_gqa_causal_d128():
    """8 query heads per K/V head, causal, d = 128 (the paired-wave dK/dV kernel)."""
    need_gpu()
    _gqa_check("gqa_causal_b2hq32hkv4n2048d128", [0, 3])


def test_mqa_d64():
    """Multi-query attention: 16 query heads over one K/V head, d = 64."""
    need_gpu()
    _gqa_check("mqa_b2hq16hkv1n1024d64", [0])


@pytest.mark.parametrize("d", [32, 64, 96, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_sweep(d, causal):
    """Ragged lengths and group sizes 1..4 against the oracle on every head (dK and dV
    with the magnitude-scaled absolute bound, as in the cases above)."""
    need_gpu()
    for i, (N, hq, hkv) in enumerate([(1, 2, 1), (17, 4, 2), (100, 3, 1), (129, 4, 1), (200, 2, 2)]):
        q, k, v, do = inputs.gen_gqa(1 + i % 2, hq, hkv, N, d, "bf16", 1200 + 5 * i + d, with_do=True)
        qd, kd, vd, dod = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), dev(do, "bf16")
        o, lse = fa.forward(qd, kd, vd, causal=causal)
        dq, dk, dv = fa.backward(qd, kd, vd, o, dod, lse, causal=causal)
        torch.cuda.synchronize()
        s = f32(d ** -0.5)
        ro, rl = oracle.attention_forward(q, k, v, causal, s)
        rq, rk, rv = oracle.attention_backward(q, k, v, do, causal, s)
        tag = f"gqa sweep N={N} Hq={hq} Hkv={hkv}"
        say(f"[gqa] {tag} d={d} causal={causal}")
        for name, got, ref, is_lse in (("O", o, ro, False), ("lse", lse, rl, True), ("dQ", dq, rq, False),
                                       ("dK", dk, rk, False), ("dV", dv, rv, False)):
            assert_close(f"{tag} {name}", host(got), ref, "bf16", lse=is_lse, magnitude_scaled=name in ("dK", "dV"))


# ------------------------------------------------------------------ small sweeps

SWEEP_N = [1, 17, 64, 100, 128, 129, 255, 300]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_sweep(dtype, d, causal):
    need_gpu()
    for i, N in enumerate(SWEEP_N):
        B, H = (1 + i % 2, 1 + (i % 3))
        q, k, v = inputs.gen_qkv((B, H, N, d), dtype, 500 + 7 * i + d)
        check_fwd_full(q, k, v, causal, d ** -0.5, dtype, f"sweep N={N}")


def test_fwd_f32_rows_per_wave():
    """The float32 forward picks 1, 2 or 4 query rows per wave from the grid size; these launches
    select 2 (B1 H4 N1000 d64, causal) and 4 (B2 H4 N1100 d128) rows per wave (the sweeps, 1)."""
    need_gpu()
    for (B, H, N, d, causal), seed in (((1, 4, 1000, 64, True), 2201), ((2, 4, 1100, 128, False), 2202)):
        q, k, v = inputs.gen_qkv((B, H, N, d), "f32", seed)
        check_fwd_full(q, k, v, causal, d ** -0.5, "f32", f"f32 B={B} H={H} N={N} d={d}")


def test_fwd_d64_causal_key_split():
    """Causal d = 64 launches with at most 256 workgroups of 128 rows split each workgroup's
    key range over two wave pairs and merge the two partial results.  Odd and even tile
    counts, a block with an empty upper half (N <= 64), ragged ends, peaky scores (scale x4),
    and one launch just above the threshold (unsplit) for contrast."""
    need_gpu()
    cases = [((1, 2, 1000), 1.0), ((2, 3, 1000), 1.0), ((1, 1, 2047), 1.0), ((1, 2, 64), 1.0),
             ((1, 1, 65), 1.0), ((2, 2, 1500), 4.0), ((1, 1, 4096), 4.0)]
    for i, ((B, H, N), mult) in enumerate(cases):
        q, k, v = inputs.gen_qkv((B, H, N, 64), "bf16", 2100 + 5 * i)
        check_fwd_full(q, k, v, True, mult * 0.125, "bf16", f"key split B={B} H={H} N={N} scale x{mult}",
                       stress=mult != 1.0)
    # 257 workgroups of 128 rows: the unsplit kernel
    q, k, v = inputs.gen_qkv((1, 257, 128, 64), "bf16", 2190)
    check_fwd_full(q, k, v, True, 0.125, "bf16", "unsplit B=1 H=257 N=128")


def test_fwd_causal_resident_grid_orders():
    """Causal launches whose whole grid is resident at once take the snake dispatch order
    (odd rounds of each XCD's list lightest first).  Every output row against the oracle for
    grids of three full rounds per XCD (B8 H12 N1024 at d = 32, and B8 H12 N1000: ragged last
    block), two full rounds and a partial one that keeps the forward order (B8 H10 N1024 d64),
    one full and one partial round (B4 H12 N1024 d64), and a grid whose share per XCD is not
    a whole number of heads (B3 H5 N1024 d64: the plain order)."""
    need_gpu()
    cases = [(8, 12, 1024, 32), (8, 12, 1000, 64), (8, 10, 1024, 64), (4, 12, 1024, 64), (3, 5, 1024, 64)]
    for i, (B, H, N, d) in enumerate(cases):
        q, k, v = inputs.gen_qkv((B, H, N, d), "bf16", 2300 + 11 * i)
        check_fwd_full(q, k, v, True, d ** -0.5, "bf16", f"resident causal grid B={B} H={H} N={N} d={d}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_sweep(d, causal):
    need_gpu()
    for i, N in enumerate([1, 17, 64, 129, 200, 384]):
        B, H = 1, 1 + i % 2
        q, k, v, do = inputs.gen_qkv((B, H, N, d), "bf16", 900 + 3 * i + d, with_do=True)
        check_bwd_heads(q, k, v, do, causal, d ** -0.5, [(0, h) for h in range(H)], f"sweep N={N}")


# ------------------------------------------------------------------ stress / structure

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [32, 64, 96, 128, 256])
def test_growing_scores_force_rescale(causal, d):
    """Scores that rise along the keys make the running maximum move on every tile (every head
    dim: each places the rescale of the output accumulator differently)."""
    need_gpu()
    N = 1024
    q, k, v = inputs.gen_qkv((1, 2, N, d), "bf16", 77)
    ramp = np.linspace(0.0, 6.0, N, dtype=np.float32)
    q[..., 0] = 4.0
    k[..., 0] = inputs.bf16_round(ramp)[None, None, :]
    q, k = inputs.bf16_round(q), inputs.bf16_round(k)
    check_fwd_full(q, k, v, causal, 1.0, "bf16", "growing scores", stress=True)
    do = inputs.gen_qkv((1, 2, N, d), "bf16", 78)[0]
    check_bwd_heads(q, k, v, do, causal, 1.0, [(0, 0), (0, 1)], "growing scores", stress=True)


def _check_fwd_chunked(q, k, v, causal, scale, tag, stress=False):
    say(f"[fwd] {tag} shape={q.shape} kv heads={k.shape[1]} causal={causal}")
    o, lse = run_fwd(q, k, v, causal, scale, "bf16")
    ro, rl = oracle.attention_forward(q, k, v, causal, f32(scale), row_chunk=1024)
    eo = assert_close(f"{tag} O", o, ro, "bf16", magnitude_scaled=stress)
    el = assert_close(f"{tag} lse", lse, rl, "bf16", lse=True, magnitude_scaled=stress)
    say(f"   O max/rel {eo[0]:.2e}/{eo[1]:.2e}  lse max {el[0]:.2e}")


def test_fwd_d128_long_kernel_cases():
    """Head dim 128 at N >= 4096 (non-causal) and N >= 16384 (causal) runs the kernel with 64
    query rows per wave: ragged lengths (masked last tile, rows past N), shared K/V heads,
    and the causal diagonal at 16K."""
    need_gpu()
    q, k, v = inputs.gen_qkv((1, 2, 4100, 128), "bf16", 90)
    _check_fwd_chunked(q, k, v, False, 128 ** -0.5, "d128 N4100")
    q, k, v = inputs.gen_gqa(1, 4, 2, 4096, 128, "bf16", 91)
    _check_fwd_chunked(q, k, v, False, 128 ** -0.5, "d128 Hq4 Hkv2 N4096")
    q, k, v = inputs.gen_qkv((1, 1, 16390, 128), "bf16", 92)
    _check_fwd_chunked(q, k, v, True, 128 ** -0.5, "d128 N16390 causal")


@pytest.mark.parametrize("causal,N", [(False, 4096), (True, 16384)])
def test_fwd_d128_long_scores_outgrow_first_tile(causal, N):
    """The 64-rows-per-wave kernel keeps tile 0's row maximum as its reference and moves it only
    when a chunk's probabilities would pass 2^64: scores that rise by about 115 in exp2 units
    along the keys force that move several times per row."""
    need_gpu()
    q, k, v = inputs.gen_qkv((1, 1, N, 128), "bf16", 93)
    ramp = np.linspace(0.0, 20.0, N, dtype=np.float32)
    q = inputs.bf16_round(q * 0.25)
    q[..., 0] = 4.0  # score rise 4 * 20 = 80 (natural log units) along the keys
    k[..., 0] = inputs.bf16_round(ramp)[None, None, :]
    k = inputs.bf16_round(k)
    _check_fwd_chunked(q, k, v, causal, 1.0, f"d128 N{N} rising scores", stress=True)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [32, 64, 96, 128, 256])
def test_scores_overflowing_the_first_reference(causal, d):
    """The 32-rows-per-wave forward first runs with tile 0's row maximum as a fixed
    reference; scores that rise by about 173 in exp2 units along the keys overflow
    float32 in that pass, and the workgroup must redo the rows with the moving reference."""
    need_gpu()
    N = 1024
    q, k, v = inputs.gen_qkv((1, 2, N, d), "bf16", 94)
    ramp = np.linspace(0.0, 30.0, N, dtype=np.float32)
    q = inputs.bf16_round(q * 0.25)
    q[..., 0] = 4.0  # score rise 4 * 30 = 120 (natural log units) along the keys
    k[..., 0] = inputs.bf16_round(ramp)[None, None, :]
    k = inputs.bf16_round(k)
    check_fwd_full(q, k, v, causal, 1.0, "bf16", f"d{d} overflowing scores", stress=True)


def test_peaky_scale():
    need_gpu()
    q, k, v = inputs.gen_qkv((2, 2, 512, 128), "bf16", 79)
    check_fwd_full(q, k, v, True, 4 * 128 ** -0.5, "bf16", "peaky x4", stress=True)


def test_causal_row0_is_v0_exactly():
    need_gpu()
    q, k, v = inputs.gen_qkv((2, 3, 256, 64), "bf16", 80)
    o, _ = run_fwd(q, k, v, True, 0.125, "bf16")
    assert np.array_equal(o[:, :, 0], v[:, :, 0].astype(np.float64))


def test_forward_and_backward_are_deterministic():
    need_gpu()
    q, k, v, do = (dev(x, "bf16") for x in inputs.gen_qkv((2, 4, 777, 64), "bf16", 81, with_do=True))
    o1, l1 = fa.forward(q, k, v, causal=True)
    o2, l2 = fa.forward(q, k, v, causal=True)
    g1 = fa.backward(q, k, v, o1, do, l1, causal=True)
    g2 = fa.backward(q, k, v, o1, do, l1, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_gqa_decode_fp8_are_deterministic():
    """Shared-K/V-head backward (split partials + fixed-order reduction), decode (fixed-order
    merge) and the FP8 forward are bitwise reproducible run to run."""
    need_gpu()
    q, k, v, do = (dev(x, "bf16") for x in inputs.gen_gqa(1, 8, 2, 300, 128, "bf16", 82, with_do=True))
    o, lse = fa.forward(q, k, v, causal=True)
    g1 = fa.backward(q, k, v, o, do, lse, causal=True)
    g2 = fa.backward(q, k, v, o, do, lse, causal=True)
    qd, kd, vd, lens = inputs.gen_decode(4, 8, 2, 1, 2000, 128, 83, min_len=300)
    td = [dev(x, "bf16") for x in (qd, kd, vd)]
    ld = torch.from_numpy(lens).to("cuda")
    d1 = fa.decode(td[0], td[1], td[2], ld)
    d2 = fa.decode(td[0], td[1], td[2], ld)
    (q8, k8, v8), sc = inputs.gen_fp8((1, 4, 300, 128), 84, (1, 2, 300, 128))
    t8 = [torch.from_numpy(x).to("cuda") for x in (q8, k8, v8)]
    f1 = fa.forward_fp8(t8[0], t8[1], t8[2], *sc, causal=True)
    f2 = fa.forward_fp8(t8[0], t8[1], t8[2], *sc, causal=True)
    torch.cuda.synchronize()
    for a, b in list(zip(g1, g2)) + list(zip(d1, d2)) + list(zip(f1, f2)):
        assert torch.equal(a, b)


def test_golden_rational_case_fp32():
    """The hand-derived closed form of tests/golden, run through the fp32 GPU path (d padded to 64)."""
    need_gpu()
    import pins
    scale, q2, k2, v2, do2, cases = pins.load_rational_case()
    pad = lambda a: np.pad(a, ((0, 0), (0, 62)))[None, None].astype(np.float32)  # noqa: E731
    for key, causal in (("noncausal", False), ("causal", True)):
        o, lse = run_fwd(pad(q2), pad(k2), pad(v2), causal, scale, "f32")
        assert np.abs(o[0, 0, :, :2] - cases[key]["O"]).max() <= 1e-5
        assert np.abs(o[0, 0, :, 2:]).max() == 0.0
        assert np.abs(lse[0, 0] - cases[key]["lse"]).max() <= 1e-5
