"""Benchmark: one training step of exact attention (forward + backward) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
    python bench.py --calibrate-copy     (HBM counter calibration: a plain 512 MiB copy, 3 times)
    python bench.py --sustain 5 --no-cpu-baseline   (adds the socket power and GFX clock that
                                          5 s of back-to-back forwards, then backwards, settle at)

--workload also accepts the shared-K/V-head cases (query heads grouped over
fewer K/V heads), e.g. gqa_causal_b2hq32hkv4n2048d128; they are timed the same
way through fa_fwd_gqa / fa_bwd_gqa.  The decode cases (new query rows against
a key/value cache, e.g. decode_b16hq32hkv8nk8192d128) time one fa_decode call
per step and report the K/V streaming rate in GB/s against the 8 TB/s HBM peak.
The FP8 cases (E4M3 inputs with per-tensor scales, e.g. fp8_fwd_b4h16n4096d128)
time one fa_fwd_fp8 call per step against the dense FP8 matrix-core peak.

A step runs the whole path once over one batch of synthetic inputs that are
already resident in device memory: fa_fwd (O, lse) then fa_bwd (dQ, dK, dV,
recomputing the score blocks from lse).  The timed region runs the K steps'
forwards back to back and then their backwards.  Workload: the non-causal
long-sequence encoder shape B=4, H=16, N=4096, d=128 in bf16, inputs i.i.d.
N(0,1) (seeded PCG64, rounded to bf16).

Throughput counts 4*B*H*N^2*d flops for the forward (halved when causal) and
2.5x that for the backward, i.e. the minimum matrix-product work; value =
(forward + backward flops) / step time.  Per-kernel durations come from HIP
events recorded on the stream the kernels run on; fwd_ms_cold / bwd_ms_cold
repeat each launch after a 512 MiB fill that evicts L2 and the Infinity Cache.  The CPU baseline times the
float64 oracle on a bounded sample of heads of the same workload.
Prints ONE JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd/bwd TFLOP/s on 1 MI355X + % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2516.6      # 256 CU x 4096 flop/clk x 2.4 GHz, dense
PEAK_FP8_TFLOPS = 5033.2      # dense E4M3, twice the bf16 rate
PEAK_HBM_GBS = 8000.0
DEFAULT_WORKLOAD = "fwd_encoder_b4h16n4096d128"


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "fa_bwd_encoder_b4h16n4096d128_hbm_traffic.md")
BWD_SOURCES = ["exact_io_aware_49_amd/csrc/fa_bwd_bf16.hip", "exact_io_aware_49_amd/csrc/fa_device.h",
               "exact_io_aware_49_amd/csrc/fa_map.h"]
FP8_TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "fa_fwd_fp8_b4h16n4096d128_hbm_traffic.md")
FP8_SOURCES = ["exact_io_aware_49_amd/csrc/fa_fwd_fp8.hip", "exact_io_aware_49_amd/csrc/fa_device.h",
               "exact_io_aware_49_amd/csrc/fa_map.h"]
DEC_TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "decode_b16hq32hkv8nk8192d128_kernel_trace.md")
DEC_SOURCES = ["exact_io_aware_49_amd/csrc/fa_decode.hip", "exact_io_aware_49_amd/csrc/fa_device.h",
               "exact_io_aware_49_amd/csrc/fa_internal.h"]


def sources_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(profile=TRAFFIC_PROFILE, sources=BWD_SOURCES):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None if it
    is missing or the kernel sources changed since it was taken."""
    try:
        text = open(profile).read()
    except OSError:
        return None
    sha = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    tot = re.search(r"hbm_bytes_per_launch:\s*([0-9]+)", text)
    if not sha or not tot or sha.group(1) != sources_sha(sources):
        return None
    return int(tot.group(1))


def fwd_flops(B, H, N, d, causal):
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


def host_info():
    """The host the oracle runs on: usable cores, CPU model, and numpy's BLAS (vendor,
    version, threads).  The oracle runs in this one process; its matrix products use
    the BLAS threads, the rest of numpy one thread."""
    usable = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas, threads = "unknown", usable
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            blas = f"{libs[0].get('internal_api')} {libs[0].get('version')}"
            threads = int(libs[0].get("num_threads", usable))
    except Exception:
        pass
    return {"cores": threads, "usable_cores": usable, "cpu_model": model, "blas": blas,
            "parallelism": f"one process; numpy BLAS on {threads} threads, elementwise numpy on one"}


def cpu_baseline(w, budget_s: float):
    """Time the float64 oracle (forward + backward) on whole query heads until ~budget_s elapse."""
    import oracle

    B, H, N, d = w.shape
    q, k, v, do = w.inputs()
    g = H // k.shape[1]
    s = float(np.float32(w.scale))
    heads = 0
    t0 = time.perf_counter()
    for b in range(B):
        for h in range(H):
            sq = (slice(b, b + 1), slice(h, h + 1))
            sk = (slice(b, b + 1), slice(h // g, h // g + 1))
            oracle.attention_forward(q[sq], k[sk], v[sk], w.causal, s)
            oracle.attention_backward(q[sq], k[sk], v[sk], do[sq], w.causal, s)
            heads += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    flops = 3.5 * fwd_flops(1, heads, N, d, w.causal)
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        **host_info(),
        "kind": "oracle",
        "sample": f"{heads} of {B * H} query heads (B={B},H={H},N={N},d={d}), float64 numpy forward+backward, "
                  f"{dt:.1f} s wall",
    }


class _Case:
    """One benchmark workload: a named workload, or a shared-K/V-head case."""

    def __init__(self, name):
        from exact_io_aware_49_amd import inputs
        self.name = name
        if name in inputs.WORKLOADS:
            w = inputs.WORKLOADS[name]
            if w.dtype != "bf16":
                raise SystemExit(f"{name} is a {w.dtype} forward-only parity case (the tests check it); "
                                 "bench.py times bf16 forward+backward steps")
            self.B, self.H, self.N, self.d = w.shape
            self.hkv, self.causal, self.scale, self.seed = w.H, w.causal, w.scale, w.seed
        elif name in inputs.GQA_CASES:
            c = inputs.GQA_CASES[name]
            self.B, self.H, self.N, self.d = c["B"], c["hq"], c["N"], c["d"]
            self.hkv, self.causal, self.scale, self.seed = c["hkv"], c["causal"], c["d"] ** -0.5, c["seed"]
        else:
            raise SystemExit(f"unknown workload {name}")
        self.shape = (self.B, self.H, self.N, self.d)

    def inputs(self):
        from exact_io_aware_49_amd import inputs
        return inputs.gen_gqa(self.B, self.H, self.hkv, self.N, self.d, "bf16", self.seed, with_do=True)


def _time_steps(step, a, stream):
    """a.warmup untimed calls, then a.steps timed ones back to back: (wall ms per step, ms per
    step between two HIP events recorded on `stream` before the first and after the last call).
    No events between the calls: for launches of tens of microseconds, an event record per call
    would add its own time to every step."""
    import torch

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(a.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall * 1e3 / a.steps, e0.elapsed_time(e1) / a.steps


def fp8_main(a, name):
    """One fa_fwd_fp8 call per step; value = forward matrix-product flops / time."""
    import torch

    import exact_io_aware_49_amd as fa
    from exact_io_aware_49_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    fa.load_library()
    c = inputs.FP8_CASES[name]
    B, hq, hkv, N, d, causal = c["B"], c["hq"], c["hkv"], c["N"], c["d"], bool(c["causal"])
    (q8, k8, v8), sc = inputs.fp8_case_inputs(c)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    qd, kd, vd = (torch.from_numpy(x).to(dev) for x in (q8, k8, v8))
    o = torch.empty((B, hq, N, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, hq, N), dtype=torch.float32, device=dev)
    scale = d ** -0.5
    stream = torch.cuda.current_stream(dev)

    def step():
        rc = fa.fa_fwd_fp8(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), sc[0], sc[1], sc[2], o.data_ptr(),
                           lse.data_ptr(), B, hq, hkv, N, d, int(causal), scale, stream.cuda_stream)
        if rc:
            raise RuntimeError(fa.fa_status_string(rc))

    ms_per_step, launch_ms = _time_steps(step, a, stream)
    ff = fwd_flops(B, hq, N, d, causal)
    value = ff / (ms_per_step * 1e-3) / 1e12
    achieved = ff / (launch_ms * 1e-3) / 1e12
    line = {
        "metric": "attention FP8 forward TFLOP/s on 1 MI355X + % of fp8 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3",
        "data": "synthetic: i.i.d. N(0,1) from PCG64, per-tensor scaled to E4M3 codes, resident in HBM",
        "config": {"workload": name, "pass": "forward", "B": B, "Hq": hq, "Hkv": hkv, "N": N, "d": d,
                   "causal": causal, "scale": scale},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_FP8_TFLOPS, 4),
                     "traffic": measured_traffic(FP8_TRAFFIC_PROFILE, FP8_SOURCES)
                     if name == "fp8_fwd_b4h16n4096d128" else None,
                     "kernel": "fa_fwd_fp8_kernel",
                     "avg_launch_ms": round(launch_ms, 4)},
        "cpu_baseline": None,
    }
    if not a.no_cpu_baseline:
        import oracle
        s = float(np.float32(scale))
        g = hq // hkv
        heads = 0
        t0 = time.perf_counter()
        for b in range(B):
            for h in range(hq):
                sq = (slice(b, b + 1), slice(h, h + 1))
                sk = (slice(b, b + 1), slice(h // g, h // g + 1))
                oracle.attention_forward_fp8(q8[sq], k8[sk], v8[sk], sc[0], sc[1], sc[2], causal, s)
                heads += 1
                if time.perf_counter() - t0 >= a.cpu_budget:
                    break
            if time.perf_counter() - t0 >= a.cpu_budget:
                break
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": round(fwd_flops(1, heads, N, d, causal) / dt / 1e12, 4),
                                "unit": "TFLOP/s", **host_info(), "kind": "oracle",
                                "sample": f"{heads} of {B * hq} query heads, float64 numpy forward of the "
                                          f"decoded inputs, {dt:.1f} s wall"}
    print(json.dumps(line), flush=True)
    return 0


def decode_main(a, name):
    """One fa_decode call per step; value = K/V bytes of the valid cache rows / time."""
    import torch

    import exact_io_aware_49_amd as fa
    from exact_io_aware_49_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    fa.load_library()
    c = inputs.DECODE_CASES[name]
    B, hq, hkv, nq, nk, d = c["B"], c["hq"], c["hkv"], c["nq"], c["nk"], c["d"]
    q, k, v, lens = inputs.gen_decode(B, hq, hkv, nq, nk, d, c["seed"], c["min_len"])
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    qd, kd, vd = (torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in (q, k, v))
    ld = torch.from_numpy(lens).to(dev)
    o = torch.empty_like(qd)
    lse = torch.empty((B, hq, nq), dtype=torch.float32, device=dev)
    wsb = fa.fa_decode_workspace_size(B, hq, hkv, nq, nk, d, fa.FA_DTYPE_BF16)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    scale = d ** -0.5
    stream = torch.cuda.current_stream(dev)

    def step():
        rc = fa.fa_decode(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), ld.data_ptr(), o.data_ptr(), lse.data_ptr(),
                          ws.data_ptr(), wsb, B, hq, hkv, nq, nk, d, int(c["causal"]), scale, fa.FA_DTYPE_BF16,
                          stream.cuda_stream)
        if rc:
            raise RuntimeError(fa.fa_status_string(rc))

    ms_per_step, launch_ms = _time_steps(step, a, stream)
    kv_bytes = 2.0 * hkv * float(lens.astype(np.int64).sum()) * d * 2
    io_bytes = kv_bytes + 2.0 * B * hq * nq * d * 2 + B * hq * nq * 4  # + Q read, O and lse written
    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = io_bytes / (launch_ms * 1e-3) / 1e9
    line = {
        "metric": "decode K/V streaming GB/s on 1 MI355X + % of 8 TB/s HBM",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: i.i.d. N(0,1) from PCG64, rounded to bf16, resident in HBM; cache lengths seeded",
        "config": {"workload": name, "B": B, "Hq": hq, "Hkv": hkv, "Nq": nq, "Nk": nk, "d": d,
                   "causal": bool(c["causal"]), "cache_rows": int(lens.sum())},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(DEC_TRAFFIC_PROFILE, DEC_SOURCES)
                     if name == "decode_b16hq32hkv8nk8192d128" else None,
                     "kernel": "fa_decode (fa_decode_kernel + fa_decode_merge_kernel)",
                     "avg_launch_ms": round(launch_ms, 4)},
        "cpu_baseline": None,
    }
    if not a.no_cpu_baseline:
        import oracle
        t0 = time.perf_counter()
        done = 0
        rows = 0
        for b in range(B):
            oracle.attention_decode(q[b:b + 1], k[b:b + 1], v[b:b + 1], lens[b:b + 1], c["causal"],
                                    float(np.float32(scale)))
            done += 1
            rows += int(lens[b])
            if time.perf_counter() - t0 >= a.cpu_budget:
                break
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": round(2.0 * hkv * rows * d * 2 / dt / 1e9, 3), "unit": "GB/s",
                                **host_info(), "kind": "oracle",
                                "sample": f"{done} of {B} sequences, float64 numpy, {dt:.1f} s wall"}
    print(json.dumps(line), flush=True)
    return 0


def sustained(fn, seconds: float):
    """Run fn() back to back for `seconds` while sampling the socket power and the GFX
    clocks with amd-smi every 0.5 s: the clock the chip holds under this load at its
    power limit.  Returns medians over the samples taken after the first second."""
    import subprocess
    import threading

    import torch

    samples = []
    stop = threading.Event()

    def sample():
        while not stop.is_set():
            try:
                r = subprocess.run(["amd-smi", "metric", "-p", "-c"], capture_output=True, text=True, timeout=10)
                txt = r.stdout
            except (OSError, subprocess.SubprocessError):
                txt = ""
            pw = re.findall(r"SOCKET_POWER:\s+(\d+)\s*W", txt)
            ck = [int(x) for x in re.findall(r"GFX_\d+:\s+CLK:\s+(\d+)\s*MHz", txt)]
            samples.append((time.perf_counter(), int(pw[0]) if pw else None, ck))
            stop.wait(0.5)

    th = threading.Thread(target=sample, daemon=True)
    t0 = time.perf_counter()
    th.start()
    calls = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
        calls += 10
    dt = time.perf_counter() - t0
    stop.set()
    th.join()
    late = [s for s in samples if s[0] - t0 >= 1.0 and s[1] is not None and s[2]]
    if not late:
        return {"ms_per_call": round(dt * 1e3 / calls, 4), "power_w": None, "gfx_mhz": None, "samples": 0}
    return {"ms_per_call": round(dt * 1e3 / calls, 4),
            "power_w": float(np.median([s[1] for s in late])),
            "gfx_mhz": float(np.median([np.mean(s[2]) for s in late])),
            "samples": len(late)}


def calibrate_copy(mib: int = 512, reps: int = 3):
    """A plain device-to-device copy of a known size, for scaling the HBM byte counters
    (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE): each copy reads and writes exactly
    mib MiB, so counter / true bytes is the factor the kernels' counts are divided by."""
    import torch

    a = torch.ones(mib * (1 << 20) // 2, dtype=torch.bfloat16, device="cuda")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(f"copied {mib} MiB x{reps}", flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for the CPU baseline")
    ap.add_argument("--sustain", type=float, default=0.0,
                    help="after the timed steps, run the forward and then the backward back to back for this many "
                         "seconds each, sampling socket power and GFX clocks with amd-smi (reported under 'sustained')")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 512 MiB device copy three times (HBM counter calibration)")
    a = ap.parse_args(argv)
    if a.calibrate_copy:
        return calibrate_copy()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (every (batch, head) pair is "
              "independent, so a multi-GPU run would shard heads with no communication). Use --gpus 1.",
              file=sys.stderr)
        return 2

    from exact_io_aware_49_amd import inputs as _inputs
    if a.workload in _inputs.DECODE_CASES:
        return decode_main(a, a.workload)
    if a.workload in _inputs.FP8_CASES:
        return fp8_main(a, a.workload)

    import torch

    import exact_io_aware_49_amd as fa

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    fa.load_library()
    w = _Case(a.workload)
    B, H, N, d = w.shape
    hkv = w.hkv
    causal = int(w.causal)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    q, k, v, do = (torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in w.inputs())
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_bytes = fa.fa_bwd_gqa_workspace_size(B, H, hkv, N, d, fa.FA_DTYPE_BF16)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    scale = float(w.scale)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream

    def fwd():
        rc = fa.fa_fwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, hkv, N,
                           d, causal, scale, fa.FA_DTYPE_BF16, sh)
        if rc:
            raise RuntimeError(fa.fa_status_string(rc))

    def bwd():
        rc = fa.fa_bwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                           dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), ws_bytes, B, H, hkv, N, d,
                           causal, scale, fa.FA_DTYPE_BF16, sh)
        if rc:
            raise RuntimeError(fa.fa_status_string(rc))

    for _ in range(a.warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()

    # The K steps' forwards run back to back, then their backwards (every step
    # sees the same resident inputs, so the order changes no work): three HIP
    # events on the launch stream give each launch's average duration without
    # an event between every two launches, which would lengthen short ones.
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for _ in range(a.steps):
        fwd()
    ev[1].record(stream)
    for _ in range(a.steps):
        bwd()
    ev[2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    fwd_ms = ev[0].elapsed_time(ev[1]) / a.steps
    bwd_ms = ev[1].elapsed_time(ev[2]) / a.steps

    # cold caches (reported beside the warm figures, not part of `value`): a 512 MiB
    # fill evicts L2 and the 256 MB Infinity Cache before each timed launch
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold = {"fwd": [], "bwd": []}
    for _ in range(5):
        for name, fn in (("fwd", fwd), ("bwd", bwd)):
            flush.zero_()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            cold[name].append(e0.elapsed_time(e1))
    del flush
    fwd_ms_cold = float(np.median(cold["fwd"]))
    bwd_ms_cold = float(np.median(cold["bwd"]))
    ms_per_step = wall * 1e3 / a.steps
    ff = fwd_flops(B, H, N, d, w.causal)
    bf = 2.5 * ff
    value = (ff + bf) / (ms_per_step * 1e-3) / 1e12
    fwd_tf = ff / (fwd_ms * 1e-3) / 1e12
    bwd_tf = bf / (bwd_ms * 1e-3) / 1e12

    # dominant by time: the backward launch (two kernels) or the forward kernel
    if bwd_ms >= fwd_ms:
        dkdv = "fa_bwd_dkdv_pair_kernel" if d == 128 else "fa_bwd_dkdv_kernel"
        dom = {"kernel": f"fa_bwd (fa_bwd_dq_kernel + {dkdv})", "flops": bf, "ms": bwd_ms}
    else:
        dom = {"kernel": "fa_fwd_bf16_kernel", "flops": ff, "ms": fwd_ms}
    achieved = dom["flops"] / (dom["ms"] * 1e-3) / 1e12
    traffic = measured_traffic() if dom["kernel"].startswith("fa_bwd") and w.name == DEFAULT_WORKLOAD else None
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic, "kernel": dom["kernel"],
                "avg_launch_ms": round(dom["ms"], 4)}

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: i.i.d. N(0,1) from PCG64, rounded to bf16, resident in HBM",
        "config": {"workload": w.name, "pass": "forward+backward", "B": B, "H": H, "N": N, "d": d,
                   "causal": bool(w.causal), "scale": scale, **({"Hkv": hkv} if hkv != H else {})},
        "fwd_ms": round(fwd_ms, 4),
        "bwd_ms": round(bwd_ms, 4),
        "fwd_ms_cold": round(fwd_ms_cold, 4),
        "bwd_ms_cold": round(bwd_ms_cold, 4),
        "fwd_tflops": round(fwd_tf, 2),
        "fwd_frac_of_peak": round(fwd_tf / PEAK_BF16_TFLOPS, 4),
        "bwd_tflops": round(bwd_tf, 2),
        "bwd_frac_of_peak": round(bwd_tf / PEAK_BF16_TFLOPS, 4),
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if a.sustain > 0:
        line["sustained"] = {"fwd": sustained(fwd, a.sustain), "bwd": sustained(bwd, a.sustain)}
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, a.cpu_budget)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
