#!/usr/bin/env python3
"""Benchmark of the fused attention forward (default) or backward on one MI355X.

Forward: one step = one attn_fwd launch over the headline workload: non-causal
MHA, B=2, N=16384, 16 heads, d=128, bf16 inputs (seeded synthetic N(0,1) data
already resident in HBM).  TFLOPS = 4*B*H*N^2*D / time (halved for causal).

Backward (--op bwd): one step = one attn_bwd call (the dQ kernel, then the
dK/dV kernel) on the same workload, with O and LSE from the forward and a
seeded N(0,1) dO.  TFLOPS = 10*B*H*N^2*D / time (halved for causal).

Decode (--op decode): one step = one attn_decode call (the split kernel, then
the merge kernel) on a decode workload: M new query rows per head against an
L-key cache, seeded N(0,1) data resident in HBM.  GB/s = algorithmic bytes
(K and V read once, Q read once, O and LSE written once) / time.

Varlen (--op varlen): one step = one attn_fwd_varlen launch over a packed batch
of variable-length sequences, optionally with a sliding window.  TFLOPS =
4*D*(allowed (row, key) pairs) / time.

FP8 (--op fp8): one step = one attn_fwd_fp8 launch over the FP8 counterpart of
the headline workload (e4m3 Q, K, V with per-tensor descales, bf16 O).  TFLOPS
= 4*B*H*N^2*D / time (halved for causal), against the dense FP8 MFMA peak.

Block-sparse (--op sparse): one step = one attn_fwd_blocksparse launch with a
local + global + random pattern of 128 x 128 blocks.  TFLOPS = 4*D*(allowed
(row, key) pairs) / time.

Prints ONE JSON line on stdout, with the roofline of the dominant kernel and
the oracle's CPU rate on a bounded sample as a reported baseline.

  python bench.py [--op fwd|bwd|decode|varlen|fp8|sparse] [--steps K] [--warmup W] [--workload NAME]
                  [--sweep] [--no-cpu-baseline]

``--sweep`` also times every workload of the catalogue and prints a table on
stderr (stdout stays one JSON line); its times come from one event pair around
about 150 ms of launches issued back to back.  Only one GPU is supported: --gpus > 1
exits with a message.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synth  # noqa: E402

METRIC = "attention fwd TFLOPS (bf16, d=128) and % of MI355X dense BF16 MFMA peak"
METRIC_VARLEN = ("packed variable-length attention fwd TFLOPS (bf16, d=128; 4*D per allowed "
                 "(row, key) pair) and % of MI355X dense BF16 MFMA peak")
METRIC_DECODE = "decode attention HBM GB/s (bf16, d=128) and % of MI355X HBM bandwidth"
PEAK_HBM_GBS = 8000.0
METRIC_BWD = ("attention bwd TFLOPS (bf16, d=128; 10*B*H*N^2*D flops) and % of MI355X "
              "dense BF16 MFMA peak")
# MI355X dense bf16 MFMA peak: 256 CUs x 4096 flop/clk/CU (v_mfma 32x32x16 bf16:
# 32768 flop per 32 clocks per SIMD, 4 SIMDs) x 2.4 GHz = 2516.6 TFLOP/s.
PEAK_TFLOPS = 256 * 4096 * 2.4e9 / 1e12
# dense e4m3 MFMA peak: v_mfma_scale 32x32x64 f8 does 131072 flop per 64 clocks
# per SIMD, twice the bf16 rate: 5033.2 TFLOP/s.
PEAK_FP8_TFLOPS = 2 * PEAK_TFLOPS
METRIC_SPARSE = ("block-sparse attention fwd TFLOPS (bf16, d=128, 128 x 128 blocks; 4*D per allowed "
                 "(row, key) pair) and % of MI355X dense BF16 MFMA peak")
METRIC_FP8 = ("attention fwd TFLOPS (FP8 e4m3 Q/K/V with per-tensor descales, bf16 O, d=128) "
              "and % of MI355X dense FP8 MFMA peak")
CSRC = os.path.join(ROOT, "scaled_dot_product_17_amd", "csrc")
KERNEL_SRC = os.path.join(CSRC, "attn_fwd.hip")
BWD_SRC = os.path.join(CSRC, "attn_bwd.hip")
DECODE_SRC = os.path.join(CSRC, "attn_decode.hip")
FP8_SRC = os.path.join(CSRC, "attn_fwd_fp8.hip")
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), for the CPU baselines."""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads() -> int:
    import oracle
    return oracle.default_threads()


def pmap(fn, items, threads):
    """fn over items on `threads` host threads (the oracle's C calls release the
    GIL, so disjoint pieces of a sample run on all cores)."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        return list(ex.map(fn, items))


def kernel_hash(src: str = KERNEL_SRC) -> str:
    with open(src, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def stored_traffic(workload: str, kernel: str = "attn_fwd", src: str = KERNEL_SRC):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, f"hbm_traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for ln in f:
            if ":" in ln and not ln.lstrip().startswith("#"):
                key, val = ln.split(":", 1)
                kv[key.strip()] = val.strip()
    if kv.get("kernel_source_sha256_16") != kernel_hash(src):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def profile_record(workload: str, tag: str, src: str, work: float, peak: float,
                   unit_scale: float = 1e12):
    """The committed rocprofv3 kernel-trace summary of a workload, if it was taken
    on the current kernel source: its file, dominant kernel, that kernel's mean
    duration, and the rate and fraction of peak that duration gives for `work`
    (flops or bytes per launch; rate = work / s / unit_scale); else None."""
    path = os.path.join(PROFILES, f"kernel_trace_{tag}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for ln in f:
            if ":" in ln and not ln.startswith((" ", "#")):
                key, val = ln.split(":", 1)
                kv[key.strip()] = val.strip()
    if kv.get("kernel_source_sha256_16") != kernel_hash(src):
        return None
    try:
        ms = float(kv["dominant_kernel_avg_ns"]) * 1e-6
        step_ms = float(kv.get("step_kernels_avg_ns", kv["dominant_kernel_avg_ns"])) * 1e-6
    except (KeyError, ValueError):
        return None
    rate = work / (ms * 1e-3) / unit_scale
    return {"file": os.path.relpath(path, ROOT), "kernel": kv.get("dominant_kernel"),
            "kernel_ms_mean": round(ms, 5), "step_kernels_ms_mean": round(step_ms, 5),
            "achieved": round(rate, 2), "frac": round(rate / peak, 4),
            "bench_in_same_session": kv.get("bench_in_same_session")}


def upload(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def time_workload(w, steps, warmup):
    """Returns (ms_per_step wall, mean launch ms from HIP events, per-launch
    list): the first two from the K launches issued back to back between two
    synchronizations (an event pair around them on the launch stream), the
    list from a second loop with an event pair around every launch."""
    import torch
    import scaled_dot_product_17_amd as sdpa
    q, k, v = w.generate()
    qg, kg, vg = upload(q), upload(k), upload(v)
    del q, k, v
    o = torch.empty_like(qg)
    lse = torch.empty((w.B, w.H_q, w.N), dtype=torch.float32, device=qg.device)
    for _ in range(warmup):
        sdpa.fwd(qg, kg, vg, causal=w.causal, scale=w.scale, out=o, lse=lse)
    stream = torch.cuda.current_stream()
    ms_step, per, mean = _event_loop(
        lambda: sdpa.fwd(qg, kg, vg, causal=w.causal, scale=w.scale, out=o, lse=lse), steps, stream)
    assert bool(torch.isfinite(lse).all()), "non-finite LSE in the benchmark output"
    del qg, kg, vg, o, lse
    torch.cuda.empty_cache()
    return ms_step, mean, per


def cpu_baseline(w, target_s: float = 12.0):
    """The oracle as it stands, on this host's cores, over a bounded sample of
    query rows of the same workload; rate in the metric's unit (TFLOPS)."""
    import oracle
    oracle.build(force=False)
    q, k, v = w.generate()
    threads = oracle.default_threads()
    rng = np.random.default_rng(1)
    total_rows = w.B * w.H_q * w.N

    def run(n):
        rows = np.sort(rng.choice(total_rows, n, replace=False)).astype(np.int64)
        t0 = time.perf_counter()
        oracle.attn_ref(q, k, v, w.causal, w.scale, rows=rows, n_threads=threads)
        dt = time.perf_counter() - t0
        i = rows % w.N
        keys = (i + 1) if w.causal else np.full(n, w.N)
        return dt, float(keys.sum()) * 4 * w.D   # 4*D flops per allowed pair
    n0 = max(threads, 32)
    dt, fl = run(n0)
    n = int(min(total_rows, max(n0, n0 * target_s / max(dt, 1e-3))))
    dt, fl = run(n)
    return {"value": fl / dt / 1e12, "unit": "TFLOPS", "cores": threads, "cpu": cpu_model(),
            "kind": "oracle",
            "sample": f"{n} random query rows of {w.name} (all {w.N} keys each, fp64), "
                      f"{dt:.1f} s"}


def bwd_inputs(w):
    """Device tensors of the backward step: q, k, v, dO, and O, LSE from attn_fwd."""
    import torch
    import scaled_dot_product_17_amd as sdpa
    q, k, v = w.generate()
    do = synth.normal_bf16(w.seed_base + 3, q.shape)
    qg, kg, vg, dog = upload(q), upload(k), upload(v), upload(do)
    del q, k, v, do
    o, lse = sdpa.fwd(qg, kg, vg, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    return qg, kg, vg, dog, o, lse


def time_back_to_back(w, target_ms: float = 150.0) -> float:
    """Mean kernel time (ms) of a workload from one HIP event pair around
    launches issued back to back on the launch stream (b2b).  A pair of events
    around every launch would also count the host's time between launches once
    a kernel is shorter than the Python call that enqueues it."""
    import torch
    import scaled_dot_product_17_amd as sdpa
    q, k, v = w.generate()
    qg, kg, vg = upload(q), upload(k), upload(v)
    del q, k, v
    o = torch.empty_like(qg)
    lse = torch.empty((w.B, w.H_q, w.N), dtype=torch.float32, device=qg.device)
    ms = b2b(lambda: sdpa.fwd(qg, kg, vg, causal=w.causal, scale=w.scale, out=o, lse=lse),
             torch.cuda.current_stream(), target_ms)
    del qg, kg, vg, o, lse
    torch.cuda.empty_cache()
    return ms


def b2b(fn, stream, target_ms: float = 150.0) -> float:
    """Mean time (ms) of fn's GPU work from one HIP event pair around calls
    issued back to back, about target_ms of work after a warm-up of the same
    length (see time_back_to_back)."""
    import torch

    def run(n):
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        b0.record(stream)
        for _ in range(n):
            fn()
        b1.record(stream)
        torch.cuda.synchronize()
        return b0.elapsed_time(b1) / n

    n = max(5, int(target_ms / max(run(3), 1e-3)))
    run(n)
    return run(n)


def _event_loop(fn, steps, stream):
    """Times `steps` calls of fn: (wall ms per call, per-call HIP event times in
    ms, mean ms per call from one event pair on the stream).  The timed region
    is the K calls issued back to back between two synchronizations, with one
    event pair around them (the wall time and the event mean both come from
    it); the per-call times come from a second loop with an event pair around
    every call, which adds microseconds between short kernels, so they only
    give the spread."""
    import torch
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    b0.record(stream)
    for _ in range(steps):
        fn()
    b1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        fn()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return wall * 1e3 / steps, [a.elapsed_time(b) for a, b in ev], b0.elapsed_time(b1) / steps


def time_bwd(w, steps, warmup):
    """Whole backward steps, then each of its two kernels alone (HIP events on
    the stream they run on).  Returns a dict of timings in ms."""
    import torch
    import scaled_dot_product_17_amd as sdpa
    qg, kg, vg, dog, o, lse = bwd_inputs(w)
    dq, dk, dv = torch.empty_like(qg), torch.empty_like(kg), torch.empty_like(vg)
    delta = torch.empty_like(lse)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    args = (w.B, w.H_q, w.H_kv, w.N, w.D, w.causal, w.scale, sp)

    def step():
        sdpa.bwd(qg, kg, vg, o, lse, dog, causal=w.causal, scale=w.scale, dq=dq, dk=dk, dv=dv,
                 delta=delta)

    def k_dq():
        st = sdpa.attn_bwd_dq(qg.data_ptr(), kg.data_ptr(), vg.data_ptr(), o.data_ptr(),
                              dog.data_ptr(), lse.data_ptr(), dq.data_ptr(), delta.data_ptr(),
                              *args)
        assert st == 0, st

    def k_dkdv():
        st = sdpa.attn_bwd_dkdv(qg.data_ptr(), kg.data_ptr(), vg.data_ptr(), dog.data_ptr(),
                                lse.data_ptr(), delta.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                *args)
        assert st == 0, st

    for _ in range(warmup):
        step()
    ms_step, per, _ = _event_loop(step, steps, stream)
    ks = max(3, steps // 2)
    _, per_dq, mean_dq = _event_loop(k_dq, ks, stream)
    _, per_kv, mean_kv = _event_loop(k_dkdv, ks, stream)
    for t in (dq, dk, dv):
        assert bool(torch.isfinite(t.float()).all()), "non-finite gradient in the benchmark"
    del qg, kg, vg, dog, o, lse, dq, dk, dv, delta
    torch.cuda.empty_cache()
    return {"ms_step": ms_step, "ms_event": float(np.mean(per)),
            "dq": mean_dq, "dkdv": mean_kv,
            "dq_p10_p90": [float(np.percentile(per_dq, 10)), float(np.percentile(per_dq, 90))],
            "dkdv_p10_p90": [float(np.percentile(per_kv, 10)), float(np.percentile(per_kv, 90))]}


def bwd_pairs(w) -> float:
    """Allowed (query, key) pairs of the workload, by the benchmark convention
    (N^2 per head, halved when causal)."""
    return w.B * w.H_q * float(w.N) * w.N * (0.5 if w.causal else 1.0)


def cpu_baseline_bwd(w):
    """The backward oracle as it stands, on this host's cores, over one K/V head
    of the same workload (with every query head of its group, all rows and keys):
    rate in the metric's unit (10*D flops per allowed pair)."""
    import oracle
    oracle.build(force=False)
    q, k, v = w.generate()
    do = synth.normal_bf16(w.seed_base + 3, q.shape)
    g = w.H_q // w.H_kv
    sl = (slice(0, 1), slice(0, g))
    threads = oracle.default_threads()
    t0 = time.perf_counter()
    oracle.attn_bwd_ref(q[sl], k[0:1, 0:1], v[0:1, 0:1], do[sl], w.causal, w.scale,
                        n_threads=threads)
    dt = time.perf_counter() - t0
    pairs = g * (w.N * (w.N + 1) / 2 if w.causal else float(w.N) * w.N)
    return {"value": pairs * 10 * w.D / dt / 1e12, "unit": "TFLOPS", "cores": threads,
            "cpu": cpu_model(), "kind": "oracle",
            "sample": f"full fp64 backward of batch 0, K/V head 0 ({g} query head(s), all "
                      f"{w.N} rows and keys) of {w.name}, {dt:.1f} s"}


def main_bwd(args, w):
    import scaled_dot_product_17_amd as sdpa
    log(f"[bench bwd] {w.name}: B={w.B} H_q={w.H_q} H_kv={w.H_kv} N={w.N} D={w.D} "
        f"causal={w.causal}")
    t = time_bwd(w, args.steps, args.warmup)
    flops = 10 * w.D * bwd_pairs(w)
    tflops = flops / (t["ms_step"] * 1e-3) / 1e12
    # per-kernel MFMA work: dQ kernel S, dP, dQ (6*D per pair); dK/dV kernel
    # S, dP, dV, dK (8*D per pair)
    kflops = {"dq": 6 * w.D * bwd_pairs(w), "dkdv": 8 * w.D * bwd_pairs(w)}
    dom = max(("dq", "dkdv"), key=lambda n: t[n])
    achieved = kflops[dom] / (t[dom] * 1e-3) / 1e12
    log(f"[bench bwd] {t['ms_step']:.3f} ms/step wall ({t['ms_event']:.3f} events): dQ kernel "
        f"{t['dq']:.3f} ms, dK/dV kernel {t['dkdv']:.3f} ms; {tflops:.1f} TFLOPS = "
        f"{100 * tflops / PEAK_TFLOPS:.1f}% of peak")
    traffic = stored_traffic(w.name, f"attn_bwd_{dom}", BWD_SRC)
    res = {
        "metric": METRIC_BWD, "value": round(tflops, 2), "unit": "TFLOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(t["ms_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16, SplitMix64 + Box-Muller)",
        "pct_of_peak": round(100 * tflops / PEAK_TFLOPS, 2),
        "config": {"workload": w.name, "op": "bwd", "B": w.B, "H_q": w.H_q, "H_kv": w.H_kv,
                   "N": w.N, "D": w.D, "causal": w.causal, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": round(PEAK_TFLOPS, 1), "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_TFLOPS, 4), "traffic": traffic,
                     "kernel": f"attn_bwd_{dom}_kernel",
                     "launch_ms_mean": round(t[dom], 4),
                     "launch_ms_p10_p90": [round(x, 4) for x in t[f"{dom}_p10_p90"]],
                     "profile": profile_record(w.name, "attn_bwd", BWD_SRC, kflops["dkdv"],
                                               PEAK_TFLOPS)},
        "kernels_ms": {"attn_bwd_dq_kernel": round(t["dq"], 4),
                       "attn_bwd_dkdv_kernel": round(t["dkdv"], 4)},
        "cpu_baseline": None,
    }
    if args.sweep:
        # ms: the whole step as sdpa.bwd runs it (its dK/dV step split over
        # `parts` of each group's query heads when the library chooses to);
        # dkdv(1): the unsplit dK/dV kernel alone
        log(f"{'workload':36s} {'ms':>9s} {'TFLOPS':>9s} {'%peak':>7s} {'parts':>5s} {'dq ms':>8s} "
            f"{'dkdv(1) ms':>10s}")
        for name, x in synth.WORKLOADS.items():
            tt = time_bwd(x, max(5, args.steps // 5), 3)
            parts = sdpa.attn_bwd_splits(x.B, x.H_q, x.H_kv, x.N, x.D, x.causal)
            tf = 10 * x.D * bwd_pairs(x) / (tt["ms_step"] * 1e-3) / 1e12
            log(f"{name:36s} {tt['ms_step']:9.3f} {tf:9.1f} {100 * tf / PEAK_TFLOPS:7.1f} "
                f"{parts:5d} {tt['dq']:8.3f} {tt['dkdv']:10.3f}")
    if not args.no_cpu_baseline:
        log("[bench bwd] timing the backward oracle on a bounded sample ...")
        res["cpu_baseline"] = cpu_baseline_bwd(w)
    print(json.dumps(res), flush=True)


def time_decode(w, steps, warmup):
    """Whole decode steps, then the split kernel alone (HIP events on the stream
    they run on).  Returns a dict of timings in ms and the split count."""
    import torch
    import scaled_dot_product_17_amd as sdpa
    q, k, v = w.generate()
    qg, kg, vg = upload(q), upload(k), upload(v)
    del q, k, v
    S = sdpa.attn_decode_splits(w.B, w.H_q, w.H_kv, w.M, w.L, w.D, 0)
    ws = torch.empty(sdpa.attn_decode_workspace_bytes(w.B, w.H_q, w.H_kv, w.M, w.L, w.D, 0),
                     dtype=torch.uint8, device=qg.device)
    o = torch.empty_like(qg)
    lse = torch.empty((w.B, w.H_q, w.M), dtype=torch.float32, device=qg.device)
    rows = w.B * w.H_q * w.M
    op = torch.empty((rows, S, w.D), dtype=torch.float32, device=qg.device)
    lp = torch.empty((rows, S), dtype=torch.float32, device=qg.device)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    args = (qg.data_ptr(), kg.data_ptr(), vg.data_ptr(), o.data_ptr(), lse.data_ptr(), w.B,
            w.H_q, w.H_kv, w.M, w.L, w.D, w.causal, w.scale, 0, ws.data_ptr(), ws.numel(), sp)

    def step():
        # the raw C-ABI call: its host cost (a few microseconds) stays well under
        # the kernels' time, so the GPU never waits for the next launch
        st = sdpa.attn_decode(*args)
        assert st == 0, st

    def split():
        st = sdpa.attn_decode_partial(qg.data_ptr(), kg.data_ptr(), vg.data_ptr(), op.data_ptr(),
                                      lp.data_ptr(), w.B, w.H_q, w.H_kv, w.M, w.L, w.D, w.causal,
                                      w.scale, S, sp)
        assert st == 0, st

    for _ in range(warmup):
        step()
    ms_step, per, _ = _event_loop(step, steps, stream)
    _, per_split, mean_split = _event_loop(split, steps, stream)
    assert bool(torch.isfinite(lse).all()), "non-finite LSE in the benchmark output"
    del qg, kg, vg, o, lse, ws, op, lp
    torch.cuda.empty_cache()
    return {"ms_step": ms_step, "ms_event": float(np.mean(per)),
            "split": mean_split,
            "split_p10_p90": [float(np.percentile(per_split, 10)),
                              float(np.percentile(per_split, 90))], "n_splits": S}


def cpu_baseline_decode(w, target_s: float = 10.0):
    """The decode oracle as it stands, on all host cores (one call per
    (batch entry, K/V head) slice at a time per core): rate in the metric's unit
    (algorithmic bytes of the workload per second)."""
    import oracle
    oracle.build(force=False)
    q, k, v = w.generate()
    threads = host_threads()
    g = w.H_q // w.H_kv
    slices = [(b, kv) for b in range(w.B) for kv in range(w.H_kv)]

    def one(bk):
        b, kv = bk
        oracle.attn_decode_ref(q[b:b + 1, kv * g:(kv + 1) * g], k[b:b + 1, kv:kv + 1],
                               v[b:b + 1, kv:kv + 1], w.causal, w.scale)
    reps, t0 = 0, time.perf_counter()
    while True:   # the whole workload, repeated to about 10 s of CPU work
        pmap(one, slices, threads)
        reps += 1
        dt = time.perf_counter() - t0
        if dt > target_s:
            break
    return {"value": reps * w.bytes / dt / 1e9, "unit": "GB/s", "cores": threads, "cpu": cpu_model(),
            "kind": "oracle",
            "sample": f"fp64 decode of the whole {w.name} workload ({len(slices)} (batch, K/V head) "
                      f"slices over {threads} threads), {reps} time(s), {dt:.1f} s"}


def decode_split_bytes(w, n_splits: int):
    """(read, write) algorithmic bytes of one split-kernel launch: K, V and Q read
    once; each split's partial O and LSE written once."""
    rows = w.B * w.H_q * w.M
    return (2 * w.B * w.H_kv * w.L * w.D * 2 + w.B * w.H_q * w.M * w.D * 2,
            rows * n_splits * (w.D + 1) * 4)


def main_decode(args, w):
    import scaled_dot_product_17_amd as sdpa
    log(f"[bench decode] {w.name}: B={w.B} H_q={w.H_q} H_kv={w.H_kv} M={w.M} L={w.L} D={w.D} "
        f"causal={w.causal}")
    t = time_decode(w, args.steps, args.warmup)
    gbs = w.bytes / (t["ms_step"] * 1e-3) / 1e9
    split_bytes = sum(decode_split_bytes(w, t["n_splits"]))
    achieved = split_bytes / (t["split"] * 1e-3) / 1e9
    log(f"[bench decode] {t['ms_step'] * 1e3:.1f} us/step ({t['n_splits']} splits): "
        f"{gbs:.0f} GB/s = {100 * gbs / PEAK_HBM_GBS:.1f}% of HBM; split kernel "
        f"{t['split'] * 1e3:.1f} us, {achieved:.0f} GB/s")
    traffic = stored_traffic(w.name, "attn_decode_split", DECODE_SRC)
    res = {
        "metric": METRIC_DECODE, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(t["ms_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16, SplitMix64 + Box-Muller)",
        "pct_of_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
        "tflops": round(w.flops / (t["ms_step"] * 1e-3) / 1e12, 2),
        "config": {"workload": w.name, "op": "decode", "B": w.B, "H_q": w.H_q, "H_kv": w.H_kv,
                   "M": w.M, "L": w.L, "D": w.D, "causal": w.causal, "n_splits": t["n_splits"],
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic, "kernel": "attn_decode_split_kernel",
                     "launch_ms_mean": round(t["split"], 5),
                     "launch_ms_p10_p90": [round(x, 5) for x in t["split_p10_p90"]],
                     "profile": profile_record(w.name, "attn_decode", DECODE_SRC, split_bytes,
                                               PEAK_HBM_GBS, 1e9)},
        "cpu_baseline": None,
    }
    if args.sweep:
        log(f"{'workload':40s} {'us':>8s} {'GB/s':>8s} {'%HBM':>6s} {'splits':>6s}")
        for name, x in synth.DECODE_WORKLOADS.items():
            tt = time_decode(x, max(5, args.steps // 5), 3)
            g = x.bytes / (tt["ms_step"] * 1e-3) / 1e9
            log(f"{name:40s} {tt['ms_step'] * 1e3:8.1f} {g:8.0f} {100 * g / PEAK_HBM_GBS:6.1f} "
                f"{tt['n_splits']:6d}")
    if not args.no_cpu_baseline:
        log("[bench decode] timing the decode oracle on a bounded sample ...")
        res["cpu_baseline"] = cpu_baseline_decode(w)
    print(json.dumps(res), flush=True)


def main_varlen(args, w):
    import torch
    import scaled_dot_product_17_amd as sdpa
    log(f"[bench varlen] {w.name}: H_q={w.H_q} H_kv={w.H_kv} total={w.total} "
        f"sequences={len(w.lengths())} causal={w.causal} window=({w.left}, {w.right})")
    q, k, v = w.generate()
    qg, kg, vg = upload(q), upload(k), upload(v)
    del q, k, v
    cu = torch.from_numpy(w.cu_seqlens()).cuda()
    max_len = int(w.lengths().max())
    o = torch.empty_like(qg)
    lse = torch.empty((w.H_q, w.total), dtype=torch.float32, device=qg.device)
    stream = torch.cuda.current_stream()
    a = (qg.data_ptr(), kg.data_ptr(), vg.data_ptr(), o.data_ptr(), lse.data_ptr(), cu.data_ptr(),
         len(w.lengths()), max_len, w.total, w.H_q, w.H_kv, w.D, w.causal, w.left, w.right,
         w.scale, stream.cuda_stream)

    def step():
        st = sdpa.attn_fwd_varlen(*a)
        assert st == 0, st

    for _ in range(args.warmup):
        step()
    ms_step, per, mean = _event_loop(step, args.steps, stream)
    assert bool(torch.isfinite(lse).all()), "non-finite LSE in the benchmark output"
    tflops = w.flops / (ms_step * 1e-3) / 1e12
    achieved = w.flops / (mean * 1e-3) / 1e12
    log(f"[bench varlen] {ms_step:.3f} ms/step: {tflops:.1f} TFLOPS = "
        f"{100 * tflops / PEAK_TFLOPS:.1f}% of peak")
    res = {
        "metric": METRIC_VARLEN, "value": round(tflops, 2), "unit": "TFLOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 and seeded sequence lengths)",
        "pct_of_peak": round(100 * tflops / PEAK_TFLOPS, 2),
        "config": {"workload": w.name, "op": "varlen", "H_q": w.H_q, "H_kv": w.H_kv,
                   "total": w.total, "sequences": len(w.lengths()), "causal": w.causal,
                   "window": [w.left, w.right], "D": w.D, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(PEAK_TFLOPS, 1),
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS, 4),
                     "traffic": stored_traffic(w.name, "attn_fwd_varlen"), "kernel": "attn_fwd_kernel<varlen>",
                     "launch_ms_mean": round(mean, 4),
                     "launch_ms_p10_p90": [round(float(np.percentile(per, 10)), 4),
                                           round(float(np.percentile(per, 90)), 4)],
                     "profile": profile_record(w.name, "attn_fwd_varlen", KERNEL_SRC, w.flops,
                                               PEAK_TFLOPS)},
        "cpu_baseline": None,
    }
    if args.sweep:
        log(f"{'workload':40s} {'ms':>8s} {'TFLOPS':>8s} {'%peak':>6s}")
        for name, x in synth.VARLEN_WORKLOADS.items():
            qq, kk, vv = x.generate()
            qx, kx, vx = upload(qq), upload(kk), upload(vv)
            cx = torch.from_numpy(x.cu_seqlens()).cuda()
            ox = torch.empty_like(qx)
            lx = torch.empty((x.H_q, x.total), dtype=torch.float32, device=qx.device)
            ax = (qx.data_ptr(), kx.data_ptr(), vx.data_ptr(), ox.data_ptr(), lx.data_ptr(),
                  cx.data_ptr(), len(x.lengths()), int(x.lengths().max()), x.total, x.H_q, x.H_kv,
                  x.D, x.causal, x.left, x.right, x.scale, stream.cuda_stream)
            fn = lambda: sdpa.attn_fwd_varlen(*ax)
            for _ in range(3):
                fn()
            ms = b2b(fn, stream)
            tf = x.flops / (ms * 1e-3) / 1e12
            log(f"{name:40s} {ms:8.3f} {tf:8.1f} {100 * tf / PEAK_TFLOPS:6.1f}")
    if not args.no_cpu_baseline:
        log("[bench varlen] timing the varlen oracle on a bounded sample ...")
        res["cpu_baseline"] = cpu_baseline_varlen(w)
    print(json.dumps(res), flush=True)


def cpu_baseline_varlen(w, target_s: float = 10.0):
    """The varlen oracle as it stands, on all host cores: (sequence, query head)
    pieces, sequences from the shortest up and every query head of each, one
    piece per thread and as many pieces at a time as threads (pieces of one
    sequence are equal work), until about 10 s of CPU work; rate in the
    metric's unit (4*D flops per allowed pair)."""
    import oracle
    oracle.build(force=False)
    q, k, v = w.generate()
    cu = w.cu_seqlens()
    lens = np.diff(cu)
    g = w.H_q // w.H_kv
    threads = host_threads()
    pieces = [(int(s), h) for s in np.argsort(lens, kind="stable") for h in range(w.H_q)]

    def run(piece):
        s, h = piece
        a, b = int(cu[s]), int(cu[s + 1])
        hk = h // g
        cu1 = np.array([0, b - a], np.int32)
        oracle.attn_varlen_ref(q[h:h + 1, a:b], k[hk:hk + 1, a:b], v[hk:hk + 1, a:b], cu1,
                               w.causal, w.scale, w.left, w.right)
        return synth.VarlenWorkload("s", 1, 1, b - a, b - a, b - a, w.causal, w.left, w.right).pairs

    done_pairs, t0, n_done, busiest = 0, time.perf_counter(), 0, 0
    while n_done < len(pieces) and time.perf_counter() - t0 <= target_s:
        chunk = pieces[n_done:n_done + threads]
        done_pairs += sum(pmap(run, chunk, threads))
        n_done += len(chunk)
        busiest = max(busiest, len(chunk))
    dt = time.perf_counter() - t0
    seqs = sorted({int(lens[s]) for s, _ in pieces[:n_done]})
    return {"value": done_pairs * 4 * w.D / dt / 1e12, "unit": "TFLOPS", "cores": busiest,
            "cpu": cpu_model(), "kind": "oracle",
            "sample": f"fp64 oracle on {n_done} (sequence, query head) pieces of {w.name} "
                      f"({w.H_q} query heads; sequence lengths {seqs}), "
                      f"{busiest} pieces at a time on {busiest} threads, {dt:.1f} s"}


def main_sparse(args, w):
    import torch
    import scaled_dot_product_17_amd as sdpa
    ptr, idx = w.csr()
    log(f"[bench sparse] {w.name}: B={w.B} H_q={w.H_q} H_kv={w.H_kv} N={w.N} causal={w.causal} "
        f"lists={len(ptr) - 1} entries={len(idx)} density={w.pairs() / (w.B * w.H_q * w.N * w.N):.4f}")
    q, k, v = w.generate()
    qg, kg, vg = upload(q), upload(k), upload(v)
    del q, k, v
    pg = torch.from_numpy(ptr).cuda()
    ig = torch.from_numpy(idx).cuda()
    o = torch.empty_like(qg)
    lse = torch.empty((w.B, w.H_q, w.N), dtype=torch.float32, device=qg.device)
    stream = torch.cuda.current_stream()
    mh = (len(ptr) - 1) // (-(-w.N // w.block))
    a = (qg.data_ptr(), kg.data_ptr(), vg.data_ptr(), o.data_ptr(), lse.data_ptr(), pg.data_ptr(),
         ig.data_ptr(), len(idx), mh, w.B, w.H_q, w.H_kv, w.N, w.D, w.causal, w.scale,
         stream.cuda_stream)

    def step():
        st = sdpa.attn_fwd_blocksparse(*a)
        assert st == 0, st

    for _ in range(args.warmup):
        step()
    ms_step, per, mean = _event_loop(step, args.steps, stream)
    assert bool(torch.isfinite(lse).all()), "non-finite LSE in the benchmark output"
    tflops = w.flops / (ms_step * 1e-3) / 1e12
    achieved = w.flops / (mean * 1e-3) / 1e12
    log(f"[bench sparse] {ms_step:.3f} ms/step: {tflops:.1f} TFLOPS = "
        f"{100 * tflops / PEAK_TFLOPS:.1f}% of peak")
    res = {
        "metric": METRIC_SPARSE, "value": round(tflops, 2), "unit": "TFLOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 and a seeded block pattern)",
        "pct_of_peak": round(100 * tflops / PEAK_TFLOPS, 2),
        "config": {"workload": w.name, "op": "sparse", "B": w.B, "H_q": w.H_q, "H_kv": w.H_kv,
                   "N": w.N, "D": w.D, "causal": w.causal, "block": w.block,
                   "pattern": {"local": w.local, "global": w.n_global, "random": w.n_random,
                               "per_head": w.per_head},
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(PEAK_TFLOPS, 1),
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS, 4),
                     "traffic": stored_traffic(w.name, "attn_fwd_blocksparse"),
                     "kernel": "attn_fwd_kernel<sparse>", "launch_ms_mean": round(mean, 4),
                     "launch_ms_p10_p90": [round(float(np.percentile(per, 10)), 4),
                                           round(float(np.percentile(per, 90)), 4)],
                     "profile": profile_record(w.name, "attn_fwd_blocksparse", KERNEL_SRC,
                                               w.flops, PEAK_TFLOPS)},
        "cpu_baseline": None,
    }
    if args.sweep:
        log(f"{'workload':46s} {'ms':>8s} {'TFLOPS':>8s} {'%peak':>6s}")
        for name, x in synth.SPARSE_WORKLOADS.items():
            qq, kk, vv = x.generate()
            xp, xi = x.csr()
            qx, kx, vx = upload(qq), upload(kk), upload(vv)
            px, ix = torch.from_numpy(xp).cuda(), torch.from_numpy(xi).cuda()
            ox = torch.empty_like(qx)
            lx = torch.empty((x.B, x.H_q, x.N), dtype=torch.float32, device=qx.device)
            mhx = (len(xp) - 1) // (-(-x.N // x.block))
            ax = (qx.data_ptr(), kx.data_ptr(), vx.data_ptr(), ox.data_ptr(), lx.data_ptr(),
                  px.data_ptr(), ix.data_ptr(), len(xi), mhx, x.B, x.H_q, x.H_kv, x.N, x.D,
                  x.causal, x.scale, stream.cuda_stream)
            fn = lambda: sdpa.attn_fwd_blocksparse(*ax)
            for _ in range(3):
                fn()
            ms = b2b(fn, stream)
            tf = x.flops / (ms * 1e-3) / 1e12
            log(f"{name:46s} {ms:8.3f} {tf:8.1f} {100 * tf / PEAK_TFLOPS:6.1f}")
    if not args.no_cpu_baseline:
        log("[bench sparse] timing the block-sparse oracle on a bounded sample ...")
        res["cpu_baseline"] = cpu_baseline_sparse(w)
    print(json.dumps(res), flush=True)


def cpu_baseline_sparse(w, target_s: float = 10.0):
    """The block-sparse oracle as it stands, on all host cores (disjoint row
    chunks), over a bounded sample of query rows; rate in the metric's unit
    (4*D flops per allowed pair)."""
    import oracle
    oracle.build(force=False)
    q, k, v = w.generate()
    ptr, idx = w.csr()
    lists = w.lists()
    nb = -(-w.N // w.block)
    rng = np.random.default_rng(3)
    total_rows = w.B * w.H_q * w.N

    def pairs_of(rows):
        n = 0
        for r in rows:
            i, h = int(r % w.N), int((r // w.N) % w.H_q)
            for kb in lists[(h if w.per_head else 0) * nb + i // w.block]:
                k0, k1 = kb * w.block, min(w.N, (kb + 1) * w.block)
                n += max(0, min(k1, i + 1) - k0) if w.causal else k1 - k0
        return n

    threads = host_threads()

    def run(n):
        rows = np.sort(rng.choice(total_rows, n, replace=False)).astype(np.int64)
        parts = [p for p in np.array_split(rows, threads) if p.size]
        t0 = time.perf_counter()
        pmap(lambda r: oracle.attn_blocksparse_ref(q, k, v, ptr, idx, w.block, w.causal, w.scale,
                                                   rows=r), parts, threads)
        return time.perf_counter() - t0, pairs_of(rows) * 4.0 * w.D
    dt, fl = run(16 * threads)
    n = int(min(total_rows, max(16 * threads, 16 * threads * target_s / max(dt, 1e-3))))
    dt, fl = run(n)
    return {"value": fl / dt / 1e12, "unit": "TFLOPS", "cores": threads, "cpu": cpu_model(),
            "kind": "oracle",
            "sample": f"{n} random query rows of {w.name} (their listed keys, fp64, {threads} "
                      f"threads), {dt:.1f} s"}


def main_fp8(args, w):
    import torch
    import scaled_dot_product_17_amd as sdpa
    log(f"[bench fp8] {w.name}: B={w.B} H_q={w.H_q} H_kv={w.H_kv} N={w.N} D={w.D} "
        f"causal={w.causal} descales=({w.descale_q:.6g}, {w.descale_k:.6g}, {w.descale_v:.6g})")
    q8, k8, v8 = w.generate()
    qg, kg, vg = (torch.from_numpy(x).cuda() for x in (q8, k8, v8))
    del q8, k8, v8
    o = torch.empty((w.B, w.H_q, w.N, w.D), dtype=torch.bfloat16, device=qg.device)
    lse = torch.empty((w.B, w.H_q, w.N), dtype=torch.float32, device=qg.device)
    stream = torch.cuda.current_stream()
    a = (qg.data_ptr(), kg.data_ptr(), vg.data_ptr(), o.data_ptr(), lse.data_ptr(), w.B, w.H_q,
         w.H_kv, w.N, w.D, w.causal, w.scale, w.descale_q, w.descale_k, w.descale_v,
         stream.cuda_stream)

    def step():
        st = sdpa.attn_fwd_fp8(*a)
        assert st == 0, st

    for _ in range(args.warmup):
        step()
    ms_step, per, mean = _event_loop(step, args.steps, stream)
    assert bool(torch.isfinite(lse).all()), "non-finite LSE in the benchmark output"
    tflops = w.flops / (ms_step * 1e-3) / 1e12
    achieved = w.flops / (mean * 1e-3) / 1e12
    log(f"[bench fp8] {ms_step:.3f} ms/step: {tflops:.1f} TFLOPS = "
        f"{100 * tflops / PEAK_FP8_TFLOPS:.1f}% of the FP8 peak "
        f"({100 * tflops / PEAK_TFLOPS:.1f}% of the bf16 peak)")
    res = {
        "metric": METRIC_FP8, "value": round(tflops, 2), "unit": "TFLOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "e4m3",
        "data": "synthetic (seeded N(0,1) rounded to e4m3 with a per-tensor descale)",
        "pct_of_peak": round(100 * tflops / PEAK_FP8_TFLOPS, 2),
        "config": {"workload": w.name, "op": "fp8", "B": w.B, "H_q": w.H_q, "H_kv": w.H_kv,
                   "N": w.N, "D": w.D, "causal": w.causal, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": round(PEAK_FP8_TFLOPS, 1), "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_FP8_TFLOPS, 4),
                     "traffic": stored_traffic(w.name, "attn_fwd_fp8", FP8_SRC),
                     "kernel": "attn_fwd_fp8_kernel", "launch_ms_mean": round(mean, 4),
                     "launch_ms_p10_p90": [round(float(np.percentile(per, 10)), 4),
                                           round(float(np.percentile(per, 90)), 4)],
                     "profile": profile_record(w.name, "attn_fwd_fp8", FP8_SRC, w.flops,
                                               PEAK_FP8_TFLOPS)},
        "cpu_baseline": None,
    }
    if args.sweep:
        log(f"{'workload':40s} {'ms':>8s} {'TFLOPS':>8s} {'%fp8peak':>8s}")
        for name, x in synth.FP8_WORKLOADS.items():
            xs = [torch.from_numpy(t).cuda() for t in x.generate()]
            ox = torch.empty((x.B, x.H_q, x.N, x.D), dtype=torch.bfloat16, device=qg.device)
            lx = torch.empty((x.B, x.H_q, x.N), dtype=torch.float32, device=qg.device)
            ax = (xs[0].data_ptr(), xs[1].data_ptr(), xs[2].data_ptr(), ox.data_ptr(),
                  lx.data_ptr(), x.B, x.H_q, x.H_kv, x.N, x.D, x.causal, x.scale, x.descale_q,
                  x.descale_k, x.descale_v, stream.cuda_stream)
            fn = lambda: sdpa.attn_fwd_fp8(*ax)
            for _ in range(3):
                fn()
            ms = b2b(fn, stream)
            tf = x.flops / (ms * 1e-3) / 1e12
            log(f"{name:40s} {ms:8.3f} {tf:8.1f} {100 * tf / PEAK_FP8_TFLOPS:8.1f}")
    if not args.no_cpu_baseline:
        log("[bench fp8] timing the FP8 oracle on a bounded sample ...")
        res["cpu_baseline"] = cpu_baseline_fp8(w)
    print(json.dumps(res), flush=True)


def cpu_baseline_fp8(w, target_s: float = 10.0):
    """The FP8 oracle as it stands, on all host cores (disjoint row chunks), over
    a bounded sample of query rows of the same workload; rate in the metric's
    unit (4*D flops per pair)."""
    import oracle
    oracle.build(force=False)
    q8, k8, v8 = w.generate()
    rng = np.random.default_rng(2)
    total_rows = w.B * w.H_q * w.N

    threads = host_threads()

    def run(n):
        rows = np.sort(rng.choice(total_rows, n, replace=False)).astype(np.int64)
        parts = [p for p in np.array_split(rows, threads) if p.size]
        t0 = time.perf_counter()
        pmap(lambda r: oracle.attn_fp8_ref(q8, k8, v8, w.descale_q, w.descale_k, w.descale_v,
                                           w.causal, w.scale, rows=r), parts, threads)
        dt = time.perf_counter() - t0
        i = rows % w.N
        keys = (i + 1) if w.causal else np.full(n, w.N)
        return dt, float(keys.sum()) * 4 * w.D
    dt, fl = run(4 * threads)
    n = int(min(total_rows, max(4 * threads, 4 * threads * target_s / max(dt, 1e-3))))
    dt, fl = run(n)
    return {"value": fl / dt / 1e12, "unit": "TFLOPS", "cores": threads, "cpu": cpu_model(),
            "kind": "oracle",
            "sample": f"{n} random query rows of {w.name} (all allowed keys each, fp64, "
                      f"{threads} threads), {dt:.1f} s"}


# ------------------------------------------------------------------ profiles
# Summaries under profiles/ are written from rocprofv3 csv output by
# ``bench.py --summarize-profile DIR --op OP [--workload W]``.  DIR holds the
# output of these runs, all of the same op and workload, taken one after the
# other in one session on the GPU (commands from the repository root):
#   bench.json       python3 bench.py --op OP --workload W > DIR/bench.json
#   kt/              rocprofv3 --kernel-trace --stats --output-format csv -d DIR/kt -o run
#                      -- python3 bench.py --op OP --workload W --no-cpu-baseline --no-configs
#   FETCH_SIZE/ WRITE_SIZE/ sqA/ sqB/ sqC/  (optional)
#                    rocprofv3 --pmc <counters> --kernel-include-regex RX --output-format csv
#                      -d DIR/<name> -o run -- python3 bench.py --op OP --workload W --steps 3
#                      --warmup 1 --no-cpu-baseline --no-configs
#   copy_FETCH_SIZE/ copy_WRITE_SIZE/  (with FETCH_SIZE/WRITE_SIZE)
#                    rocprofv3 --pmc FETCH_SIZE|WRITE_SIZE --output-format csv -d DIR/copy_<c>
#                      -o run -- python3 bench.py --calibrate-copy 1024
SQ_SETS = {
    "sqA": "SQ_VALU_MFMA_BUSY_CYCLES SQ_ACTIVE_INST_VALU SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT "
           "SQ_ACTIVE_INST_LDS SQ_BUSY_CYCLES GRBM_GUI_ACTIVE",
    "sqB": "SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_INSTS_VALU_TRANS_F32 SQ_WAVE_CYCLES "
           "SQ_WAIT_INST_LDS GRBM_GUI_ACTIVE",
    "sqC": "SQ_VALU_MFMA_COEXEC_CYCLES SQ_WAIT_INST_ANY SQ_WAIT_ANY SQ_ACTIVE_INST_ANY "
           "SQ_INSTS_SALU SQ_ACTIVE_INST_MISC GRBM_GUI_ACTIVE",
}


def kernel_key(name: str) -> str:
    """'void (anonymous namespace)::k<a, b>((anonymous namespace)::P)' -> 'k<a, b>'."""
    s = name.replace("(anonymous namespace)::", "")
    if s.startswith("void "):
        s = s[5:]
    i = s.find("(")
    return s[:i] if i > 0 else s


def template_args(key: str):
    i, j = key.find("<"), key.rfind(">")
    return [a.strip() for a in key[i + 1:j].split(",")] if 0 <= i < j else []


def profile_spec(op: str, w):
    """What the summaries of one op measure: the kernel source, the include
    regex of the counter runs, the step's kernels (predicates on kernel keys),
    the dominant kernel's algorithmic work per launch, and the algorithmic bytes
    of each kernel whose HBM traffic is summarised."""
    def fwd_kind(varlen, sparse):
        def pred(safe):
            return lambda k: (k.startswith("attn_fwd_kernel<")
                              and template_args(k)[1:3] == [str(varlen).lower(), str(sparse).lower()]
                              and template_args(k)[4] == str(safe).lower())
        return pred(False), pred(True)
    if op in ("fwd", "varlen", "sparse"):
        fast, exact = fwd_kind(op == "varlen", op == "sparse")
        step = [("fast", fast), ("exact (non-finite V check)", exact)]
    if op == "fwd":
        qkv = w.B * (w.H_q + 2 * w.H_kv) * w.N * w.D * 2
        wr = w.B * w.H_q * w.N * (w.D * 2 + 4)
        return dict(tag="attn_fwd", src=KERNEL_SRC, rx="attn_fwd_kernel", step=step,
                    desc=f"{'causal' if w.causal else 'non-causal'} B={w.B}, H_q={w.H_q}, "
                         f"H_kv={w.H_kv}, N={w.N}, D={w.D}, bf16",
                    work=w.flops, unit="TFLOP/s", scale=1e12, peak=PEAK_TFLOPS,
                    traffic=[("", fast, qkv, wr, "(Q, K, V read once; O, LSE written once)")],
                    sq=(fast, w.flops / (4 * w.D) / (32 * 32), "wave x 32-key-block"))
    if op == "fp8":
        fast = lambda k: k.startswith("attn_fwd_fp8_kernel<") and template_args(k)[2] == "false"
        exact = lambda k: k.startswith("attn_fwd_fp8_kernel<") and template_args(k)[2] == "true"
        qkv = w.B * (w.H_q + 2 * w.H_kv) * w.N * w.D
        wr = w.B * w.H_q * w.N * (w.D * 2 + 4)
        return dict(tag="attn_fwd_fp8", src=FP8_SRC, rx="attn_fwd_fp8", desc=(
                    f"{'causal' if w.causal else 'non-causal'} B={w.B}, H_q={w.H_q}, H_kv={w.H_kv}, "
                    f"N={w.N}, D={w.D}, e4m3 Q/K/V, bf16 O"),
                    step=[("fast", fast), ("exact (non-finite V check)", exact)],
                    work=w.flops, unit="TFLOP/s", scale=1e12, peak=PEAK_FP8_TFLOPS,
                    traffic=[("", fast, qkv, wr, "(e4m3 Q, K, V read once; bf16 O and fp32 LSE "
                                                 "written once)")],
                    sq=(fast, w.flops / (4 * w.D) / (32 * 64), "wave x 64-key-block"))
    if op == "varlen":
        lens = w.lengths()
        rd = (w.H_q + 2 * w.H_kv) * w.total * w.D * 2 + (len(lens) + 1) * 4
        wr = w.H_q * w.total * (w.D * 2 + 4)
        return dict(tag="attn_fwd_varlen", src=KERNEL_SRC, rx="attn_fwd_kernel", step=step,
                    desc=f"packed {'causal ' if w.causal else ''}varlen, H_q={w.H_q}, H_kv={w.H_kv}, "
                         f"{w.total} tokens in {len(lens)} sequences, window ({w.left}, {w.right}), "
                         f"D={w.D}, bf16",
                    work=4 * w.D * w.pairs, unit="TFLOP/s", scale=1e12, peak=PEAK_TFLOPS,
                    traffic=[("", fast, rd, wr, "(Q, K, V and cu_seqlens read once; O and LSE "
                                                "written once)")], sq=None)
    if op == "sparse":
        ptr, idx = w.csr()
        rd = w.B * (w.H_q + 2 * w.H_kv) * w.N * w.D * 2 + 4 * (len(ptr) + len(idx))
        wr = w.B * w.H_q * w.N * (w.D * 2 + 4)
        return dict(tag="attn_fwd_blocksparse", src=KERNEL_SRC, rx="attn_fwd_kernel", step=step,
                    desc=f"block-sparse B={w.B}, H_q={w.H_q}, H_kv={w.H_kv}, N={w.N}, D={w.D}, "
                         f"{w.block}x{w.block} blocks ({w.local} local, {w.n_global} global, "
                         f"{w.n_random} random per query block), bf16",
                    work=4 * w.D * w.pairs(), unit="TFLOP/s", scale=1e12, peak=PEAK_TFLOPS,
                    traffic=[("", fast, rd, wr, "(Q read once; every K and V block is listed by "
                                                "some query block, so K and V once; the block "
                                                "lists once; O and LSE written once)")], sq=None)
    if op == "decode":
        split = lambda k: k.startswith("attn_decode_split_kernel")
        merge = lambda k: k.startswith("attn_lse_merge_kernel")
        return dict(tag="attn_decode", src=DECODE_SRC, rx="attn_decode_split",
                    desc=f"decode B={w.B}, H_q={w.H_q}, H_kv={w.H_kv}, M={w.M}, L={w.L}, D={w.D}, "
                         f"bf16",
                    step=[("split", split), ("merge", merge)], work=None, unit="GB/s", scale=1e9,
                    peak=PEAK_HBM_GBS, traffic=None, sq=None)
    if op == "bwd":
        dq = lambda k: k.startswith("attn_bwd_dq_kernel")
        dkdv = lambda k: k.startswith("attn_bwd_dkdv_kernel")
        tq = w.B * w.H_q * w.N * w.D * 2
        tkv = w.B * w.H_kv * w.N * w.D * 2
        r4 = w.B * w.H_q * w.N * 4
        return dict(tag="attn_bwd", src=BWD_SRC, rx="attn_bwd",
                    desc=f"{'causal' if w.causal else 'non-causal'} B={w.B}, H_q={w.H_q}, "
                         f"H_kv={w.H_kv}, N={w.N}, D={w.D}, bf16",
                    step=[("dkdv", dkdv), ("dq", dq)], work=8 * w.D * bwd_pairs(w),
                    unit="TFLOP/s", scale=1e12, peak=PEAK_TFLOPS,
                    traffic=[("_dq", dq, 3 * tq + 2 * tkv + r4, tq + r4,
                              "(reads Q, K, V, O, dO, LSE once; writes dQ, delta once)"),
                             ("_dkdv", dkdv, 2 * tq + 2 * tkv + 2 * r4, 2 * tkv,
                              "(reads Q, dO, K, V, LSE, delta once; writes dK, dV once)")],
                    sq=(dkdv, bwd_pairs(w) / (32 * 32), "wave-pair x 32x32-sub-block"))
    raise ValueError(op)


def _csv_one(d, pattern):
    import glob
    f = glob.glob(os.path.join(d, "**", pattern), recursive=True)
    if not f:
        raise FileNotFoundError(f"no {pattern} under {d}")
    return f[0]


def _per_dispatch(d, pred):
    """{counter: [value per dispatch]} over the dispatches whose kernel key satisfies pred."""
    import csv
    acc = {}
    with open(_csv_one(d, "run_counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            if not pred(kernel_key(r["Kernel_Name"])):
                continue
            key = (r["Dispatch_Id"], r["Counter_Name"])
            acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (_, c), v in acc.items():
        out.setdefault(c, []).append(v)
    return out


def summarize_profile(d: str, op: str, w) -> list:
    """Writes the profiles/ summaries of one profiling session (see above);
    returns the files written."""
    import csv
    import statistics
    sp = profile_spec(op, w)
    h = kernel_hash(sp["src"])
    tag, name = sp["tag"], w.name
    wl = f"--op {op} --workload {name}"
    pmc_cmd = f"bench.py {wl} --steps 3 --warmup 1 --no-cpu-baseline --no-configs"
    with open(os.path.join(d, "bench.json")) as f:
        bench = json.loads([ln for ln in f.read().splitlines() if ln.startswith("{")][-1])
    written = []
    if op == "decode":
        rd_alg, wr_alg = decode_split_bytes(w, int(bench["config"]["n_splits"]))
        sp["work"] = rd_alg + wr_alg
        sp["traffic"] = [("_split", sp["step"][0][1], rd_alg, wr_alg,
                          f"(K, V, Q read once; partial O and LSE of {bench['config']['n_splits']} "
                          f"splits written once)")]

    # kernel trace
    rows = []
    with open(_csv_one(os.path.join(d, "kt"), "run_kernel_stats.csv")) as f:
        for r in csv.DictReader(f):
            rows.append((kernel_key(r["Name"]), r))
    step_avg = {}
    for label, pred in sp["step"]:
        hit = [r for k, r in rows if pred(k)]
        if hit:
            calls = sum(int(r["Calls"]) for r in hit)
            step_avg[label] = (sum(float(r["AverageNs"]) * int(r["Calls"]) for r in hit) / calls,
                               [k for k, r in rows if pred(k)], calls)
    dom_label = sp["step"][0][0]
    if dom_label not in step_avg:
        raise RuntimeError(f"the dominant kernel of {op} is not in the kernel trace")
    dom_ns, dom_keys, dom_calls = step_avg[dom_label]
    step_ns = sum(v[0] for v in step_avg.values())
    rf = bench.get("roofline", {})
    L = [f"# rocprofv3 kernel-trace summary of bench.py {wl}: {sp['desc']}.",
         "# Commands, from the repository root on the GPU, one after the other in one session:",
         f"#   python3 bench.py {wl} > <dir>/bench.json",
         f"#   cd /tmp && TMPDIR=/tmp rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/kt "
         f"-o run -- python3 <repo>/bench.py {wl} --no-cpu-baseline --no-configs",
         f"#   python3 bench.py --summarize-profile <dir> {wl}",
         f"kernel_source_sha256_16: {h}",
         f"dominant_kernel: {' | '.join(dom_keys)}",
         f"dominant_kernel_avg_ns: {dom_ns:.0f}",
         f"dominant_kernel_calls: {dom_calls}"]
    for label, (ns, keys, calls) in step_avg.items():
        if label != dom_label:
            L.append(f"other_step_kernel: {label}: {' | '.join(keys)}: avg_ns {ns:.0f}, calls {calls}")
    L.append(f"step_kernels_avg_ns: {step_ns:.0f}")
    if sp["work"]:
        rate = sp["work"] / (dom_ns * 1e-9) / sp["scale"]
        L.append(f"dominant_kernel_rate: {rate:.2f} {sp['unit']} = {rate / sp['peak']:.4f} of "
                 f"{sp['peak']:.1f} ({sp['work']:.6g} algorithmic units per launch)")
    L.append(f"bench_in_same_session: value={bench.get('value')} {bench.get('unit')}, "
             f"ms_per_step={bench.get('ms_per_step')}, launch_ms_mean={rf.get('launch_ms_mean')}, "
             f"frac={rf.get('frac')}")
    L.append("kernel stats (all kernels of the rocprofv3 run):")
    for k, r in rows:
        L.append(f"  {k if len(k) <= 100 else k[:97] + '...'}")
        L.append(f"    calls={r['Calls']} avg_ns={float(r['AverageNs']):.0f} min_ns={r['MinNs']} "
                 f"max_ns={r['MaxNs']} pct={float(r['Percentage']):.2f}")
    out = os.path.join(PROFILES, f"kernel_trace_{tag}_{name}.txt")
    with open(out, "w") as f:
        f.write("\n".join(L) + "\n")
    written.append(out)

    # HBM traffic
    if sp["traffic"] and os.path.isdir(os.path.join(d, "FETCH_SIZE")):
        fc = _per_dispatch(os.path.join(d, "copy_FETCH_SIZE"), lambda k: "copyBuffer" in k)["FETCH_SIZE"]
        wc = _per_dispatch(os.path.join(d, "copy_WRITE_SIZE"), lambda k: "copyBuffer" in k)["WRITE_SIZE"]
        fs, ws = 1024 * 1024 / statistics.median(fc), 1024 * 1024 / statistics.median(wc)
        for suffix, pred, rd_alg, wr_alg, note in sp["traffic"]:
            fa = _per_dispatch(os.path.join(d, "FETCH_SIZE"), pred)["FETCH_SIZE"]
            wa = _per_dispatch(os.path.join(d, "WRITE_SIZE"), pred)["WRITE_SIZE"]
            fr, wr = statistics.mean(fa), statistics.mean(wa)
            rd, wt = fr * 1024 * fs, wr * 1024 * ws
            alg = rd_alg + wr_alg
            L = [f"# HBM traffic per launch of the {tag}{suffix} kernel (fast path) of bench.py {wl}: "
                 f"{sp['desc']}.",
                 f"# rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per dispatch, one counter per run), each "
                 f"scaled by what the same counter reads for a plain 1 GiB device-to-device copy.",
                 "# Commands, from the repository root on the GPU, in one session:",
                 f"#   cd /tmp && TMPDIR=/tmp rocprofv3 --pmc FETCH_SIZE --kernel-include-regex {sp['rx']} "
                 f"--output-format csv -d <dir>/FETCH_SIZE -o run -- python3 <repo>/{pmc_cmd}",
                 f"#   cd /tmp && TMPDIR=/tmp rocprofv3 --pmc WRITE_SIZE --kernel-include-regex {sp['rx']} "
                 f"--output-format csv -d <dir>/WRITE_SIZE -o run -- python3 <repo>/{pmc_cmd}",
                 "#   cd /tmp && TMPDIR=/tmp rocprofv3 --pmc FETCH_SIZE --output-format csv -d "
                 "<dir>/copy_FETCH_SIZE -o run -- python3 <repo>/bench.py --calibrate-copy 1024",
                 "#   cd /tmp && TMPDIR=/tmp rocprofv3 --pmc WRITE_SIZE --output-format csv -d "
                 "<dir>/copy_WRITE_SIZE -o run -- python3 <repo>/bench.py --calibrate-copy 1024",
                 f"#   python3 bench.py --summarize-profile <dir> {wl}",
                 f"kernel_source_sha256_16: {h}",
                 f"fetch_kib_per_dispatch_raw: {fr:.1f}   (dispatches: {len(fa)}, min {min(fa):.1f}, "
                 f"max {max(fa):.1f})",
                 f"write_kib_per_dispatch_raw: {wr:.1f}   (dispatches: {len(wa)})",
                 f"copy_1GiB_fetch_kib_raw: {statistics.median(fc):.1f}   -> fetch scale {fs:.4f}",
                 f"copy_1GiB_write_kib_raw: {statistics.median(wc):.1f}   -> write scale {ws:.4f}",
                 f"hbm_read_bytes_per_launch: {rd:.0f}",
                 f"hbm_write_bytes_per_launch: {wt:.0f}",
                 f"hbm_bytes_per_launch: {rd + wt:.0f}",
                 f"algorithmic_bytes_per_launch: {alg}   {note}",
                 f"traffic_over_algorithmic: {(rd + wt) / alg:.3f}   (reads {rd / rd_alg:.3f}x, "
                 f"writes {wt / wr_alg:.3f}x the algorithmic bytes)"]
            out = os.path.join(PROFILES, f"hbm_traffic_{tag}{suffix}_{name}.txt")
            with open(out, "w") as f:
                f.write("\n".join(L) + "\n")
            written.append(out)

    # SQ counters
    if sp["sq"] and all(os.path.isdir(os.path.join(d, s)) for s in SQ_SETS):
        pred, units, unit_desc = sp["sq"]
        sq = {}
        for s in SQ_SETS:
            for k, v in _per_dispatch(os.path.join(d, s), pred).items():
                if k == "GRBM_GUI_ACTIVE" and k in sq:
                    continue
                sq[k] = statistics.mean(v)
        el = sq["GRBM_GUI_ACTIVE"] / 8
        tot = el * 1024
        mf = sq["SQ_INSTS_MFMA"]
        ms = dom_ns * 1e-6
        L = [f"# rocprofv3 SQ counters per dispatch of the {tag} kernel (fast path) of bench.py {wl}: "
             f"{sp['desc']}.",
             "# Three passes of 7 counters each, from the repository root on the GPU, in one session:",
             f"#   cd /tmp && TMPDIR=/tmp rocprofv3 --pmc <set> --kernel-include-regex {sp['rx']} "
             f"--output-format csv -d <dir>/<set> -o run -- python3 <repo>/{pmc_cmd}"]
        L += [f"#   {k}: {v}" for k, v in SQ_SETS.items()]
        L += [f"#   python3 bench.py --summarize-profile <dir> {wl}",
              f"kernel_source_sha256_16: {h}", "raw (summed over the device):"]
        L += [f"  {k}: {sq[k]:.4g}" for k in sorted(sq)]
        L += [f"derived (GRBM_GUI_ACTIVE is summed over the 8 XCDs; 1024 SIMDs; {units:.0f} "
              f"{unit_desc} units per launch):",
              f"  elapsed cycles per XCD: {el:.4g}   (over the {ms:.3f} ms mean of the kernel trace: "
              f"about {el / (ms * 1e-3) / 1e9:.2f} GHz)",
              f"  MFMA busy / (elapsed x SIMDs): {100 * sq['SQ_VALU_MFMA_BUSY_CYCLES'] / tot:.1f}%   "
              f"(MFMA instructions per launch {mf:.4g})",
              f"  VALU active / (elapsed x SIMDs): {100 * 4 * sq['SQ_ACTIVE_INST_VALU'] / tot:.1f}%   "
              f"(SQ_ACTIVE_INST_VALU counts 4-cycle units)",
              f"  MFMA+VALU co-execution / MFMA busy: "
              f"{100 * sq['SQ_VALU_MFMA_COEXEC_CYCLES'] / sq['SQ_VALU_MFMA_BUSY_CYCLES']:.1f}%",
              f"  waves waiting (waitcnt or barrier) / wave cycles: "
              f"{100 * sq['SQ_WAIT_ANY'] / sq['SQ_WAVE_CYCLES']:.1f}%",
              f"  per {unit_desc} unit: {sq['SQ_INSTS_VALU'] / units:.1f} VALU instructions "
              f"({mf / units:.1f} of them MFMA), {sq['SQ_INSTS_VALU_TRANS_F32'] / units:.1f} "
              f"transcendental, {sq['SQ_INSTS_LDS'] / units:.1f} LDS, "
              f"{sq['SQ_INSTS_SALU'] / units:.1f} SALU",
              f"  LDS bank conflicts: {sq['SQ_LDS_BANK_CONFLICT']:.0f}; LDS busy "
              f"{100 * sq['SQ_LDS_IDX_ACTIVE'] / (el * 256):.1f}% of CU cycles"]
        out = os.path.join(PROFILES, f"sq_counters_{tag}_{name}.txt")
        with open(out, "w") as f:
            f.write("\n".join(L) + "\n")
        written.append(out)
    return written


def workload_of(args):
    """The workload an op runs: --workload, else the op's headline workload."""
    table, default = {
        "fwd": (synth.WORKLOADS, synth.HEADLINE), "bwd": (synth.WORKLOADS, synth.HEADLINE),
        "decode": (synth.DECODE_WORKLOADS, synth.DECODE_HEADLINE),
        "varlen": (synth.VARLEN_WORKLOADS, "varlen_causal_h16_t32768"),
        "fp8": (synth.FP8_WORKLOADS, synth.FP8_HEADLINE),
        "sparse": (synth.SPARSE_WORKLOADS, next(iter(synth.SPARSE_WORKLOADS))),
    }[args.op]
    name = args.workload or default
    if name not in table:
        sys.exit(f"{name} is not a workload of --op {args.op}")
    return table[name]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--op", choices=("fwd", "bwd", "decode", "varlen", "fp8", "sparse"),
                    default="fwd")
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None,
                    choices=sorted(synth.WORKLOADS) + sorted(synth.DECODE_WORKLOADS)
                    + sorted(synth.VARLEN_WORKLOADS) + sorted(synth.FP8_WORKLOADS)
                    + sorted(synth.SPARSE_WORKLOADS),
                    help="default: the headline workload of the op")
    ap.add_argument("--sweep", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="forward: skip the per-config list (every forward workload timed back "
                         "to back after the headline)")
    ap.add_argument("--summarize-profile", metavar="DIR", default=None,
                    help="write the profiles/ summaries of one profiling session held in DIR "
                         "(for --op and --workload; needs no GPU) and exit")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB three times (the "
                         "known-size reference for scaling HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: there is no multi-GPU path (the heads of a "
              "step shard across GPUs with no exchange; run one process per GPU)", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        sys.exit("--steps must be >= 1 and --warmup >= 0")
    if args.summarize_profile:
        for f in summarize_profile(args.summarize_profile, args.op, workload_of(args)):
            log(f"[profile] wrote {os.path.relpath(f, ROOT)}")
        return

    import torch
    import scaled_dot_product_17_amd as sdpa
    if not torch.cuda.is_available():
        sys.exit("no GPU visible")
    if args.calibrate_copy > 0:
        n = args.calibrate_copy * (1 << 20)
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for i in range(3):
            t0 = time.perf_counter()
            dst.copy_(src)
            torch.cuda.synchronize()
            dt = time.perf_counter() - t0
            log(f"[copy] {args.calibrate_copy} MiB copy {i}: {dt * 1e3:.3f} ms, "
                f"{2 * n / dt / 1e9:.0f} GB/s read + write (wall time)")
        return
    sdpa.load()

    w = workload_of(args)
    mains = {"varlen": main_varlen, "sparse": main_sparse, "fp8": main_fp8,
             "decode": main_decode, "bwd": main_bwd}
    if args.op in mains:
        mains[args.op](args, w)
        return
    log(f"[bench] {w.name}: B={w.B} H_q={w.H_q} H_kv={w.H_kv} N={w.N} D={w.D} causal={w.causal}")
    ms_step, ms_launch, per = time_workload(w, args.steps, args.warmup)
    tflops = w.flops / (ms_step * 1e-3) / 1e12
    achieved = w.flops / (ms_launch * 1e-3) / 1e12
    log(f"[bench] {ms_step:.3f} ms/step wall, {ms_launch:.3f} ms/launch (events), "
        f"{tflops:.1f} TFLOPS = {100 * tflops / PEAK_TFLOPS:.1f}% of peak")

    traffic = stored_traffic(w.name)
    res = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16, SplitMix64 + Box-Muller)",
        "pct_of_peak": round(100 * tflops / PEAK_TFLOPS, 2),
        "config": {"workload": w.name, "B": w.B, "H_q": w.H_q, "H_kv": w.H_kv, "N": w.N,
                   "D": w.D, "causal": w.causal, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": round(PEAK_TFLOPS, 1), "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_TFLOPS, 4),
                     "traffic": traffic, "kernel": "attn_fwd_kernel",
                     "launch_ms_mean": round(ms_launch, 4),
                     "launch_ms_p10_p90": [round(float(np.percentile(per, 10)), 4),
                                           round(float(np.percentile(per, 90)), 4)],
                     "profile": profile_record(w.name, "attn_fwd", KERNEL_SRC, w.flops,
                                               PEAK_TFLOPS)},
        "configs": None,
        "cpu_baseline": None,
    }
    if not args.no_configs or args.sweep:
        # every forward workload, grouped as the five configurations of the
        # metric, timed back to back in this run after the headline
        log(f"{'config':6s} {'workload':36s} {'ms':>9s} {'TFLOPS':>9s} {'%peak':>7s}")
        res["configs"] = []
        for name, x in synth.WORKLOADS.items():
            ms = time_back_to_back(x)
            tf = x.flops / (ms * 1e-3) / 1e12
            cfg = synth.config_of(x)
            log(f"{cfg:6s} {name:36s} {ms:9.3f} {tf:9.1f} {100 * tf / PEAK_TFLOPS:7.1f}")
            res["configs"].append({"config": cfg, "workload": name, "ms": round(ms, 4),
                                   "tflops": round(tf, 2), "frac": round(tf / PEAK_TFLOPS, 4)})
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on a bounded sample ...")
        res["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
