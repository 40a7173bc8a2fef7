#!/usr/bin/env python3
"""Throughput of the fused attention forward on one MI355X.

One step = one fused forward (one kernel launch) over the whole workload with
inputs already resident in device memory.  Default workload: bf16, causal,
B=2, H=32, N=4096, d=128 (the shape the >= 50 % of MFMA peak target is set
on).  FLOPs per step follow the metric's convention: 4*B*H*N^2*d, halved for
causal.  Prints ONE JSON line.

Besides the headline number the line carries:
  roofline     -- achieved TFLOP/s of the fused kernel (algorithmic FLOPs per
                  launch / mean launch time from HIP events on the launch
                  stream) against the bf16 dense MFMA peak of 2500 TFLOP/s;
  cpu_baseline -- the fp64 oracle timed on the host cores on a bounded,
                  evenly spaced sample of the same workload's query rows,
                  scaled to TFLOP/s with the same FLOP convention;
  unfused      -- the three-kernel baseline (S and P through device memory)
                  timed the same way;
  workloads    -- the other bf16 workloads, fused, timed the same way;
  backward     -- the backward pass (fa_bwd_bf16: three launches) on the same
                  workload with a seeded dO, timed the same way, with its own
                  roofline (nominal backward FLOPs 10*B*H*N^2*d, halved for
                  causal, per call / mean call time) and its own oracle
                  baseline (the full fp64 backward of a few heads);
  decode       -- decode over a paged key/value cache (fa_decode_paged_bf16: two
                  launches) on the decode workload, HBM-bound: achieved GB/s =
                  algorithmic bytes (keys and values of every valid position, q,
                  o, lse, block-table entries) per call / mean call time, against
                  8000 GB/s; its oracle baseline runs the whole workload.

  fp8          -- the FP8 forward on the same workload: the attention kernel
                  alone (E4M3 Q and K codes already in device memory) and the
                  whole path with the quantisation of Q and K; roofline against
                  the mixed peak of FP8 Q K^T (5000) and bf16 P V (2500),
                  1 / (0.5 / 5000 + 0.5 / 2500) = 3333 TFLOP/s.

--path backward / --path decode / --path fp8 make that pass the timed step instead.

Order: the headline's inputs go to the device first, then the other legs run
back to back on the GPU, then the headline's warm-up and timed steps, and only
then the oracle baselines (host work).  So the timed steps start on a GPU that
has been busy: an idle GPU drops its clock, and raising it again takes longer
than a few warm-up launches (tens of milliseconds).  After the
timed steps the shader clock is sampled with rocm-smi while the same kernel
keeps running, and roofline.frac_at_measured_clock rates the kernel against the
MFMA peak scaled to that clock.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HEADLINE = "bf16_causal_b2h32n4096d128"
PEAK_BF16_TFLOPS = 2500.0
PEAK_F32_TFLOPS = 157.3  # dense fp32 MFMA
PEAK_SCLK_MHZ = 2400.0  # the clock the published peaks assume
METRIC = "attention fwd TFLOP/s (bf16, causal/non-causal) and % of MI355X MFMA peak"
BWD_METRIC = "attention bwd TFLOP/s (bf16, nominal 10*N^2*d per head) and % of MI355X MFMA peak"
DEC_METRIC = "paged decode attention GB/s (bf16, keys and values read once) and % of MI355X HBM bandwidth"
PEAK_HBM_GBS = 8000.0
DECODE_HEADLINE = "decode_b64h32d128_len2048"
FP8_METRIC = "attention fwd TFLOP/s with FP8 (E4M3) Q and K, bf16 V, and % of the mixed FP8/bf16 MFMA peak"
PEAK_FP8_MIXED_TFLOPS = 1.0 / (0.5 / 5000.0 + 0.5 / 2500.0)

# Sources each timed path is built from: a traffic figure measured on other
# sources is stale and is not reported.
# (fa_launch.h holds host-side declarations only; the sizes kernels share with
# the host live in fa_sizes.h.)
KERNEL_SOURCES = {
    "fused": ["fa_fwd_bf16.hip", "fa_epilogue.h", "fa_tile.h", "fa_common.h"],
    "fused_f32": ["fa_fwd_f32.hip", "fa_common.h"],
    "unfused": ["fa_unfused.hip", "fa_epilogue.h", "fa_tile.h", "fa_common.h"],
    "backward": ["fa_bwd_bf16.hip", "fa_epilogue.h", "fa_tile.h", "fa_common.h"],
    "decode": ["fa_decode_bf16.hip", "fa_common.h", "fa_sizes.h"],
    "fp8": ["fa_fwd_fp8.hip", "fa_epilogue.h", "fa_tile.h", "fa_common.h", "fa_sizes.h"],
}


# The GPU machines allot 16 host CPUs to a job that drives one GPU, whatever the
# node shows; the oracle runs on that share.
HOST_SHARE = 16


def host_cpus() -> int:
    """CPUs this process may run on (what nproc reports)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def host_threads() -> int:
    return max(1, min(HOST_SHARE, host_cpus()))


def host_cpu_model() -> str:
    """lscpu's model name (from /proc/cpuinfo if lscpu is missing)."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_fields(threads: int) -> dict:
    return {"cores": threads, "host_cpus": host_cpus(), "cpu_model": host_cpu_model(),
            "threads_note": f"the oracle runs on {threads} threads: the job's share of the host "
                            f"({HOST_SHARE} CPUs per GPU job), of {host_cpus()} CPUs the node shows"}


def sample_sclk(torch, launch, seconds: float = 1.0):
    """Median shader clock (MHz, rocm-smi) while `launch` runs back to back for about
    `seconds`; None if rocm-smi is unavailable."""
    import re
    import subprocess
    import threading
    samples, stop = [], threading.Event()

    def poll():
        while not stop.is_set():
            try:
                out = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True,
                                     timeout=5).stdout
                m = re.search(r'"sclk clock speed:": "\((\d+)Mhz\)"', out)
                if m:
                    samples.append(int(m.group(1)))
            except (OSError, subprocess.SubprocessError):
                return
            time.sleep(0.02)

    th = threading.Thread(target=poll, daemon=True)
    th.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            launch()
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=10)
    if not samples:
        return None
    samples.sort()
    return {"sclk_mhz_median": samples[len(samples) // 2], "sclk_mhz_min": samples[0], "sclk_mhz_max": samples[-1],
            "samples": len(samples), "how": f"rocm-smi --showclocks while the timed kernel runs back to back "
                                             f"for {seconds:.1f} s after the timed steps"}


def device_inputs(torch, x):
    if x.workload.dtype == "bf16":
        def dev(bits):
            return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
        q, k, v = dev(x.q_bits), dev(x.k_bits), dev(x.v_bits)
    else:
        q, k, v = (torch.from_numpy(a).cuda() for a in (x.q, x.k, x.v))
    lim = None if x.kv_limit is None else torch.from_numpy(x.kv_limit).cuda()
    return q, k, v, lim


LAST_HOST_US = [0.0]  # host time per call of the last timed loop (microseconds)


def time_launches(torch, launch, steps: int, warmup: int) -> float:
    """Mean milliseconds per launch, HIP events on the current (launch) stream."""
    for _ in range(warmup):
        launch()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        launch()
    end.record(stream)
    LAST_HOST_US[0] = (time.perf_counter() - t0) / steps * 1e6
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def launch_spread(torch, launch, n: int) -> dict:
    """Median and minimum milliseconds of n single launches, each between its own
    pair of HIP events on the launch stream (run after, and apart from, the timed
    steps, whose mean is the reported rate)."""
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in ev:
        a.record(stream)
        launch()
        b.record(stream)
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)
    return {"launches": n, "median_ms": round(t[n // 2] if n % 2 else 0.5 * (t[n // 2 - 1] + t[n // 2]), 5),
            "min_ms": round(t[0], 5)}


def fused_launcher(torch, binding, x):
    """Device copies of x's inputs and outputs, and a function launching the fused
    forward on them (one step)."""
    w = x.workload
    q, k, v, lim = device_inputs(torch, x)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=q.device)
    fn = binding.fa_fwd_bf16 if w.dtype == "bf16" else binding.fa_fwd_f32
    stream = torch.cuda.current_stream()

    def launch():
        fn(q, k, v, o, lse, w.causal, w.scale, lim, stream)

    return launch


def measure_fused(torch, binding, x, steps, warmup, spread=0, clock=None, launch=None):
    """Mean ms per fused launch; with spread > 0 also launch_spread over that many
    launches; with clock given (True or False) a third value, the shader clock
    sampled while the kernel runs on (None when clock is False)."""
    launch = launch or fused_launcher(torch, binding, x)
    ms = time_launches(torch, launch, steps, warmup)
    sp = launch_spread(torch, launch, spread) if spread else None
    clk = sample_sclk(torch, launch) if clock else None
    if clock is not None:
        return ms, sp, clk
    return (ms, sp) if spread else ms


def measure_unfused(torch, binding, x, steps, warmup):
    w = x.workload
    q, k, v, lim = device_inputs(torch, x)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=q.device)
    ws = torch.empty(binding.fa_unfused_workspace_bytes(w.B, w.H, w.N, 2), dtype=torch.uint8, device=q.device)
    stream = torch.cuda.current_stream()

    def launch():
        binding.fa_fwd_unfused_bf16(q, k, v, o, lse, w.causal, w.scale, lim, ws, stream)

    ms = time_launches(torch, launch, steps, warmup)
    del q, k, v, o, lse, lim, ws
    return ms


def measure_backward(torch, binding, x, g, steps, warmup, spread=0):
    """Mean ms per fa_bwd_bf16 call (three launches) on O and LSE from one forward;
    with spread > 0 also launch_spread over that many calls."""
    w = x.workload
    q, k, v, lim = device_inputs(torch, x)
    o, lse = binding.attention(q, k, v, causal=w.causal, scale=w.scale, kv_limit=lim)
    dout = torch.from_numpy(g.dout_bits.view(np.int16)).view(torch.bfloat16).cuda()
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(binding.fa_bwd_workspace_bytes(w.B, w.H, w.N), dtype=torch.uint8, device=q.device)
    stream = torch.cuda.current_stream()

    def launch():
        binding.fa_bwd_bf16(q, k, v, o, dout, lse, dq, dk, dv, w.causal, w.scale, lim, ws, stream)

    ms = time_launches(torch, launch, steps, warmup)
    sp = launch_spread(torch, launch, spread) if spread else None
    del q, k, v, o, lse, lim, dout, dq, dk, dv, ws
    return (ms, sp) if spread else ms


def unfused_bytes(w) -> int:
    """Minimum bytes of the unfused three-kernel forward: the S and P round trips
    over rows of ld = N rounded up to 64, plus Q, K, V read and O, LSE written."""
    elem = 2 if w.dtype == "bf16" else 4
    ld = -(-w.N // 64) * 64
    rows = w.B * w.H * w.N
    return rows * ld * (4 + 4 + elem + elem) + 4 * rows * w.d * elem + rows * 4


def decode_bytes(xd) -> int:
    """Algorithmic bytes of one paged decode call."""
    w = xd.workload
    pages = int(sum(-(-int(n) // inputs_page(xd)) for n in xd.seq_lens))
    return xd.kv_bytes() + 2 * (w.B * w.H * w.d * 2) + w.B * w.H * 4 + pages * 4 + w.B * 4


def inputs_page(xd) -> int:
    return int(xd.k_cache.shape[2])


def measure_decode(torch, binding, xd, steps, warmup):
    """(mean ms per fa_decode_paged_bf16 call (split and combine launches), launch_spread of the calls)."""
    w = xd.workload
    dev16 = lambda bits: torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    q, kc, vc = dev16(xd.q_bits), dev16(xd.k_bits), dev16(xd.v_bits)
    bt = torch.from_numpy(xd.block_table).cuda()
    sl = torch.from_numpy(xd.seq_lens).cuda()
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H), dtype=torch.float32, device=q.device)
    ws = torch.empty(binding.fa_decode_workspace_bytes(w.B, w.H, w.d, w.max_pages), dtype=torch.uint8,
                     device=q.device)
    stream = torch.cuda.current_stream()

    def launch():
        binding.fa_decode_paged_bf16(q, kc, vc, bt, sl, o, lse, w.scale, ws, stream)

    ms = time_launches(torch, launch, steps, warmup)
    spread = launch_spread(torch, launch, SPREAD_LAUNCHES)
    del q, kc, vc, bt, sl, o, lse, ws
    return ms, spread


def cpu_baseline_decode(xd):
    """The oracle's paged decode over the whole workload."""
    import oracle
    threads = host_threads()
    q, kc, vc = (np.ascontiguousarray(a, dtype=np.float64) for a in (xd.q, xd.k_cache, xd.v_cache))
    t0 = time.perf_counter()
    oracle.decode_paged(q, kc, vc, xd.block_table, xd.seq_lens, xd.workload.scale, nthreads=threads)
    dt = time.perf_counter() - t0
    return {"value": decode_bytes(xd) / dt / 1e9, "unit": "GB/s", **host_fields(threads), "kind": "oracle",
            "sample": f"the whole {xd.workload.name} workload, fp64, {dt:.3f} s; same algorithmic bytes",
            "seconds": round(dt, 3)}


def decode_entry(torch, binding, xd, steps, warmup, traffic_file, cpu: bool):
    ms, spread = measure_decode(torch, binding, xd, steps, warmup)
    gbs = decode_bytes(xd) / (ms * 1e-3) / 1e9
    spread["GB/s_at_median"] = round(decode_bytes(xd) / (spread["median_ms"] * 1e-3) / 1e9, 1)
    spread["GB/s_at_min"] = round(decode_bytes(xd) / (spread["min_ms"] * 1e-3) / 1e9, 1)
    entry = {"metric": DEC_METRIC, "workload": xd.workload.name, "value": round(gbs, 1), "unit": "GB/s",
             "ms_per_step": round(ms, 5), "per_launch": spread, "bytes_per_step": decode_bytes(xd),
             "TFLOP/s": round(xd.flops() / (ms * 1e-3) / 1e12, 2),
             "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                          "frac": round(gbs / PEAK_HBM_GBS, 4),
                          "traffic": load_traffic(traffic_file, "decode", xd.workload.name),
                          "note": "one call = two launches (splits, then their merge); achieved = algorithmic "
                                  "bytes per call / mean call time"}}
    if cpu:
        entry["cpu_baseline"] = cpu_baseline_decode(xd)
    return entry


def measure_fp8(torch, binding, x, steps, warmup):
    """(ms of the FP8 attention kernel alone, ms of quantise K + attention with Q
    encoded in the kernel, ms of quantise Q + quantise K + attention, launch_spread
    of the attention kernel)."""
    from flashattention_forward_attn_amd import inputs
    w = x.workload
    q, k, v, lim = device_inputs(torch, x)
    signs = torch.from_numpy(inputs.fp8_signs(w.d)).cuda()
    qc, qe = binding.fp8_quantize(q, signs, binding.FP8_Q_TILE)
    kc, ke = binding.fp8_quantize(k, signs, binding.FP8_K_TILE)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream()

    def attend():
        binding.fa_fwd_fp8(qc, qe, kc, ke, v, o, lse, w.causal, w.scale, lim, stream)

    def whole():
        # k quantised by its kernel, q rotated and encoded inside the attention kernel
        binding.fa_fp8_quantize_bf16(k, signs, kc, ke, binding.FP8_K_TILE, stream)
        binding.fa_fwd_fp8_qbf16(q, signs, kc, ke, v, o, lse, w.causal, w.scale, lim, stream)

    def two_steps():
        binding.fa_fp8_quantize_bf16(q, signs, qc, qe, binding.FP8_Q_TILE, stream)
        binding.fa_fp8_quantize_bf16(k, signs, kc, ke, binding.FP8_K_TILE, stream)
        attend()

    ms = time_launches(torch, attend, steps, warmup)
    spread = launch_spread(torch, attend, SPREAD_LAUNCHES)
    ms_whole = time_launches(torch, whole, max(10, steps // 2), max(5, warmup // 4))
    ms_two = time_launches(torch, two_steps, max(10, steps // 2), max(5, warmup // 4))
    del q, k, v, lim, signs, qc, qe, kc, ke, o, lse
    return ms, ms_whole, ms_two, spread


def cpu_baseline_fp8(x, target_seconds: float):
    """The oracle's FP8 path (quantise, then attention on the codes) on the first heads."""
    import oracle
    from flashattention_forward_attn_amd import inputs
    w = x.workload
    threads = host_threads()
    signs = inputs.fp8_signs(w.d)
    nh = 1
    while True:
        sl = lambda a: np.ascontiguousarray(a[:1, :nh], dtype=np.float64)
        q, k, v = sl(x.q), sl(x.k), sl(x.v)
        lim = None if x.kv_limit is None else np.ascontiguousarray(x.kv_limit[:1])
        t0 = time.perf_counter()
        qc, qe = oracle.fp8_quantize(q, signs, tile_rows=32, nthreads=threads)
        kc, ke = oracle.fp8_quantize(k, signs, tile_rows=64, nthreads=threads)
        oracle.attention_fp8(qc, qe, 32, kc, ke, 64, v, causal=w.causal, scale=w.scale, kv_limit=lim, nthreads=threads)
        dt = time.perf_counter() - t0
        if dt * 2 > target_seconds or nh * 2 > w.H:
            break
        nh *= 2
    flops = w.flops() / (w.B * w.H) * nh
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", **host_fields(threads), "kind": "oracle",
            "sample": f"heads 0..{nh - 1} of batch item 0 of {w.name}: quantisation and attention on the codes, "
                      f"fp64, {dt:.1f} s", "seconds": round(dt, 3)}


def fp8_entry(torch, binding, x, steps, warmup, traffic_file, cpu: bool, cpu_seconds: float):
    w = x.workload
    ms, ms_whole, ms_two, spread = measure_fp8(torch, binding, x, steps, warmup)
    tf = w.flops() / (ms * 1e-3) / 1e12
    spread["TFLOP/s_at_median"] = round(w.flops() / (spread["median_ms"] * 1e-3) / 1e12, 2)
    spread["TFLOP/s_at_min"] = round(w.flops() / (spread["min_ms"] * 1e-3) / 1e12, 2)
    entry = {"metric": FP8_METRIC, "value": round(tf, 2), "unit": "TFLOP/s", "ms_per_step": round(ms, 5),
             "per_launch": spread,
             "with_quantisation": {"ms_per_step": round(ms_whole, 5),
                                   "TFLOP/s": round(w.flops() / (ms_whole * 1e-3) / 1e12, 2),
                                   "calls": "fa_fp8_quantize_bf16 (k) + fa_fwd_fp8_qbf16",
                                   "two_steps_ms": round(ms_two, 5),
                                   "two_steps_TFLOP/s": round(w.flops() / (ms_two * 1e-3) / 1e12, 2)},
             "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": round(PEAK_FP8_MIXED_TFLOPS, 1),
                          "unit": "TFLOP/s", "frac": round(tf / PEAK_FP8_MIXED_TFLOPS, 4),
                          "traffic": load_traffic(traffic_file, "fp8", w.name),
                          "note": "attention kernel alone; half the nominal FLOPs on FP8 (Q K^T), half on bf16 (P V)"}}
    if cpu:
        entry["cpu_baseline"] = cpu_baseline_fp8(x, cpu_seconds)
    return entry


def effective_flops(x) -> float:
    """FLOPs of the valid (query, key) pairs only: 4 d per pair."""
    w = x.workload
    i = np.arange(w.N, dtype=np.int64)
    lim = np.full((w.B, w.N), w.N, np.int64) if x.kv_limit is None else np.minimum(x.kv_limit.astype(np.int64), w.N)
    if w.causal:
        lim = np.minimum(lim, i[None, :] + 1)
    return float(4.0 * w.d * w.H * lim.sum())


def cpu_baseline(x, target_seconds: float):
    """Oracle on an evenly spaced sample of query rows, calibrated to about target_seconds."""
    import oracle
    w = x.workload
    threads = host_threads()
    rows_total = w.B * w.H * w.N
    flops_per_row = w.flops() / rows_total
    # the oracle takes fp64; widen once so the timed calls do no conversion
    q, k, v = (np.ascontiguousarray(a, dtype=np.float64) for a in (x.q, x.k, x.v))
    n_cal = min(rows_total, 64 * threads)
    ids = np.linspace(0, rows_total - 1, n_cal).astype(np.int64)
    t0 = time.perf_counter()
    oracle.attention_rows(q, k, v, ids, w.causal, w.scale, x.kv_limit, nthreads=threads)
    cal = time.perf_counter() - t0
    n = int(min(rows_total, max(n_cal, n_cal * target_seconds / max(cal, 1e-6))))
    ids = np.unique(np.linspace(0, rows_total - 1, n).astype(np.int64))
    t0 = time.perf_counter()
    oracle.attention_rows(q, k, v, ids, w.causal, w.scale, x.kv_limit, nthreads=threads)
    dt = time.perf_counter() - t0
    return {
        "value": ids.size * flops_per_row / dt / 1e12,
        "unit": "TFLOP/s",
        **host_fields(threads),
        "kind": "oracle",
        "sample": f"{ids.size} of {rows_total} query rows of {w.name}, evenly spaced, fp64, "
                  f"{dt:.1f} s; FLOPs per row = workload FLOPs / rows",
        "seconds": round(dt, 3),
    }


def cpu_baseline_backward(x, g):
    """The oracle's full fp64 backward over the first heads of batch item 0, one
    head per host thread (the oracle runs heads in parallel)."""
    import oracle
    w = x.workload
    threads = host_threads()
    nh = min(w.H, threads)
    sl = lambda a: np.ascontiguousarray(a[:1, :nh], dtype=np.float64)
    q, k, v, dout = sl(x.q), sl(x.k), sl(x.v), sl(g.dout)
    lim = None if x.kv_limit is None else np.ascontiguousarray(x.kv_limit[:1])
    t0 = time.perf_counter()
    oracle.attention_bwd(q, k, v, dout, w.causal, w.scale, lim, nthreads=threads)
    dt = time.perf_counter() - t0
    flops = w.bwd_flops() / (w.B * w.H) * nh
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        **host_fields(threads),
        "kind": "oracle",
        "sample": f"full backward of heads 0..{nh - 1} of batch item 0 of {w.name}, fp64, {dt:.1f} s; "
                  f"nominal backward FLOPs of those heads",
        "seconds": round(dt, 3),
    }


def load_traffic(path_file: str, path: str, workload: str, sources: str | None = None):
    """Measured HBM bytes per launch for (path, workload), or None if absent or
    stale (taken on other kernel sources: those of `sources`, default `path`)."""
    if not os.path.exists(path_file):
        return None
    with open(path_file) as f:
        t = json.load(f).get(path, {}).get(workload)
    if t and t.get("kernel_source_sha256") == _kernel_digest(sources or path):
        return t.get("bytes_per_launch")
    return None


def measure_extras(torch, binding, inputs, x, g, w, args):
    """The unfused baseline, the other bf16 workloads, the backward, the FP8 forward
    and the paged decode, each timed the same way, back to back on the GPU.  Their
    oracle baselines (host work) are returned as deferred jobs, run after the
    headline's timed steps."""
    out, deferred = {}, []
    ums = measure_unfused(torch, binding, x, max(5, args.steps // 5), 3)
    ugbs = unfused_bytes(w) / (ums * 1e-3) / 1e9
    out["unfused"] = {"ms_per_step": round(ums, 4), "TFLOP/s": round(w.flops() / (ums * 1e-3) / 1e12, 2),
                      "GB/s": round(ugbs, 1), "hbm_frac": round(ugbs / PEAK_HBM_GBS, 4),
                      "traffic": load_traffic(args.traffic, "unfused", w.name)}
    others = {}
    for name, ow in inputs.WORKLOADS.items():
        if name == w.name or ow.dtype != "bf16":
            continue
        ox = inputs.generate(ow)
        oms = measure_fused(torch, binding, ox, args.steps, args.warmup)
        entry = {"ms": round(oms, 5), "TFLOP/s": round(ow.flops() / (oms * 1e-3) / 1e12, 2),
                 "frac": round(ow.flops() / (oms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                 "traffic": load_traffic(args.traffic, "fused", name)}
        if ox.kv_limit is not None:
            entry["effective_TFLOP/s"] = round(effective_flops(ox) / (oms * 1e-3) / 1e12, 2)
        others[name] = entry
        del ox
    out["workloads"] = others
    if g is not None:
        bms = measure_backward(torch, binding, x, g, max(20, args.steps // 2), max(10, args.warmup // 4))
        btf = w.bwd_flops() / (bms * 1e-3) / 1e12
        out["backward"] = {
            "metric": BWD_METRIC, "value": round(btf, 2), "unit": "TFLOP/s", "ms_per_step": round(bms, 5),
            "flops_per_step": w.bwd_flops(),
            "roofline": {"bound": "mfma", "achieved": round(btf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(btf / PEAK_BF16_TFLOPS, 4),
                         "traffic": load_traffic(args.traffic, "backward", w.name), "note": BWD_NOTE},
        }
        out["fp8"] = fp8_entry(torch, binding, x, args.steps, args.warmup, args.traffic, False, args.cpu_seconds)
        xd = inputs.generate_decode(inputs.DECODE_WORKLOADS[args.decode_workload])
        out["decode"] = decode_entry(torch, binding, xd, max(20, args.steps // 2), max(10, args.warmup // 4),
                                     args.traffic, False)
        if not args.no_cpu_baseline:
            deferred.append(lambda: out["backward"].__setitem__("cpu_baseline", cpu_baseline_backward(x, g)))
            deferred.append(lambda: out["fp8"].__setitem__("cpu_baseline", cpu_baseline_fp8(x, args.cpu_seconds)))
            deferred.append(lambda: out["decode"].__setitem__("cpu_baseline", cpu_baseline_decode(xd)))
    return out, deferred


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200, help="untimed launches first (also lets the clocks ramp)")
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the unfused baseline and other workloads")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the shader-clock sample after the timed steps (about a second of extra launches; "
                         "for runs under a profiler)")
    ap.add_argument("--traffic", default=os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                                                      "traffic.json"),
                    help="measured HBM bytes per launch (from rocprofv3 FETCH_SIZE/WRITE_SIZE), if present")
    ap.add_argument("--path", choices=("fused", "unfused", "backward", "decode", "fp8"), default="fused",
                    help="time the fused kernel (default), the unfused three-kernel baseline, the "
                         "backward pass, the paged decode or the FP8 forward as the step")
    ap.add_argument("--decode-workload", default=DECODE_HEADLINE)
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of this many MiB (twice untimed, "
                         "then 13 timed for its TB/s) and exit; its FETCH_SIZE/WRITE_SIZE calibrate the "
                         "traffic counters")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the forward pass shards over (batch, head) with no communication between GPUs)",
              file=sys.stderr)
        return 2

    import torch
    from flashattention_forward_attn_amd import binding, inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if args.copy_probe:
        n = args.copy_probe * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        # the same copy timed: a read+write stream, the practical ceiling for kernels
        # that read and write about as much (the unfused softmax)
        ms = time_launches(torch, lambda: dst.copy_(src), 10, 3)
        print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4,
                          "copy_ms": round(ms, 4), "copy_TBps_read_plus_write": round(2 * n * 4 / (ms * 1e-3) / 1e12, 3)}),
              flush=True)
        return 0
    binding.load()

    if args.path == "decode":
        xd = inputs.generate_decode(inputs.DECODE_WORKLOADS[args.decode_workload])
        entry = decode_entry(torch, binding, xd, args.steps, args.warmup, args.traffic, not args.no_cpu_baseline)
        line = {"metric": DEC_METRIC, "value": entry["value"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
                "warmup": args.warmup, "ms_per_step": entry["ms_per_step"], "higher_is_better": True,
                "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
                "data": "synthetic (seeded numpy draws, inputs resident in HBM)",
                "config": {"workload": xd.workload.name, "B": xd.workload.B, "H": xd.workload.H, "d": xd.workload.d,
                           "max_len": xd.workload.max_len, "page": 16, "path": "decode",
                           "bytes_per_step": entry["bytes_per_step"], "parallelism": "single GPU"},
                "roofline": entry["roofline"], "per_launch": entry["per_launch"]}
        if "cpu_baseline" in entry:
            line["cpu_baseline"] = entry["cpu_baseline"]
        print(json.dumps(line), flush=True)
        return 0

    if args.path == "fp8":
        w = inputs.WORKLOADS[args.workload]
        x = inputs.generate(w)
        entry = fp8_entry(torch, binding, x, args.steps, args.warmup, args.traffic, not args.no_cpu_baseline,
                          args.cpu_seconds)
        line = {"metric": FP8_METRIC, "value": entry["value"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
                "warmup": args.warmup, "ms_per_step": entry["ms_per_step"], "higher_is_better": True,
                "scaling": "weak", "vs_baseline": None, "dtype": "fp8-e4m3 (Q, K) / bf16 (V, P)",
                "data": "synthetic (seeded numpy draws, inputs resident in HBM)",
                "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                           "path": "fp8", "flops_per_step": w.flops(), "parallelism": "single GPU"},
                "roofline": entry["roofline"], "with_quantisation": entry["with_quantisation"],
                "per_launch": entry["per_launch"]}
        if "cpu_baseline" in entry:
            line["cpu_baseline"] = entry["cpu_baseline"]
        print(json.dumps(line), flush=True)
        return 0

    w = inputs.WORKLOADS[args.workload]
    if w.dtype != "bf16" and args.path == "backward":
        print("the backward pass is bf16 only", file=sys.stderr)
        return 2
    x = inputs.generate(w)
    g = inputs.grad_output(w) if w.dtype == "bf16" else None
    # The other legs run first: the headline's warm-up and timed steps then start
    # on a GPU that has been busy, as a kernel inside a model step would.
    extras, deferred = {}, []
    launch = fused_launcher(torch, binding, x) if args.path == "fused" else None
    if not args.no_extras and args.path == "fused":
        extras, deferred = measure_extras(torch, binding, inputs, x, g, w, args)
    spread = None
    clock = None
    if args.path == "backward":
        ms, spread = measure_backward(torch, binding, x, g, args.steps, args.warmup, spread=SPREAD_LAUNCHES)
        tflops = w.bwd_flops() / (ms * 1e-3) / 1e12
    elif args.path == "fused":
        ms, spread, clock = measure_fused(torch, binding, x, args.steps, args.warmup, spread=SPREAD_LAUNCHES,
                                          clock=not args.no_clock, launch=launch)
        host_us = LAST_HOST_US[0]
        tflops = w.flops() / (ms * 1e-3) / 1e12
    else:
        ms = measure_unfused(torch, binding, x, args.steps, args.warmup)
        tflops = w.flops() / (ms * 1e-3) / 1e12
    # host work only after every timed GPU leg
    for job in deferred:
        job()
    traffic = load_traffic(args.traffic, args.path, w.name,
                           "fused_f32" if args.path == "fused" and w.dtype == "f32" else None)
    peak = PEAK_F32_TFLOPS if w.dtype == "f32" and args.path == "fused" else PEAK_BF16_TFLOPS

    line = {
        "metric": BWD_METRIC if args.path == "backward" else METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded numpy draws, inputs resident in HBM)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                   "scale": "1/sqrt(d)",
                   "flops_per_step": w.bwd_flops() if args.path == "backward" else w.flops(), "path": args.path,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(tflops / peak, 4), "traffic": traffic},
    }
    if clock is not None:
        # the same fraction against the MFMA peak at the clock the GPU ran at
        line["roofline"]["clock"] = clock
        line["roofline"]["frac_at_measured_clock"] = round(
            tflops / (peak * clock["sclk_mhz_median"] / PEAK_SCLK_MHZ), 4)
    if spread is not None:
        fl = w.bwd_flops() if args.path == "backward" else w.flops()
        spread["TFLOP/s_at_median"] = round(fl / (spread["median_ms"] * 1e-3) / 1e12, 2)
        spread["TFLOP/s_at_min"] = round(fl / (spread["min_ms"] * 1e-3) / 1e12, 2)
        line["per_launch"] = spread
    if args.path == "fused":
        line["host_us_per_call"] = round(host_us, 1)
    if args.path == "unfused":
        ub = unfused_bytes(w)
        gbs = ub / (ms * 1e-3) / 1e9
        line["roofline"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                            "note": "three kernels per step; achieved = the unfused method's own minimum bytes "
                                    "(S written and read in fp32, P written and read in the input precision, "
                                    "Q, K, V read, O and LSE written) / mean step time"}
        line["config"]["bytes_per_step"] = ub
    if args.path == "backward":
        line["roofline"]["note"] = BWD_NOTE
    if extras:
        if "unfused" in extras:
            extras["unfused"]["fused_speedup"] = round(extras["unfused"]["ms_per_step"] / ms, 2)
        line.update(extras)
    if not args.no_cpu_baseline:
        if args.path == "backward":
            line["cpu_baseline"] = cpu_baseline_backward(x, g)
        else:
            line["cpu_baseline"] = cpu_baseline(x, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


# single launches timed one by one after the timed steps (median and minimum)
SPREAD_LAUNCHES = 51

BWD_NOTE = ("one call = three launches (row statistics, dK/dV, dQ); achieved = nominal FLOPs "
            "(10*N^2*d per head, halved for causal) / mean call time; the kernels execute 14*N^2*d "
            "(the dQ kernel recomputes S and dP)")


def _kernel_digest(path: str) -> str:
    """sha256 over the sources the given path's kernels are built from."""
    import hashlib
    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "flashattention_forward_attn_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(KERNEL_SOURCES[path]):
        with open(os.path.join(here, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()


if __name__ == "__main__":
    sys.exit(main())
