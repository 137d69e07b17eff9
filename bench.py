"""Benchmark: causal bf16 exact attention, forward + backward, on one MI355X.

One step is the whole hot path over one batch of synthetic input: the forward
kernel (O and LSE), then the backward: preparation (two small kernels), dQ
(which also forms the exact row dot D), dK/dV. The
workload is B=2, Hq=32, Hkv=8 (grouped-query attention), N=16384, d=128,
causal, bf16 inputs ~ N(0, 1) from a fixed seed, dO ~ N(0, 1).

Throughput counts 4*B*Hq*N^2*d FLOP for the forward, halved under the causal
mask, and 2.5 times that for the backward. Inputs are resident in device memory
before the timed region; each kernel is bracketed by HIP events on the stream
it runs on. Prints one JSON line.

    python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--no-cpu-baseline]

With --varlen NAME it measures the forward and backward passes over packed
sequences of different lengths (flash_attn_fwd_varlen, flash_attn_bwd_varlen)
against the MFMA roofline, counting 4*Hq*d FLOP per visible (query, key) pair of
every sequence for the forward and 2.5 times that for the backward.

With --window W it measures the forward and backward passes of the same
workload under a sliding-window causal mask of W keys (flash_attn_fwd_window,
flash_attn_bwd_window), counting 4*d FLOP per visible pair for the forward and
2.5 times that for the backward: sum over rows of min(i + 1, W) pairs per head.

With --f32 NAME it measures the forward on fp32 inputs (flash_attn_fwd_f32) at that
workload's shape, against the fp32 matrix peak (157.3 TFLOP/s).

With --fp8 NAME it measures the forward on E4M3 inputs (flash_attn_fwd_e4m3) at
that workload's shape, against the FP8 MFMA peak (twice the bf16 one).

With --decode NAME it measures instead the decode path (a few query rows over
a long key/value cache) on one of the decode workloads, against the HBM
roofline: the bytes the step must move (K and V once, Q, O and LSE) over the
time of one call (range kernel and merge). Before each timed call a 512 MiB
read evicts the cache from the 256 MB last-level cache, so K and V come from
HBM.
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
sys.path.insert(0, ROOT)

import attn_inputs as ai  # noqa: E402

METRIC = "attention fwd/bwd TFLOP/s (bf16, causal) and % of MI355X bf16 MFMA peak"
WORKLOAD = "gqa16k"
# MI355X dense bf16 MFMA peak: 256 CUs x 2.4 GHz x 4096 FLOP per clock per CU.
RATED_MHZ = 2400.0
PEAK_BF16_TFLOPS = 256 * RATED_MHZ * 1e6 * 4096 / 1e12
# What the timed step computes in: bf16 tensors in and out, bf16 MFMA operands in
# the forward, fp16 MFMA operands (power-of-two scaled copies of the bf16 inputs,
# P and dS rounded to fp16) in the backward, fp32 accumulation and softmax.
DTYPE_FWD_BWD = "bf16 fwd / fp16-operand bwd"
PRECISION = {"io": "bf16 (LSE fp32)", "fwd_mfma": "bf16 x bf16 -> fp32",
             "bwd_mfma": "fp16 x fp16 -> fp32 (scaled copies of the bf16 inputs; P, dS in fp16)",
             "softmax": "fp32"}
PRECISION_FWD = {"io": "bf16 (LSE fp32)", "fwd_mfma": "bf16 x bf16 -> fp32", "softmax": "fp32"}
PEAK_HBM_GBS = 8000.0
KERNELS = ("fwd", "bwd_pre", "bwd_dq", "bwd_dkdv")


def pair_count(w) -> float:
    """(query, key) pairs per query head as the FLOP formula counts them: N^2, halved when causal."""
    return w.N * w.N / (2.0 if w.causal else 1.0)


def algorithmic(w) -> dict:
    """Algorithmic work per launch of each kernel.

    fwd:      S = QK^T and O += PV, 4*d FLOP per visible pair.
    bwd_dkdv: S (rebuilt), dP = dO V^T, dV += P^T dO, dK += dS^T Q, 8*d FLOP per pair.
    bwd_dq:   dQ += dS K, 2*d FLOP per pair (its S and dP are a second evaluation
              of the same products, and its P K product only corrects dQ for
              the exact row dot, so neither is counted again).
    bwd_pre:  reads Q, K, V, dO (max pass), then Q, K, V, dO, O and LSE, writes the
              fp16 copies, D and the log2-scaled LSE.
    """
    heads = w.B * w.Hq
    pairs = heads * pair_count(w)
    rows = heads * w.N
    return {
        "fwd": ("flop", 4 * w.d * pairs),
        "bwd_dkdv": ("flop", 8 * w.d * pairs),
        "bwd_dq": ("flop", 2 * w.d * pairs),
        "bwd_pre": ("bytes", 2 * 2 * (2 * w.B * w.Hq + 2 * w.B * w.Hkv) * w.N * w.d
                    + rows * (2 * 2 * w.d + 4 + 4 + 4)),
    }


# Sources each timed kernel is built from (hashed to tie a traffic record to the kernel it measured).
KERNEL_SOURCES = {
    "decode": ("fa_decode.hip", "fa_device.h", "fa_params.h"),
    "fwd": ("fa_fwd.hip", "fa_device.h", "fa_params.h"),
    "bwd_dq": ("fa_bwd.hip", "fa_device.h", "fa_params.h"),
    "bwd_dkdv": ("fa_bwd.hip", "fa_device.h", "fa_params.h"),
    "fwd8": ("fa_fwd8.hip", "fa_device.h", "fa_params.h"),
}


def sources_sha256(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "exact_io_aware_60_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str = WORKLOAD):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (profiles/traffic_<workload>.md: FETCH_SIZE and WRITE_SIZE, each scaled by what
    the counter reads for a 1 GiB device copy), or None when there is no record or
    the kernel's sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    want = sources_sha256(kernel)
    with open(path) as fh:
        for line in fh:
            m = re.match(r"traffic-record: kernel=(\w+) bytes=(\d+) sources_sha256=(\w+)", line.strip())
            if m and m.group(1) == kernel and m.group(3) == want:
                return int(m.group(2))
    return None


def copy_calibration(mib: int, device) -> None:
    """A plain device copy of `mib` MiB, 3 times (it reads and writes exactly
    that much per launch), so that a profiled run holds the reference kernel
    for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    if mib <= 0:
        return
    src = torch.ones(mib << 20, dtype=torch.uint8, device=device)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


class ClockSampler:
    """Samples the GPU's current engine clock from sysfs (pp_dpm_sclk, the line
    marked '*') every `period` seconds on a host thread, between start() and
    stop(). The rated peak assumes 2.4 GHz; under sustained MFMA load the clock
    runs lower, and the peak scaled by the sampled mean is the clock-adjusted
    peak. Returns None where the file is not readable."""

    def __init__(self, period: float = 0.002, settle: float = 0.0):
        import glob
        import threading
        self.period = period
        self.settle = settle            # seconds of samples dropped at the start (the average lags)
        self.paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.samples: list[float] = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        for path in self.paths:
            try:
                with open(path) as fh:
                    for line in fh:
                        if line.rstrip().endswith("*"):
                            m = re.search(r"(\d+)\s*[Mm][Hh]z", line)
                            if m:
                                return float(m.group(1))
            except OSError:
                continue
        return None

    def _run(self):
        t0 = time.perf_counter()
        while not self._stop.is_set():
            mhz = self._read()
            if mhz is not None and time.perf_counter() - t0 >= self.settle:
                self.samples.append(mhz)
            time.sleep(self.period)

    def start(self) -> "ClockSampler":
        if self.paths:
            self._thread.start()
        return self

    def stop(self):
        if not self.paths:
            return None
        self._stop.set()
        self._thread.join()
        if not self.samples:
            return None
        xs = self.samples
        return {"source": "sysfs pp_dpm_sclk (the power manager's average engine clock), sampled every 2 ms "
                          "while the step repeats back to back for about a second after the timed steps "
                          "(the first 0.25 s dropped)",
                "mean_mhz": sum(xs) / len(xs), "min_mhz": min(xs), "max_mhz": max(xs), "samples": len(xs),
                "rated_mhz": RATED_MHZ}


def sustained_clock(step, step_ms: float, seconds: float = 1.2):
    """Repeat `step` back to back for about `seconds` of GPU time while the
    sampler reads the engine clock (outside the timed region, so the metric is
    unaffected). Batches of about 50 ms keep the queue short."""
    import torch
    sampler = ClockSampler(settle=0.25)
    if not sampler.paths:
        return None
    per_batch = max(1, int(50.0 / max(step_ms, 1e-3)))
    torch.cuda.synchronize()
    sampler.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(per_batch):
            step()
        torch.cuda.synchronize()
    return sampler.stop()


def host_info() -> dict:
    """The host the oracle ran on: CPU model, os.cpu_count() and the cores this
    process may use."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0))}


def cpu_baseline(w) -> dict:
    """The fp64 oracle timed on the host cores on a bounded sample: the first
    (batch, K/V head) group (its G query heads) restricted to the first
    `n` positions, forward and backward (forward alone for a workload without
    a backward pass). Under the causal mask that prefix is a self-contained
    problem of the same shape family."""
    import oracle
    fwd_only = not w.backward
    n = int(os.environ.get("BENCH_CPU_SAMPLE_N", "32768" if fwd_only else "13312"))
    n = min(n, w.N)
    inp = ai.make_inputs(w)
    G = w.G
    q = ai.bf16_bits_to_f64(inp["q"][0:1, 0:G, :n])
    k = ai.bf16_bits_to_f64(inp["k"][0:1, 0:1, :n])
    v = ai.bf16_bits_to_f64(inp["v"][0:1, 0:1, :n])
    do = None if fwd_only else ai.bf16_bits_to_f64(inp["do"][0:1, 0:G, :n])
    del inp
    orc = oracle.default()
    t0 = time.perf_counter()
    orc.fwd(q, k, v, w.causal, w.scale)
    if not fwd_only:
        orc.bwd(q, k, v, do, w.causal, w.scale)
    dt = time.perf_counter() - t0
    flop = (1.0 if fwd_only else 3.5) * 4 * G * n * n / (2.0 if w.causal else 1.0) * w.d
    passes = "forward" if fwd_only else "forward + backward"
    prefix = "causal prefix" if w.causal else "prefix"
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": orc.num_threads(), "kind": "oracle",
            **host_info(),
            "sample": f"fp64 {passes} of batch 0, K/V head 0 ({G} query heads), first {n} of "
                      f"{w.N} positions ({prefix}); {dt:.1f} s",
            "seconds": dt}


def decode_bytes(w) -> int:
    """Bytes a decode step must move: the K and V rows in use once, Q read, O written (bf16), LSE (fp32)."""
    lens = ai.decode_seqlens(w)
    keys = w.B * w.Nk if lens is None else int(lens.sum())
    return 2 * 2 * w.Hkv * keys * w.d + 2 * 2 * w.B * w.Hq * w.Nq * w.d + 4 * w.B * w.Hq * w.Nq


def decode_cpu_baseline(w) -> dict:
    """The fp64 oracle on the whole decode workload (it runs in seconds)."""
    import oracle
    inp = ai.make_decode_inputs(w)
    lens = ai.decode_seqlens(w)
    if lens is None:
        lens = np.full(w.B, w.Nk)
    orc = oracle.default()
    dt = 0.0
    for b in range(w.B):
        L = int(lens[b])
        q = ai.bf16_bits_to_f64(inp["q"][b:b + 1])
        k = ai.bf16_bits_to_f64(inp["k"][b:b + 1, :, :L])
        v = ai.bf16_bits_to_f64(inp["v"][b:b + 1, :, :L])
        pos = L - w.Nq + np.arange(w.Nq, dtype=np.int64)
        t0 = time.perf_counter()
        orc.fwd(q, k, v, w.causal, w.scale, qpos=pos if w.causal else None)
        dt += time.perf_counter() - t0
    return {"value": decode_bytes(w) / dt / 1e9, "unit": "GB/s", "cores": orc.num_threads(), "kind": "oracle",
            **host_info(),
            "sample": f"the whole {w.name} step in fp64 (the bytes of its bf16 inputs and outputs per second); "
                      f"{dt:.2f} s", "seconds": dt}


def decode_main(args) -> int:
    import torch
    import exact_io_aware_60_amd as fa

    fa.lib()
    w = ai.DECODE_WORKLOADS[args.decode]
    inp = ai.make_decode_inputs(w)

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    q, k, v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
    del inp
    lens = ai.decode_seqlens(w)
    sl = None if lens is None else torch.as_tensor(lens).cuda()
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device=q.device)
    ws_bytes = fa.decode_workspace_size(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, w.causal)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=q.device)
    # 512 MiB of floats, summed (read once, nothing written back) before each call
    flush = torch.zeros(128 << 20, dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    args_c = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
              None if sl is None else sl.data_ptr(), w.B, w.Hq, w.Hkv, w.Nq, w.Nk,
              w.d, w.causal, w.scale, ws.data_ptr(), ws_bytes, sp)

    def call():
        st = fa.decode_raw(*args_c)
        if st != 0:
            raise RuntimeError(f"decode: {fa.strerror(st)}")

    for _ in range(args.warmup):
        flush.sum()
        call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s in range(args.steps):
        flush.sum()
        ev[s][0].record(stream)
        call()
        ev[s][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    times = [a.elapsed_time(b) for a, b in ev]
    ms = sum(times) / len(times)
    copy_calibration(args.copy_calibration, q.device)
    nbytes = decode_bytes(w)
    gbs = nbytes / (ms * 1e-3) / 1e9
    out = {
        "metric": "decode step HBM throughput (bf16 K/V cache read once)",
        "value": gbs,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
                   "causal": w.causal, "passes": "decode",
                   "keys_in_use": None if lens is None else int(lens.sum())},
        "ms_min": min(times),
        "wall_ms_per_step": wall / args.steps * 1e3,
        "roofline": {"bound": "hbm", "kernel": "decode (range kernel + merge)", "achieved": gbs,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                     "traffic": measured_traffic("decode", w.name),
                     "traffic_unit": "bytes per call (HBM read + write, rocprofv3 counters)",
                     "avg_launch_ms": ms, "algorithmic_bytes_per_launch": nbytes},
        "workspace_bytes": ws_bytes,
        "device": torch.cuda.get_device_name(0),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = decode_cpu_baseline(w)
    print(json.dumps(out), flush=True)
    return 0


def window_main(args) -> int:
    import torch
    import exact_io_aware_60_amd as fa

    fa.lib()
    w = ai.WORKLOADS[WORKLOAD]
    W = int(args.window)
    inp = ai.make_inputs(w)

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    q, k, v, do = dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["do"])
    del inp
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_bytes = fa.bwd_workspace_size(w.B, w.Hq, w.Hkv, w.N, w.d, True)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    P = [t.data_ptr() for t in (q, k, v, o, lse, do, dq, dk, dv)]

    def fwd():
        st = fa.fwd_window_raw(P[0], P[1], P[2], P[3], P[4], w.B, w.Hq, w.Hkv, w.N, w.d, W, w.scale, sp)
        if st != 0:
            raise RuntimeError(f"fwd_window: {fa.strerror(st)}")

    def bwd():
        st = fa.bwd_window_raw(*P, w.B, w.Hq, w.Hkv, w.N, w.d, W, w.scale, ws.data_ptr(), ws_bytes, sp)
        if st != 0:
            raise RuntimeError(f"bwd_window: {fa.strerror(st)}")

    for _ in range(args.warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        ev[s_][0].record(stream)
        fwd()
        ev[s_][1].record(stream)
        bwd()
        ev[s_][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    bwd_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps
    ms_avg = fwd_ms + bwd_ms
    n = np.arange(w.N, dtype=np.float64)
    pairs = w.B * w.Hq * float(np.minimum(n + 1, W).sum())
    flop = 4.0 * w.d * pairs
    tflops = flop / (fwd_ms * 1e-3) / 1e12
    step_tflops = 3.5 * flop / (ms_avg * 1e-3) / 1e12
    out = {
        "metric": "attention fwd/bwd TFLOP/s with a sliding-window causal mask (bf16) and % of MI355X bf16 MFMA peak",
        "value": step_tflops,
        "passes": {"fwd": {"ms": fwd_ms, "tflops": tflops, "frac_of_peak": tflops / PEAK_BF16_TFLOPS},
                   "bwd": {"ms": bwd_ms, "tflops": 2.5 * flop / (bwd_ms * 1e-3) / 1e12,
                           "frac_of_peak": 2.5 * flop / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}},
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_avg,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_FWD_BWD,
        "precision": PRECISION,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "d": w.d, "window": W,
                   "passes": "fwd+bwd (sliding window)"},
        "wall_ms_per_step": wall / args.steps * 1e3,
        "roofline": {"bound": "mfma", "kernel": "fwd_kernel (window)", "achieved": tflops, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": tflops / PEAK_BF16_TFLOPS, "traffic": None,
                     "avg_launch_ms": fwd_ms, "algorithmic_flop_per_launch": flop},
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(out), flush=True)
    return 0


def varlen_main(args) -> int:
    import torch
    import exact_io_aware_60_amd as fa

    fa.lib()
    w = ai.VARLEN_WORKLOADS[args.varlen]
    inp = ai.make_varlen_inputs(w)

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    q, k, v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
    do = torch.randn_like(q)
    lens = inp["lengths"]
    cu = torch.as_tensor(inp["cu_seqlens"]).cuda()
    del inp
    total, ms = int(lens.sum()), int(lens.max())
    o = torch.empty_like(q)
    lse = torch.empty((w.Hq, total), dtype=torch.float32, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_bytes = fa.bwd_workspace_size(1, w.Hq, w.Hkv, total, w.d, True)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    args_c = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), cu.data_ptr(), len(lens), ms,
              total, w.Hq, w.Hkv, w.d, w.causal, w.scale, sp)
    args_b = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(), dq.data_ptr(),
              dk.data_ptr(), dv.data_ptr(), cu.data_ptr(), len(lens), ms, total, w.Hq, w.Hkv, w.d, w.causal, w.scale,
              ws.data_ptr(), ws_bytes, sp)

    def call():
        st = fa.fwd_varlen_raw(*args_c)
        if st != 0:
            raise RuntimeError(f"fwd_varlen: {fa.strerror(st)}")

    def call_b():
        st = fa.bwd_varlen_raw(*args_b)
        if st != 0:
            raise RuntimeError(f"bwd_varlen: {fa.strerror(st)}")

    for _ in range(args.warmup):
        call()
        call_b()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        ev[s_][0].record(stream)
        call()
        ev[s_][1].record(stream)
        call_b()
        ev[s_][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    bwd_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps
    ms_avg = fwd_ms + bwd_ms
    pairs = float(sum(int(n) * int(n) for n in lens)) / (2.0 if w.causal else 1.0)
    flop = 4.0 * w.Hq * w.d * pairs
    tflops = flop / (fwd_ms * 1e-3) / 1e12
    out = {
        "metric": "attention fwd/bwd TFLOP/s over packed sequences (bf16) and % of MI355X bf16 MFMA peak",
        "value": 3.5 * flop / (ms_avg * 1e-3) / 1e12,
        "passes": {"fwd": {"ms": fwd_ms, "tflops": tflops, "frac_of_peak": tflops / PEAK_BF16_TFLOPS},
                   "bwd": {"ms": bwd_ms, "tflops": 2.5 * flop / (bwd_ms * 1e-3) / 1e12,
                           "frac_of_peak": 2.5 * flop / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}},
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_avg,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_FWD_BWD,
        "precision": PRECISION,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "total": total, "max_seqlen": ms,
                   "min_len": int(lens.min()), "d": w.d, "causal": w.causal, "passes": "fwd+bwd (packed sequences)"},
        "wall_ms_per_step": wall / args.steps * 1e3,
        "roofline": {"bound": "mfma", "kernel": "fwd_kernel (packed)", "achieved": tflops, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": tflops / PEAK_BF16_TFLOPS, "traffic": None,
                     "avg_launch_ms": fwd_ms, "algorithmic_flop_per_launch": flop},
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(out), flush=True)
    return 0


# MI355X dense FP8 (E4M3) MFMA peak: twice the bf16 rate.
PEAK_FP8_TFLOPS = 2 * PEAK_BF16_TFLOPS


def fp8_main(args) -> int:
    """The forward on E4M3 inputs (flash_attn_fwd_e4m3) at a fixed-length
    workload's shape: quantised once before the timed region (the quantisers
    are timed apart), then the forward kernel alone in the timed steps, against
    the FP8 MFMA peak."""
    import torch
    import exact_io_aware_60_amd as fa

    fa.lib()
    w = ai.WORKLOADS[args.fp8]
    rows = 128
    inp = ai.make_inputs(w, with_grad=False)

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    q, k, v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
    del inp
    stream = torch.cuda.current_stream()
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    for _ in range(2):
        e0.record(stream)
        q8, qs = fa.quantize_e4m3(q, rows)
        k8, ks = fa.quantize_e4m3(k, rows)
        e1.record(stream)
        v8t, vs = fa.quantize_e4m3_vt(v, rows)
        e2.record(stream)
    torch.cuda.synchronize()
    quant_ms = {"q_and_k": e0.elapsed_time(e1), "v_transposed": e1.elapsed_time(e2)}
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=q.device)
    P = [t.data_ptr() for t in (q8, qs, k8, ks, v8t, vs, o, lse)]
    sp = stream.cuda_stream

    def fwd():
        st = fa.fwd_e4m3_raw(*P, w.B, w.Hq, w.Hkv, w.N, w.d, w.causal, w.scale, rows, sp)
        if st != 0:
            raise RuntimeError(f"fwd_e4m3: {fa.strerror(st)}")

    for _ in range(args.warmup):
        fwd()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        ev[s_][0].record(stream)
        fwd()
        ev[s_][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    copy_calibration(args.copy_calibration, q.device)
    flop = algorithmic(w)["fwd"][1]
    tflops = flop / (ms * 1e-3) / 1e12
    out = {
        "metric": "attention fwd TFLOP/s on E4M3 inputs (FP8 MFMA, causal) and % of MI355X FP8 MFMA peak",
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3",
        "precision": {"io": "E4M3 codes with fp32 run scales in, bf16 O, fp32 LSE",
                      "mfma": "e4m3 x e4m3 -> fp32 (S and P.V; P rounded to e4m3)", "softmax": "fp32"},
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "d": w.d, "causal": w.causal,
                   "passes": "fwd (e4m3)", "rows_per_scale": rows},
        "quantize_ms": quant_ms,
        "wall_ms_per_step": wall / args.steps * 1e3,
        "roofline": {"bound": "mfma", "kernel": "fwd8_kernel", "achieved": tflops, "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": tflops / PEAK_FP8_TFLOPS,
                     "traffic": measured_traffic("fwd8", w.name),
                     "traffic_unit": "bytes per launch (HBM read + write, rocprofv3 counters)",
                     "avg_launch_ms": ms, "algorithmic_flop_per_launch": flop},
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(out), flush=True)
    return 0


# MI355X dense fp32 matrix peak (the rated figure; a sixteenth of the bf16 rate).
PEAK_FP32_TFLOPS = 157.3


def f32_main(args) -> int:
    """The forward on fp32 inputs (flash_attn_fwd_f32) at a fixed-length
    workload's shape (the fp32 draws, not rounded), against the fp32 matrix peak."""
    import torch
    import exact_io_aware_60_amd as fa

    fa.lib()
    w = ai.WORKLOADS[args.f32]
    if w.d > 128:
        print(f"--f32 takes head dimensions up to 128; {w.name} has d = {w.d}", file=sys.stderr)
        return 2

    def draw(t, shape):
        return torch.from_numpy(ai.normal_f32(shape, 9100 + w.cfg_id, t)).cuda()

    q = draw(0, (w.B, w.Hq, w.N, w.d))
    k, v = draw(1, (w.B, w.Hkv, w.N, w.d)), draw(2, (w.B, w.Hkv, w.N, w.d))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    P = [t.data_ptr() for t in (q, k, v, o, lse)]

    def fwd():
        st = fa.fwd_f32_raw(*P, w.B, w.Hq, w.Hkv, w.N, w.d, w.causal, w.scale, sp)
        if st != 0:
            raise RuntimeError(f"fwd_f32: {fa.strerror(st)}")

    for _ in range(args.warmup):
        fwd()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        ev[s_][0].record(stream)
        fwd()
        ev[s_][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    copy_calibration(args.copy_calibration, q.device)
    flop = algorithmic(w)["fwd"][1]
    tflops = flop / (ms * 1e-3) / 1e12
    out = {
        "metric": "attention fwd TFLOP/s on fp32 inputs (fp32 MFMA) and % of MI355X fp32 MFMA peak",
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "precision": {"io": "fp32 q, k, v in; fp32 O and LSE out", "mfma": "fp32 x fp32 -> fp32", "softmax": "fp32"},
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "d": w.d, "causal": w.causal,
                   "passes": "fwd (fp32)"},
        "wall_ms_per_step": wall / args.steps * 1e3,
        "roofline": {"bound": "mfma", "kernel": "fwd32_kernel", "achieved": tflops, "peak": PEAK_FP32_TFLOPS,
                     "unit": "TFLOP/s", "frac": tflops / PEAK_FP32_TFLOPS, "traffic": None,
                     "avg_launch_ms": ms, "algorithmic_flop_per_launch": flop},
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the second of repeated steps after the timed ones that samples the engine clock "
                         "(profiled runs then hold only the warm-up and timed launches)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run a plain device copy of MIB MiB (3 times) after the timed steps, so that one "
                         "profiled run holds the reference kernel for scaling the FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--decode", choices=sorted(ai.DECODE_WORKLOADS), default=None,
                    help="measure the decode path on this workload instead of the forward + backward step")
    ap.add_argument("--window", type=int, default=0, metavar="W",
                    help="measure the gqa16k forward under a sliding-window causal mask of W keys instead")
    ap.add_argument("--flush-mib", type=int, default=0, metavar="MIB",
                    help="before each timed step, write MIB MiB of scratch memory (outside the step's events), so "
                         "that no input is still in the last-level cache; default 0: warm")
    ap.add_argument("--workload", choices=sorted(ai.WORKLOADS), default=WORKLOAD,
                    help="the fixed-length workload of the step (default gqa16k); workloads without a backward "
                         "pass time the forward alone")
    ap.add_argument("--varlen", choices=sorted(ai.VARLEN_WORKLOADS), default=None,
                    help="measure the forward pass over this packed variable-length workload instead")
    ap.add_argument("--f32", choices=sorted(ai.WORKLOADS), default=None,
                    help="measure the forward on fp32 inputs (flash_attn_fwd_f32) at this workload's shape instead")
    ap.add_argument("--fp8", choices=sorted(ai.WORKLOADS), default=None,
                    help="measure the forward on E4M3 inputs (flash_attn_fwd_e4m3) at this workload's shape instead")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: the attention path here is single-GPU (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        return 2
    if args.decode:
        import torch
        if not torch.cuda.is_available():
            print("bench.py needs a GPU", file=sys.stderr)
            return 2
        return decode_main(args)
    if args.window > 0:
        import torch
        if not torch.cuda.is_available():
            print("bench.py needs a GPU", file=sys.stderr)
            return 2
        return window_main(args)
    if args.varlen:
        import torch
        if not torch.cuda.is_available():
            print("bench.py needs a GPU", file=sys.stderr)
            return 2
        return varlen_main(args)
    if args.f32:
        import torch
        if not torch.cuda.is_available():
            print("bench.py needs a GPU", file=sys.stderr)
            return 2
        return f32_main(args)
    if args.fp8:
        import torch
        if not torch.cuda.is_available():
            print("bench.py needs a GPU", file=sys.stderr)
            return 2
        return fp8_main(args)

    import torch
    import exact_io_aware_60_amd as fa

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    fa.lib()
    w = ai.WORKLOADS[args.workload]
    nk = 4 if w.backward else 1          # launches per step: fwd (+ bwd preparation, dQ, dK/dV)
    B, Hq, Hkv, N, d = w.B, w.Hq, w.Hkv, w.N, w.d
    inp = ai.make_inputs(w)

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    q, k, v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
    do = dev(inp["do"]) if w.backward else torch.empty_like(q)
    del inp
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    if w.backward:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws_bytes = fa.bwd_workspace_size(B, Hq, Hkv, N, d, w.causal)
    else:
        dq = dk = dv = o                 # never written: the step is the forward alone
        ws_bytes = 256
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    ptrs = [t.data_ptr() for t in (q, k, v, o, lse, do, dq, dk, dv)]

    def call(i: int) -> None:
        if i == 0:
            st = fa.fwd_raw(ptrs[0], ptrs[1], ptrs[2], ptrs[3], ptrs[4], B, Hq, Hkv, N, d, w.causal, w.scale, sp)
        else:
            st = fa.bwd_stage_raw(i - 1, *ptrs, B, Hq, Hkv, N, d, w.causal, w.scale, ws.data_ptr(), ws_bytes, sp)
        if st != 0:
            raise RuntimeError(f"{KERNELS[i]}: {fa.strerror(st)}")

    for _ in range(args.warmup):
        for i in range(nk):
            call(i)
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nk + 1)] for _ in range(args.steps)]
    scratch = torch.empty(args.flush_mib << 20, dtype=torch.uint8, device=q.device) if args.flush_mib > 0 else None
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        if scratch is not None:
            scratch.fill_(s & 0xFF)
        ev[s][0].record(stream)
        for i in range(nk):
            call(i)
            ev[s][i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    ktime = {name: 0.0 for name in KERNELS[:nk]}
    for s in range(args.steps):
        for i, name in enumerate(KERNELS[:nk]):
            ktime[name] += ev[s][i].elapsed_time(ev[s][i + 1])
    kavg = {name: t / args.steps for name, t in ktime.items()}
    step_ms = sum(ev[s][0].elapsed_time(ev[s][nk]) for s in range(args.steps)) / args.steps
    fwd_flop = 4.0 * B * Hq * N * N * d / (2.0 if w.causal else 1.0)
    bwd_flop = 2.5 * fwd_flop if w.backward else 0.0
    fwd_ms = kavg["fwd"]
    bwd_ms = kavg["bwd_pre"] + kavg["bwd_dkdv"] + kavg["bwd_dq"] if w.backward else None
    value = (fwd_flop + bwd_flop) / step_ms / 1e9

    def one_step():
        for i in range(nk):
            call(i)

    clock = None if args.no_clock else sustained_clock(one_step, step_ms)

    copy_calibration(args.copy_calibration, q.device)

    alg = algorithmic(w)
    dom = max(("fwd", "bwd_dkdv", "bwd_dq")[:3 if w.backward else 1], key=lambda n: kavg[n])
    kind, amount = alg[dom]
    achieved = amount / (kavg[dom] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS, "traffic": measured_traffic(dom, w.name),
                "traffic_unit": "bytes per launch (HBM read + write, rocprofv3 counters)",
                "avg_launch_ms": kavg[dom], "algorithmic_flop_per_launch": amount}
    # fraction of the peak at the clock the GPU actually ran at (sampled mean)
    adj = (clock["mean_mhz"] / RATED_MHZ) if clock else None
    if adj:
        roofline["frac_clock_adjusted"] = roofline["frac"] / adj

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_FWD_BWD if w.backward else "bf16",
        "precision": PRECISION if w.backward else PRECISION_FWD,
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "Hq": Hq, "Hkv": Hkv, "N": N, "d": d, "causal": w.causal,
                   "passes": "fwd+bwd" if w.backward else "fwd",
                   "cache": f"flushed ({args.flush_mib} MiB written before each step)" if args.flush_mib else "warm"},
        "passes": {
            "fwd": {"ms": fwd_ms, "tflops": fwd_flop / fwd_ms / 1e9,
                    "frac_of_peak": fwd_flop / fwd_ms / 1e9 / PEAK_BF16_TFLOPS,
                    "frac_of_clock_adjusted_peak": fwd_flop / fwd_ms / 1e9 / PEAK_BF16_TFLOPS / adj if adj else None},
            "bwd": None if not w.backward else {
                "ms": bwd_ms, "tflops": bwd_flop / bwd_ms / 1e9,
                "frac_of_peak": bwd_flop / bwd_ms / 1e9 / PEAK_BF16_TFLOPS,
                "frac_of_clock_adjusted_peak": bwd_flop / bwd_ms / 1e9 / PEAK_BF16_TFLOPS / adj if adj else None},
        },
        "clock": clock,
        "kernel_ms": kavg,
        "wall_ms_per_step": wall / args.steps * 1e3,
        "roofline": roofline,
        "device": torch.cuda.get_device_name(0),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
