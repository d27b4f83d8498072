#!/usr/bin/env python3
"""Benchmark the MI355X attention forward; prints ONE JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3]

A step is one ``attn_fwd`` call over the whole workload (every step of the
fused forward: Q tile load, K/V streaming, QK^T, online softmax, PV, O and
lse stores), on inputs already resident in device memory.  The default
workload is B=2, H=16, N=4096, d=128 bf16 (the 4096-length case whose
4096x4096 score matrix must never be materialised); ``--workload`` selects any
of the five synthetic workloads.

Timing: with --warmup W, first --settle seconds (0.25 by default) of untimed
back-to-back launches, then W untimed warmup launches; without it, the
automatic warmup below.  Then exactly K launches back to back on
torch's current stream, bracketed by torch.cuda.synchronize() on both sides
(wall clock for ms_per_step) and by two HIP events recorded on that same
stream just before the first and just after the last launch (mean kernel
duration for the roofline).  The launches go through a plan that marshals the
arguments once, so the host keeps ahead of the GPU.  After the timed region,
single launches are timed one by one for p20 / median / p80 (kernel_ms), and
for the two small workloads also after a 512 MB write that evicts L2 and the
Infinity Cache (kernel_ms.cold).

Roofline: flops = 4*B*H*N^2*d per launch against the dense bf16/fp16 MFMA
peak of 2500 TFLOP/s (fp32 workloads: 157.3 TFLOP/s fp32 matrix peak).
``traffic`` is read from profiles/traffic.json (rocprofv3 FETCH_SIZE and
WRITE_SIZE counters, calibrated against a plain copy) and reported only while
the kernel source is unchanged since those counters were taken.

cpu_baseline: the fp64 CPU oracle, as it stands, timed on this host's cores on
a bounded sample of the same workload (whole heads until ~10 s have passed).

clock: while the timed launches run, a thread samples the shader clock the
driver reports (the current level of sysfs pp_dpm_sclk) and the socket power
(hwmon power1_input); ``frac_at_clock`` relates the achieved rate to the peak
at that clock (the spec peaks are quoted at 2.4 GHz).  From an idle GPU the
throughput takes some 25 ms of back-to-back launches to settle, hence the
defaults: at least 0.3 s of warmup launches, then about 1 s of timed ones
(both at least 200; --warmup and --steps set exact counts, and an explicit
--warmup count is preceded by the settle phase, reported as ``settle``).
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}
METRIC = "attention fwd TFLOP/s (4·B·H·N²·d) and % of MI355X bf16 MFMA peak"
METRIC_CAUSAL = "attention fwd causal TFLOP/s (4·B·H·d·N(N+1)/2) and % of MI355X bf16 MFMA peak"
METRIC_BWD = "attention bwd TFLOP/s (10·B·H·N²·d) and % of MI355X bf16 MFMA peak"
METRIC_BWD_CAUSAL = "attention bwd causal TFLOP/s (10·B·H·d·N(N+1)/2) and % of MI355X bf16 MFMA peak"
METRIC_DECODE = ("attention decode GB/s (Q, K, V read once, O and lse written once) "
                 "and % of MI355X HBM peak")
HBM_PEAK_GBPS = 8000.0
KERNEL_SRCS = [os.path.join(ROOT, "attention_attn_fwd_07_amd", "csrc", f)
               for f in ("attn_fwd.hip", "attn_common.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_hash() -> str:
    """Hash of the forward kernels' sources (the code the profiles describe)."""
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(w) -> int:
    """Q, K, V read once, O written once, lse written once."""
    return 4 * w.B * w.H * w.N * w.d * w.elem_bytes + 4 * w.B * w.H * w.N


def decode_bytes(w: dict) -> int:
    """Algorithmic bytes of a call with N queries against Nk keys: Q, K and V
    read once, O and lse written once."""
    e = 4 if w["dtype"] == "f32" else 2
    B, H, N, Nk, d = w["B"], w["H"], w["N"], w["Nk"], w["d"]
    return 2 * B * H * Nk * d * e + 2 * B * H * N * d * e + 4 * B * H * N


def decode_splits(w: dict) -> int:
    """Key splits for a decode-shaped call (few queries, many keys): enough
    (head, split) blocks for about two per compute unit, at most 64 splits and
    at most one per 64-key tile."""
    bh = w["B"] * w["H"]
    tiles = (w["Nk"] + 63) // 64
    return max(1, min(64, tiles, -(-512 // bh)))


def traffic_for(w):
    """Measured HBM bytes per launch, if counters exist for this exact kernel."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    key = w["key"] if isinstance(w, dict) else str(w.key)
    entry = rec.get("workloads", {}).get(key)
    if not entry or rec.get("kernel_sha256_16") != kernel_source_hash():
        return None
    return entry.get("hbm_bytes_per_launch")


def cpu_baseline(w, q, k, v, budget_s: float = 10.0):
    """Time the oracle on a bounded sample of the workload.

    Units of work are whole heads (N <= 8192) or 512-query-row slices of a head
    (longer sequences), each against all N keys, taken in order until the
    budget is used.  The rate is scaled to the metric's unit (TFLOP/s of the
    4*rows*N*d algorithmic flops the sample covers).
    """
    import numpy as np

    import oracle

    cores = len(os.sched_getaffinity(0))
    q64, k64, v64 = (t.double().numpy() for t in (q, k, v))
    rows_per_unit = w.N if w.N <= 8192 else 512
    done, t0 = 0, time.perf_counter()
    for b in range(w.B):
        for h in range(w.H):
            for r0 in range(0, w.N, rows_per_unit):
                rows = np.arange(r0, min(w.N, r0 + rows_per_unit))
                idx = np.stack([np.full(len(rows), b), np.full(len(rows), h), rows], axis=1)
                oracle.attention_rows(q64, k64, v64, w.scale, idx, workers=cores)
                done += len(rows)
                if time.perf_counter() - t0 >= budget_s:
                    break
            else:
                continue
            break
        else:
            continue
        break
    dt = time.perf_counter() - t0
    total = w.B * w.H * w.N
    return {"value": round(4.0 * done * w.N * w.d / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": cores, "kind": "oracle",
            "sample": f"{done} of {total} query rows (units of {rows_per_unit} rows of one head),"
                      f" each against all {w.N} keys; fp64 numpy on {cores} threads; {dt:.1f} s",
            "full_workload_seconds_extrapolated": round(dt * total / done, 1)}


def per_launch_ms(launch, stream, reps: int, flush=None) -> dict:
    """Kernel time of single launches (HIP events on the launch stream around
    each one), as p20 / median / p80 in ms.  With ``flush``, it runs before
    every launch (outside the events) to evict L2 and the Infinity Cache."""
    import torch
    times = []
    for _ in range(reps):
        if flush is not None:
            flush()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        launch()
        e1.record(stream)
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    times.sort()

    def pct(p):
        return round(times[min(len(times) - 1, int(p * len(times)))], 5)
    return {"p20": pct(0.2), "median": pct(0.5), "p80": pct(0.8), "n": len(times)}


SPEC_CLOCK_MHZ = 2400.0


def gpu_sysfs_dir():
    """The GPU's sysfs device directory: the one card that reports shader clock
    levels (None if there is none, or several, which could not be told apart)."""
    cards = [d for d in sorted(glob.glob("/sys/class/drm/card*/device"))
             if os.path.exists(os.path.join(d, "pp_dpm_sclk"))]
    return cards[0] if len(cards) == 1 else None


def parse_sclk(text: str):
    """Current shader clock in MHz from pp_dpm_sclk (the starred line)."""
    m = re.search(r"(\d+)\s*Mhz\s*\*", text, re.IGNORECASE)
    return float(m.group(1)) if m else None


class ClockSampler:
    """Samples the shader clock and the socket power from sysfs on a thread,
    every ``period_s`` seconds between __enter__ and __exit__."""

    def __init__(self, period_s: float = 0.002, sysfs_dir=None):
        self.dir = sysfs_dir if sysfs_dir is not None else gpu_sysfs_dir()
        self.period = period_s
        self.sclk, self.power = [], []
        self.window_s = 0.0
        self._stop = threading.Event()
        self._thread = None
        hw = sorted(glob.glob(os.path.join(self.dir, "hwmon", "hwmon*"))) if self.dir else []
        self._hwmon = hw[0] if hw else None

    def _read(self, path):
        try:
            with open(path) as f:
                return f.read()
        except OSError:
            return None

    def _loop(self):
        while not self._stop.is_set():
            t = self._read(os.path.join(self.dir, "pp_dpm_sclk"))
            f = parse_sclk(t) if t else None
            if f is not None:
                self.sclk.append(f)
            if self._hwmon:
                pw = self._read(os.path.join(self._hwmon, "power1_input"))
                if pw and pw.strip().isdigit():
                    self.power.append(int(pw) * 1e-6)
            self._stop.wait(self.period)

    def __enter__(self):
        self._t0 = time.perf_counter()
        if self.dir:
            self._thread = threading.Thread(target=self._loop, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread:
            self._thread.join()
        self.window_s = time.perf_counter() - self._t0
        return False

    # The driver's clock and power figures are averages over its own window of
    # some tenths of a second: over a shorter run they still describe the idle
    # GPU before it (a 6 ms run once read 345 MHz while it ran at well over
    # 1.5 GHz), so below this window nothing measured is reported.
    MIN_WINDOW_S = 0.25

    def summary(self, achieved: float, peak: float):
        """Mean clock and power over the samples, and the achieved rate as a
        fraction of the peak at the mean clock; None without samples.  For a
        window shorter than MIN_WINDOW_S the clock, power and fraction fields
        are null (only the window and the sample count are given)."""
        if not self.sclk:
            return None
        cap = self._read(os.path.join(self._hwmon, "power1_cap")) if self._hwmon else None
        out = {"sclk_mhz": None, "sclk_mhz_min": None, "sclk_mhz_max": None,
               "samples": len(self.sclk), "window_s": round(self.window_s, 3),
               "power_w": None,
               "power_cap_w": (round(int(cap) * 1e-6, 1) if cap and cap.strip().isdigit()
                               else None),
               "peak_at_clock": None, "frac_at_clock": None,
               "source": "sysfs pp_dpm_sclk (current level), hwmon power1_input"}
        if self.window_s < self.MIN_WINDOW_S:
            out["note"] = (f"window under {self.MIN_WINDOW_S} s: the driver's clock and power "
                           "averages would describe the idle GPU before the run")
            return out
        f = sum(self.sclk) / len(self.sclk)
        peak_f = peak * f / SPEC_CLOCK_MHZ
        out.update({"sclk_mhz": round(f, 1), "sclk_mhz_min": min(self.sclk),
                    "sclk_mhz_max": max(self.sclk),
                    "power_w": (round(sum(self.power) / len(self.power), 1) if self.power
                                else None),
                    "peak_at_clock": round(peak_f, 1),
                    "frac_at_clock": round(achieved / peak_f, 4)})
        return out


def time_batch(launch, n: int) -> float:
    """Seconds for n back-to-back launches (synchronised on both sides)."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n):
        launch()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def auto_warmup(launch, min_launches: int, min_seconds: float):
    """Untimed launches in batches of 20 until at least ``min_launches`` and
    ``min_seconds`` have passed (the shader clock ramps up from idle over the
    first tens of milliseconds of load).  Returns (launches, seconds per
    launch in the last batch)."""
    n, t, last = 0, 0.0, 0.0
    while n < min_launches or t < min_seconds:
        last = time_batch(launch, 20)
        n += 20
        t += last
    return n, last / 20


def timed_launches(launch, stream, steps, warmup, settle_s=0.0):
    """W untimed launches (``warmup``, or the automatic warmup), then exactly K
    (``steps``, or about 1 s of them, at least 200) back to back, bracketed by
    torch.cuda.synchronize() for the wall clock and by two HIP events on the
    launch stream for the mean kernel time.  With an explicit ``warmup`` count,
    ``settle_s`` seconds of untimed back-to-back launches come first, so that
    a short timed region does not fall inside the power manager's ramp from
    idle (the automatic warmup is already that long).  Returns (W, K, kernel ms
    per launch, wall ms per launch, the clock sampler of the timed region, the
    settle phase as {"launches", "seconds"} or None)."""
    import torch
    settle = None
    if warmup is not None and settle_s > 0:
        n, _ = auto_warmup(launch, min_launches=0, min_seconds=settle_s)
        settle = {"launches": n, "seconds": settle_s}
    if warmup is not None:
        W = warmup
        t_w = time_batch(launch, W) if W > 0 else 0.0
        per_launch_s = t_w / W if W > 0 else None
    else:
        W, per_launch_s = auto_warmup(launch, min_launches=200, min_seconds=0.3)
    if steps is not None:
        K = steps
    else:
        K = 200 if per_launch_s is None else max(200, min(100000, int(1.0 / per_launch_s)))
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with ClockSampler() as clock:
        t0 = time.perf_counter()
        ev0.record(stream)
        for _ in range(K):
            launch()
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    return W, K, ev0.elapsed_time(ev1) / K, wall * 1e3 / K, clock, settle


def calibrate_copy(nbytes: int, reps: int) -> None:
    """A plain device copy of known size, for scaling the HBM byte counters."""
    import torch
    n = nbytes // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "reps": reps}))


def cpu_baseline_decode(w: dict, q, k, v, scale: float, budget_s: float = 10.0):
    """The oracle on whole heads of the decode workload until the budget is
    used, as GB/s of the algorithmic bytes of the heads done."""
    import numpy as np

    import oracle

    cores = len(os.sched_getaffinity(0))
    q64, k64, v64 = (t.double().numpy() for t in (q, k, v))
    heads = [(b, h) for b in range(w["B"]) for h in range(w["H"])]
    done, t0 = 0, time.perf_counter()
    for (b, h) in heads:
        idx = np.stack([np.full(w["N"], b), np.full(w["N"], h), np.arange(w["N"])], axis=1)
        oracle.attention_rows(q64, k64, v64, scale, idx, workers=cores)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    per_head = decode_bytes(w) / len(heads)
    return {"value": round(done * per_head / dt / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{done} of {len(heads)} heads, each {w['N']} query row(s) against all "
                      f"{w['Nk']} keys; fp64 numpy on {cores} threads; {dt:.2f} s"}


def run_decode(args) -> int:
    """The decode workload through attn_fwd_splitkv: one JSON line in GB/s."""
    import numpy as np
    import torch

    import attention_attn_fwd_07_amd as attn
    import datagen

    w = dict(datagen.DECODE, key="decode")
    q, k, v = datagen.make_qkv_kv(w["B"], w["H"], w["N"], w["Nk"], w["d"], w["dtype"], w["seed"])
    scale = float(np.float32(1.0 / np.sqrt(w["d"])))
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty(qd.shape[:3], dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    splits = args.splitkv or decode_splits(w)
    nbytes_ws = attn.splitkv_workspace_size(w["B"], w["H"], w["N"], w["d"], splits, w["Nk"])
    ws = torch.empty(max(1, nbytes_ws // 4), dtype=torch.float32, device=dev)
    launch = attn.plan(qd, kd, vd, o, lse, scale, stream, splits=splits, workspace=ws)
    W, K, kern_ms, ms_per_step, clock, settle = timed_launches(launch, stream, args.steps,
                                                               args.warmup, args.settle)
    dist = per_launch_ms(launch, stream, max(10, min(K, 50)))
    flushbuf = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold = per_launch_ms(launch, stream, 20, flush=lambda: flushbuf.fill_(1))
    del flushbuf
    nbytes = decode_bytes(w)
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (kern_ms * 1e-3) / 1e9
    clk = clock.summary(achieved, HBM_PEAK_GBPS)
    if clk is not None:  # the clock-scaled peak is a compute figure: not for HBM
        clk["peak_at_clock"] = clk["frac_at_clock"] = None
    line = {
        "metric": METRIC_DECODE,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1, "steps": K, "warmup": W, "settle": settle,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w["dtype"], "data": "synthetic",
        "config": {"workload": w["name"], "B": w["B"], "H": w["H"], "N": w["N"],
                   "Nk": w["Nk"], "d": w["d"], "dtype": w["dtype"], "scale": scale,
                   "values": "N(0,1)", "mode": f"fwd split-KV S={splits}", "causal": False},
        "pct_of_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "kernel_ms": dict({"mean": round(kern_ms, 5)}, **dist, cold=cold),
        "algorithmic_bytes": nbytes,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic_for(w)},
        "clock": clk,
        "kernel_sha256_16": kernel_source_hash(),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_decode(w, q, k, v, scale, args.cpu_budget)
    print(json.dumps(line), flush=True)
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed launches (default: enough for about 1 s, at least 200)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed launches first (default: about 0.3 s of them, at least 200)")
    ap.add_argument("--settle", type=float, default=0.25, metavar="SECONDS",
                    help="with --warmup W: untimed back-to-back launches for this long before "
                         "the W warmup launches (from an idle GPU the throughput takes some "
                         "25 ms of load to settle); 0 times the ramp as well")
    ap.add_argument("--workload", type=int, default=3, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing (profiling runs)")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain copy of BYTES (counter calibration)")
    ap.add_argument("--causal", action="store_true",
                    help="causal variant (flops counted over the N(N+1)/2 visible pairs)")
    ap.add_argument("--splitkv", type=int, default=0, metavar="S",
                    help="forward through attn_fwd_splitkv with S key splits (+ merge)")
    ap.add_argument("--decode", action="store_true",
                    help="one query per head against 65536 cached keys (B=1, H=32, d=128, "
                         "bf16) through the split-KV path; reported in GB/s against HBM")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward (dQ, dK, dV) instead of the forward; "
                         "flops counted as 10 B H N^2 d (the five products; N(N+1)/2 pairs "
                         "in place of N^2 when causal)")
    args = ap.parse_args(argv)
    if ((args.steps is not None and args.steps < 1) or (args.warmup is not None and args.warmup < 0)
            or not 0.0 <= args.settle <= 60.0):
        print("bench.py: --steps must be at least 1, --warmup at least 0 and --settle in "
              "[0, 60] seconds", file=sys.stderr)
        return 2

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this attention forward runs on one GPU; several-GPU runs are not "
              "supported (heads or batches would shard with no communication).",
              file=sys.stderr)
        return 2

    import torch

    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy, max(1, args.steps or 3))
        return 0

    import attention_attn_fwd_07_amd as attn
    import datagen

    if not torch.cuda.is_available():
        print("bench.py: no GPU available", file=sys.stderr)
        return 1
    if args.decode:
        return run_decode(args)
    w = datagen.WORKLOADS[args.workload]
    q, k, v = datagen.workload_inputs(w.key)
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty(qd.shape[:3], dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    # One checked plan: the timed loop only relaunches it, so host-side Python
    # work stays far below a kernel's duration and the GPU never waits on it.
    mode = "fwd"
    pairs = w.N * w.N if not args.causal else w.N * (w.N + 1) // 2  # visible (i, j)
    flops = 4 * w.B * w.H * pairs * w.d
    if args.backward:
        attn.fwd(qd, kd, vd, w.scale, causal=args.causal)  # warm the forward once
        o, lse = attn.fwd(qd, kd, vd, w.scale, causal=args.causal)
        g = datagen.make_grad(w.B, w.H, w.N, w.d, w.dtype, seed=w.key).to(dev)
        grads = [torch.empty_like(qd) for _ in range(3)]
        ws = torch.empty(attn.bwd_workspace_size(w.B, w.H, w.N, w.d) // 4, dtype=torch.float32,
                         device=dev)

        def launch():
            attn.attn_bwd(qd, kd, vd, o, lse, g, *grads, w.scale, ws, stream,
                          causal=args.causal)
        flops = 10 * w.B * w.H * pairs * w.d
        mode = "bwd"
    elif args.splitkv:
        ws = torch.empty(attn.splitkv_workspace_size(w.B, w.H, w.N, w.d, args.splitkv) // 4,
                         dtype=torch.float32, device=dev)
        launch = attn.plan(qd, kd, vd, o, lse, w.scale, stream, splits=args.splitkv,
                           workspace=ws)
        mode = f"fwd split-KV S={args.splitkv}"
    else:
        launch = attn.plan(qd, kd, vd, o, lse, w.scale, stream, causal=args.causal)
    if args.causal:
        mode += " causal"
    W, K, kern_ms, ms_per_step, clock, settle = timed_launches(launch, stream, args.steps,
                                                               args.warmup, args.settle)

    # After the timed region: the per-launch spread, and for the small
    # workloads the same with L2 and the 256 MB Infinity Cache flushed first
    # by writing a 512 MB buffer (cold inputs).
    dist = per_launch_ms(launch, stream, max(10, min(K, 50)))
    cold = None
    if w.key in (1, 2):
        flushbuf = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        cold = per_launch_ms(launch, stream, 20, flush=lambda: flushbuf.fill_(1))
        del flushbuf
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (kern_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]

    line = {
        "metric": ((METRIC_BWD_CAUSAL if args.causal else METRIC_BWD) if args.backward
                   else (METRIC_CAUSAL if args.causal else METRIC)),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "settle": settle,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": dict(w.describe(), mode=mode, causal=bool(args.causal)),
        "pct_of_peak": round(100.0 * value / peak, 2),
        "kernel_ms": dict({"mean": round(kern_ms, 5)}, **{k: v for k, v in dist.items()},
                          **({"cold": cold} if cold else {})),
        "hbm_gbps_algorithmic": (round(algorithmic_bytes(w) / (kern_ms * 1e-3) / 1e9, 1)
                                 if not args.backward else None),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": traffic_for(w) if mode == "fwd" else None},
        "clock": clock.summary(achieved, peak),
        "kernel_sha256_16": kernel_source_hash(),
    }
    if not args.no_cpu_baseline:
        if mode == "fwd":
            line["cpu_baseline"] = cpu_baseline(w, q, k, v, args.cpu_budget)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
