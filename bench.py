#!/usr/bin/env python3
"""Benchmark of the exact-attention hot path on one MI355X.

One step = one forward pass over the pages' headline workload
[B=16, N=1024, H=32, d=128] fp16, non-causal (inputs resident in HBM). The line
also carries the split-KV decode step at B=8, Nq=1, Nk=8192, Hq=32, Hkv=8,
d=128 bf16 with 16 splits, the forward at N=4096 (the 50%-of-peak target
shape), a packed variable-length batch, the backward pass, and a sweep over the
pages' other workloads (long sequences causal and not, the sharpened bf16
repeat, the GQA head-dim sweep, decode with Nq=8; inputs drawn on the device),
and a power probe: board power and clock while the N=4096 forward runs with
Gaussian and with constant Q, and while the headline runs.

Timing: the headline times exactly --steps steps between two HIP events (its
mean is `ms_per_step`); every other workload runs at least 50 steps and at least
one second. Each timed region is cut into blocks by events on the launch stream,
and the line reports the mean, the median and the minimum of the per-step times
of those blocks. Per-kernel durations of multi-kernel steps (decode, backward)
come from the HIP activity trace of torch.profiler over a few extra steps.

  python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_F16 = 2500.0     # TFLOP/s, MI355X dense fp16/bf16 (published)
PEAK_HBM = 8000.0          # GB/s, MI355X HBM3E (published)
METRIC = "attention fwd TFLOP/s (4·B·H·N²·d) & % MFMA peak; split-KV decode µs/step"
# RTX 3080, official FA2 kernel at [16,1024,32,128]: 5.32 ms ("ampere_flash_attention_from_scratch"
# README, Performance Test), i.e. 25.84 TFLOP/s under the page's 2·B·H·N²·d count, doubled
PAGES_HEADLINE_TFLOPS_4X = 51.68
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fa_fwd_headline_traffic.json")
KERNEL_SOURCES = ("fa_fwd_kernel.h", "fa_device.h", "fa_launch.h")
MIN_ITERS, MIN_SECONDS = 50, 1.0
TIMING = {"min_seconds": MIN_SECONDS}   # --min-seconds may lower it for profiler runs


def code_only(text: str) -> str:
    """C++ source with comments removed and whitespace collapsed: a comment edit
    leaves the kernel, and so its hash, unchanged."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def fwd_args_only(text: str) -> str:
    """The forward kernel's argument struct out of the launch header (the other
    kernels' argument structs there do not change the forward kernel)."""
    import re
    m = re.search(r"struct FwdArgs \{.*?\};", text, flags=re.S)
    return m.group(0) if m else text


def kernel_source_hash(read=None) -> str:
    """Hash of the forward kernel's code (comments and layout ignored)."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        path = os.path.join("exact_tiled_attention_21_amd", "csrc", f)
        if read is None:
            with open(os.path.join(ROOT, path), encoding="utf-8") as fh:
                text = fh.read()
        else:
            text = read(path)
        if f == "fa_launch.h":
            text = fwd_args_only(text)
        h.update(code_only(text).encode())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None if the
    kernel sources changed since they were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def prewarm(fn, seconds, torch):
    """Run fn for `seconds` of wall time before any counted step: the GPU raises
    its clocks over the first tens of milliseconds of sustained load, and the
    metric is the sustained rate."""
    if seconds <= 0:
        return
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


def progress(msg: str) -> None:
    """One line per finished leg on stderr (the JSON result is the only stdout line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def block_sizes(steps: int, blocks: int = 10):
    """Split `steps` into at most `blocks` nearly equal runs of consecutive steps."""
    blocks = max(1, min(blocks, steps))
    base, extra = divmod(steps, blocks)
    return [base + (1 if i < extra else 0) for i in range(blocks)]


def timed(fn, steps, warmup, torch, warm_s=0.0):
    """Exactly `steps` calls of fn(i) after warm-up, timed by HIP events on the current
    stream (the stream the library launches on). Events between blocks of steps give
    per-step times per block; returns the mean over all steps and the median and the
    minimum over the blocks, in ms."""
    prewarm(fn, warm_s, torch)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    sizes = block_sizes(steps)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(sizes) + 1)]
    i = 0
    ev[0].record()
    for b, n in enumerate(sizes):
        for _ in range(n):
            fn(i)
            i += 1
        ev[b + 1].record()
    torch.cuda.synchronize()
    per = [ev[b].elapsed_time(ev[b + 1]) / n for b, n in enumerate(sizes)]
    total = ev[0].elapsed_time(ev[-1])
    return {"mean_ms": total / steps, "median_ms": statistics.median(per), "min_ms": min(per),
            "steps": steps, "blocks": len(sizes)}


def timed_auto(fn, torch, warm_s, warmup=5):
    """At least MIN_ITERS steps and at least MIN_SECONDS of them (step count from a
    short trial run)."""
    prewarm(fn, warm_s, torch)
    trial = timed(fn, 10, 2, torch)
    n = max(MIN_ITERS, int(math.ceil(TIMING["min_seconds"] * 1e3 / max(trial["mean_ms"], 1e-4))))
    return timed(fn, min(n, 200000), warmup, torch)


def stats_fields(t, scale=1.0, unit="ms", digits=4):
    """mean / median / min of a timing, in `unit` (scale converts from ms)."""
    return {f"{unit}": round(t["mean_ms"] * scale, digits), f"median_{unit}": round(t["median_ms"] * scale, digits),
            f"min_{unit}": round(t["min_ms"] * scale, digits), "steps": t["steps"]}


def kernel_times(fn, n, torch):
    """Average device duration per launch of every kernel fn launches, in µs, from the
    HIP activity trace torch.profiler collects over n steps; None when the trace is
    unavailable (e.g. under another profiler)."""
    if os.environ.get("FA_BENCH_NO_KERNEL_TRACE"):
        return None
    try:
        from torch.profiler import ProfilerActivity, profile
        fn()
        torch.cuda.synchronize()
        with profile(activities=[ProfilerActivity.CUDA]) as prof:
            for i in range(n):
                fn(i)
            torch.cuda.synchronize()
        out = {}
        for e in prof.key_averages():
            name = e.key
            total = getattr(e, "device_time_total", None)
            if total is None:
                total = getattr(e, "cuda_time_total", 0.0)
            if "fa_" not in name or not total or not e.count:
                continue
            short = name.split("(")[0].replace("void ", "").replace("fa::", "")
            out[short] = {"us": round(total / e.count, 2), "launches": e.count}
        return out or None
    except Exception as ex:  # pragma: no cover - depends on the ROCm tracer
        return {"error": f"{type(ex).__name__}: {ex}"[:200]}


def upload(w, torch):
    """Seeded 16-bit inputs of workload w, copied to the GPU before any timing."""
    import numpy as np
    dt = torch.float16 if w.dtype == "f16" else torch.bfloat16
    return tuple(torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to("cuda:0").view(dt)
                 for x in w.inputs())


def device_inputs(w, torch, dev):
    """Seeded N(0,1) inputs of workload w generated on the device (Q and K times the
    workload's multiplier), for throughput runs too large to draw on the host."""
    g = torch.Generator(device=dev)
    g.manual_seed(w.wid)
    dt = torch.float16 if w.dtype == "f16" else torch.bfloat16
    out = []
    for shape, mult in zip(w.shapes(), (w.qk_mult, w.qk_mult, 1.0)):
        x = torch.randn(shape, device=dev, generator=g, dtype=torch.float32)
        out.append((x * mult).to(dt))
        del x
    return out


# ------------------------------------------------------------------ CPU baseline (the oracle)

def _oracle_seconds(w, batches, heads, rows=None):
    """Wall time of the oracle on the given batches and query heads (all key rows; the
    given query rows, or all), and the (batch, head, row) units that covered."""
    import numpy as np
    import oracle
    q, k, v = [oracle.widen(x, w.dtype) for x in w.inputs(batches=batches)]
    group = w.Hq // w.Hkv
    if heads < w.Hq:   # whole KV groups, so the head map stays that of the workload
        ng = max(1, heads // group)
        q = np.ascontiguousarray(q[:, :, :ng * group])
        k = np.ascontiguousarray(k[:, :, :ng])
        v = np.ascontiguousarray(v[:, :, :ng])
        heads = ng * group
    t0 = time.perf_counter()
    oracle.attention(q, k, v, causal=w.causal, scale=w.scale)
    return time.perf_counter() - t0, len(batches) * heads


def cpu_baseline(w, budget_s=12.0):
    """The oracle, as it stands, on the host cores: the first nb batches of the workload
    (all heads, all query rows, all keys), nb grown until a run takes ~budget_s / 3;
    with the whole workload still short of that, whole-workload runs are repeated
    until ~budget_s have passed."""
    import oracle
    oracle.build(force=False)
    threads = oracle.num_threads()
    cache = {}

    def run(nb):
        if nb not in cache:
            cache.clear()
            cache[nb] = [oracle.widen(x, w.dtype) for x in w.inputs(batches=list(range(nb)))]
        q, k, v = cache[nb]
        t0 = time.perf_counter()
        oracle.attention(q, k, v, causal=w.causal, scale=w.scale)
        return time.perf_counter() - t0

    nb = 1
    took = run(nb)
    while took < budget_s / 3 and nb < w.B:
        nb = min(w.B, max(nb * 2, int(nb * budget_s / 3 / max(took, 1e-3))))
        took = run(nb)
    reps = 1
    while nb == w.B and took < budget_s:
        took += run(nb)
        reps += 1
    flops = 4.0 * nb * reps * w.Hq * w.pairs() * w.d
    what = f"batches 0..{nb - 1}" if nb < w.B else f"the whole workload x{reps}"
    return {"value": flops / took / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{w.name}: {what}, all {w.Hq} heads, {w.Nq} query rows x {w.Nk} keys, fp64 "
                      f"({took:.1f} s)", "seconds": took}


def cpu_baseline_sweep(names, budget_per_s=1.5):
    """The oracle on the pages' other workloads: the tiny one whole; the others on
    batch element 0 with as many leading KV groups of query heads as fit about
    budget_per_s, the time scaled linearly to the whole workload (the cost is
    linear in batches and heads) and labelled extrapolated."""
    import oracle
    import synthetic
    oracle.build(force=False)
    rows = []
    for name in names:
        w = synthetic.WORKLOADS[name]
        if w.B * w.Hq * w.pairs() * w.d <= (1 << 29):
            took, reps = 0.0, 0
            while took < 0.2 or reps == 0:
                t, _ = _oracle_seconds(w, list(range(w.B)), w.Hq)
                took += t
                reps += 1
            sec, kind = took / reps, f"whole workload x{reps}"
        else:
            group = w.Hq // w.Hkv
            t1, units = _oracle_seconds(w, [0], group)   # one KV group of batch 0
            heads = min(w.Hq, max(group, int(group * budget_per_s / max(t1, 1e-4)) // group * group))
            if heads > group:
                t1, units = _oracle_seconds(w, [0], heads)
            sec = t1 * (w.B * w.Hq) / units
            kind = f"extrapolated from batch 0, heads 0..{units - 1} ({t1:.2f} s) to {w.B}x{w.Hq}"
        progress(f"oracle {name}: {sec:.3f} s ({kind})")
        if w.decode:
            rows.append({"workload": name, "us_per_step": round(sec * 1e6, 1), "sample": kind})
        else:
            rows.append({"workload": name, "seconds": round(sec, 3),
                         "tflops": round(w.flops() / sec / 1e12, 5), "sample": kind})
    return {"cores": oracle.num_threads(), "kind": "oracle", "rows": rows}


# ------------------------------------------------------------------ GPU legs

# The forward's VALU work per query-key pair (score), as wave64 instructions: one FMA
# (scale and reference max), one exponential, half a conversion to the 16-bit type (two
# per instruction) and half a dot2 (row sum of the rounded probabilities, two per
# instruction); bf16 adds an fp32 add (the unrounded sum for the LSE) and another half
# dot2. Issue cost per wave64 instruction on one SIMD, from a register-only probe on
# MI355X (exponentials and FMA-class instructions share the issue port, their times
# add): 7.1 cycles for v_exp_f32, 2.36 for an FMA-class instruction (3.7 ns and 1.22 ns
# at the 1.93 GHz where a 32x32x16 MFMA took its 32 cycles).
CYC_EXP, CYC_VALU = 7.1, 2.36
SIMDS, CLOCK_GHZ = 1024, 2.4


def valu_bound_tflops(w) -> float:
    """FLOP rate at which the softmax VALU work alone keeps every SIMD's issue port
    busy at the published clock: 4 d FLOP per score, one score per lane."""
    other = 2.0 if w.dtype == "f16" else 3.5
    cycles_per_64_scores = CYC_EXP + other * CYC_VALU
    scores_per_s = SIMDS * CLOCK_GHZ * 1e9 * 64 / cycles_per_64_scores
    return scores_per_s * 4.0 * w.d / 1e12


def fwd_row(name, w, t):
    tf = w.flops() / (t["mean_ms"] * 1e-3) / 1e12
    row = {"workload": name, **stats_fields(t), "tflops": round(tf, 2),
           "tflops_median": round(w.flops() / (t["median_ms"] * 1e-3) / 1e12, 2),
           "tflops_pages_convention": round(tf / 2, 2), "mfma_peak_frac": round(tf / PEAK_MFMA_F16, 4)}
    vb = valu_bound_tflops(w)
    row["valu_bound_tflops"] = round(vb, 1)
    row["bound"] = "valu" if vb < PEAK_MFMA_F16 else "mfma"
    row["bound_frac"] = round(tf / min(vb, PEAK_MFMA_F16), 4)
    if w.causal:   # the same time against the un-halved 4 B H N^2 d count
        row["tflops_unhalved_count"] = round(4.0 * w.B * w.Hq * w.Nq * w.Nk * w.d / (t["mean_ms"] * 1e-3) / 1e12, 2)
    return row


def sweep(args, torch, dev):
    """Forward throughput over the pages' other workloads (long sequences, causal and
    not, the sharpened bf16 repeat, the GQA head-dim sweep) and decode with Nq = 8."""
    import synthetic
    from exact_tiled_attention_21_amd import attention, decode, decode_workspace_bytes
    rows = []
    names = [n for n, w in synthetic.WORKLOADS.items()
             if not w.decode and (n.startswith("long_") or n.startswith("gqa_"))]
    for name in names:
        w = synthetic.WORKLOADS[name]
        q, k, v = device_inputs(w, torch, dev)
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device=dev)
        t = timed_auto(lambda i=0: attention(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse),
                       torch, min(args.prewarm_s, 0.3))
        rows.append(fwd_row(name, w, t))
        progress(f"{name}: {rows[-1]['tflops']} TFLOP/s")
        del q, k, v, o, lse
        torch.cuda.empty_cache()
    wd = synthetic.WORKLOADS["decode_bf16_nq8"]
    sets = [device_inputs(dataclasses.replace(wd, wid=wd.wid + 1000 * r), torch, dev) for r in range(4)]
    ws = torch.empty(decode_workspace_bytes(wd.B, wd.Nq, wd.Hq, wd.d, wd.num_splits), dtype=torch.uint8, device=dev)
    o = torch.empty_like(sets[0][0])

    def dstep(i=0):
        qq, kk, vv = sets[i % len(sets)]
        decode(qq, kk, vv, num_splits=wd.num_splits, scale=wd.scale, workspace=ws, out=o)

    t = timed_auto(dstep, torch, min(args.prewarm_s, 0.3))
    kv_bytes = 2 * wd.B * wd.Nk * wd.Hkv * wd.d * 2
    rows.append({"workload": wd.name, **stats_fields(t, 1e3, "us", 2),
                 "kv_GBps": round(kv_bytes / (t["mean_ms"] * 1e-3) / 1e9, 1), "kv_sets_rotated": len(sets),
                 "kernels_us": kernel_times(dstep, 40, torch)})
    del sets, ws, o
    torch.cuda.empty_cache()
    return rows


def smi_sample():
    """Socket power (W) and the mean graphics clock (MHz) over the XCDs, from one
    `amd-smi metric -p -c` reading; None where the tool is missing or says nothing."""
    import re
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "-p", "-c", "--json"], capture_output=True, text=True,
                           timeout=20)
    except (OSError, subprocess.SubprocessError):
        return None
    p = re.findall(r'"socket_power": \{\s*"value": ([0-9.]+)', r.stdout)
    c = [float(x) for x in re.findall(r'"gfx_[0-7]": \{\s*"clk": \{\s*"value": ([0-9.]+)', r.stdout)]
    if not p or not c:
        return None
    return float(p[0]), sum(c) / len(c)


def power_probe(seconds, torch, attention):
    """The [16,4096,32,128] f16 forward run back to back for `seconds` per input
    set while another thread samples board power and clock: once with Gaussian
    Q (the workload) and once with every Q element 1.0 (same instructions, same
    K and V). The difference shows how far the matrix cores' switching, not the
    instruction stream, sets the clock under the power limit. Then the headline
    workload [16,1024,32,128] with its Gaussian inputs, the same way."""
    import threading
    import synthetic
    w4 = synthetic.WORKLOADS["long_f16_4096_full"]
    wh = synthetic.WORKLOADS["headline_f16_1024"]
    out = {"workload": f"[{w4.B},{w4.Nq},{w4.Hq},{w4.d}] f16, no mask", "seconds": seconds}
    for name, w in (("gaussian_q", w4), ("constant_q", w4), ("headline_gaussian_q", wh)):
        q, k, v = device_inputs(w, torch, torch.device("cuda:0"))
        if name == "constant_q":
            q = torch.ones_like(q)
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device=q.device)
        fn = lambda i=0: attention(q, k, v, causal=False, scale=w.scale, out=o, lse=lse)
        prewarm(fn, 1.0, torch)
        samples, done = [], threading.Event()

        def sampler():
            while not done.is_set():
                x = smi_sample()
                if x is not None:
                    samples.append(x)
                done.wait(0.5)
        th = threading.Thread(target=sampler)
        th.start()
        t = timed_for(fn, seconds, torch)
        done.set()
        th.join()
        row = {"tflops": round(w.flops() / (t * 1e-3) / 1e12, 1)}
        if w is not w4:
            row["workload"] = f"[{w.B},{w.Nq},{w.Hq},{w.d}] f16, no mask"
        if samples:
            row["socket_power_w"] = round(statistics.mean(x[0] for x in samples), 1)
            row["gfx_clock_mhz"] = round(statistics.mean(x[1] for x in samples), 1)
            row["samples"] = len(samples)
        out[name] = row
        del q, k, v, o, lse
        torch.cuda.empty_cache()
    return out


def timed_for(fn, seconds, torch):
    """Mean ms per call of fn over at least `seconds` of back-to-back calls."""
    n, t0 = 0, time.perf_counter()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            fn()
        n += 20
        torch.cuda.synchronize()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--only", choices=["fwd", "headline", "fwd4096", "decode", "bwd", "none", "all"],
                    default="all")
    ap.add_argument("--prewarm-s", type=float, default=1.0,
                    help="seconds of untimed launches per workload before its warmup steps")
    ap.add_argument("--no-sweep", action="store_true", help="skip the sweep over the other workloads")
    ap.add_argument("--no-kernel-trace", action="store_true",
                    help="skip the per-kernel durations (use under an outside profiler)")
    ap.add_argument("--min-seconds", type=float, default=MIN_SECONDS,
                    help="timed seconds per workload besides the headline (at least 50 steps); "
                         "less for profiler runs")
    ap.add_argument("--fwd4096-batch", type=int, default=16, metavar="B",
                    help="batch of the N=4096 forward leg (smaller for counter runs whose totals "
                         "would pass 2^32)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="also run a plain device copy of MIB MiB (calibrates HBM byte counters)")
    ap.add_argument("--power-probe", type=float, default=None, metavar="SECONDS",
                    help="run the N=4096 forward for SECONDS with Gaussian and with constant Q "
                         "while sampling board power and clock (amd-smi); 0 skips it (default: "
                         "3 s in the full run, none with --only)")
    ap.add_argument("--gemm-probe", type=int, default=0, metavar="N",
                    help="also time torch's fp16 N x N x N matmul (the library GEMM: the MFMA rate "
                         "and clock a tuned dense kernel sustains on this GPU)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (the units "
              "(batch, KV head) are independent, so a sharded run is N copies of this one). "
              "Run with --gpus 1.", file=sys.stderr)
        return 2
    if args.no_kernel_trace:
        os.environ["FA_BENCH_NO_KERNEL_TRACE"] = "1"
    TIMING["min_seconds"] = args.min_seconds

    import numpy as np
    import torch
    import synthetic
    from exact_tiled_attention_21_amd import attention, decode, decode_workspace_bytes

    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"
    dev = torch.device("cuda:0")
    result = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
              "higher_is_better": True, "scaling": "weak", "data": "synthetic",
              "prewarm_s": args.prewarm_s}

    # ---- forward, headline workload (the line's value)
    w = synthetic.WORKLOADS["headline_f16_1024"]
    if args.copy_probe:
        src = torch.empty(args.copy_probe << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_probe_bytes"] = 2 * src.numel()   # read + write
        del src, dst
    if args.gemm_probe:
        n = args.gemm_probe
        ga = torch.randn(n, n, device=dev, dtype=torch.float16)
        gb = torch.randn(n, n, device=dev, dtype=torch.float16)
        tg = timed(lambda i=0: ga @ gb, 40, 3, torch, 0.5)
        result["gemm_probe"] = {"n": n, **stats_fields(tg),
                                "tflops": round(2.0 * n ** 3 / (tg["mean_ms"] * 1e-3) / 1e12, 1)}
        del ga, gb
        torch.cuda.empty_cache()
    if args.only in ("fwd", "headline", "all"):
        q, k, v = upload(w, torch)
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device=dev)
        t = timed(lambda i=0: attention(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse),
                  args.steps, args.warmup, torch, args.prewarm_s)
        ms = t["mean_ms"]
        tflops = w.flops() / (ms * 1e-3) / 1e12
        traffic = measured_traffic()
        result.update({
            "value": round(tflops, 2), "unit": "TFLOP/s", "ms_per_step": round(ms, 4),
            "median_ms_per_step": round(t["median_ms"], 4), "min_ms_per_step": round(t["min_ms"], 4),
            "vs_baseline": round(tflops / PAGES_HEADLINE_TFLOPS_4X, 2),
            "vs_baseline_basis": "the pages' official FA2 kernel on an RTX 3080 at this workload "
                                 "(5.32 ms = 51.68 TFLOP/s under 4·B·H·N²·d); context only",
            "dtype": "f16",
            "config": {"workload": w.name, "B": w.B, "Nq": w.Nq, "Nk": w.Nk, "Hq": w.Hq, "Hkv": w.Hkv,
                       "d": w.d, "causal": w.causal},
            "tflops_pages_convention": round(tflops / 2, 2),
            "mfma_peak_frac": round(tflops / PEAK_MFMA_F16, 4),
            # one library call is one launch of the forward kernel: the per-step time
            # between events on the launch stream is that kernel's duration
            "roofline": {"bound": "mfma", "kernel": "fa_fwd_kernel<128,f16,noncausal>",
                         "achieved": round(tflops, 2), "peak": PEAK_MFMA_F16, "unit": "TFLOP/s",
                         "frac": round(tflops / PEAK_MFMA_F16, 4), "traffic": traffic,
                         "flop_per_launch": w.flops()},
        })
        progress(f"headline: {result['value']} TFLOP/s")
        del q, k, v, o, lse
        torch.cuda.empty_cache()

    if args.only in ("fwd", "fwd4096", "all"):
        # forward at N = 4096 (the 50%-of-peak target shape)
        w4 = synthetic.WORKLOADS["long_f16_4096_full"]
        if args.fwd4096_batch != w4.B:
            w4 = dataclasses.replace(w4, B=args.fwd4096_batch)
        q, k, v = upload(w4, torch)
        o = torch.empty_like(q)
        t4 = timed_auto(lambda i=0: attention(q, k, v, scale=w4.scale, out=o), torch, args.prewarm_s)
        result["fwd_4096"] = fwd_row(w4.name, w4, t4)
        progress(f"fwd_4096: {result['fwd_4096']['tflops']} TFLOP/s")
        del q, k, v, o
        torch.cuda.empty_cache()

    if args.only in ("fwd", "all"):
        # packed variable-length batch: 16 sequences of seeded lengths in [256, 2048],
        # headline heads and head dim (FLOPs counted per sequence)
        from exact_tiled_attention_21_amd import attention_varlen
        rng = np.random.default_rng([w.wid, 99])
        lens = rng.integers(256, 2049, size=16)
        tot = int(lens.sum())
        qv, kv_, vv_ = upload(dataclasses.replace(w, B=1, Nq=tot, Nk=tot), torch)
        qv, kv_, vv_ = qv[0], kv_[0], vv_[0]
        cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).to(dev)
        ov = torch.empty_like(qv)
        tv = timed_auto(lambda i=0: attention_varlen(qv, kv_, vv_, cu, cu, int(lens.max()), scale=w.scale, out=ov,
                                                         validate=False),
                        torch, args.prewarm_s)
        fl = float(sum(4.0 * w.Hq * int(n) * int(n) * w.d for n in lens))
        result["fwd_varlen"] = {"workload": "16 packed sequences, lengths 256..2048 (seeded), Hq=Hkv=32, d=128, f16",
                                "tokens": tot, **stats_fields(tv),
                                "tflops": round(fl / (tv["mean_ms"] * 1e-3) / 1e12, 2)}
        progress(f"fwd_varlen: {result['fwd_varlen']['tflops']} TFLOP/s")
        del qv, kv_, vv_, ov
        torch.cuda.empty_cache()

    if args.only in ("fwd", "all") and not args.no_sweep:
        result["sweep"] = sweep(args, torch, dev)

    # ---- split-KV decode, rotating over KV sets larger than the 256 MB infinity cache
    if args.only in ("decode", "all"):
        wd = synthetic.WORKLOADS["decode_bf16_nq1"]
        sets = [upload(dataclasses.replace(wd, wid=wd.wid + 1000 * r), torch) for r in range(4)]
        ws = torch.empty(decode_workspace_bytes(wd.B, wd.Nq, wd.Hq, wd.d, wd.num_splits), dtype=torch.uint8,
                         device=dev)
        o = torch.empty_like(sets[0][0])
        lse = torch.empty((wd.B, wd.Hq, wd.Nq), dtype=torch.float32, device=dev)

        def dstep(i=0):
            qq, kk, vv = sets[i % len(sets)]
            decode(qq, kk, vv, num_splits=wd.num_splits, scale=wd.scale, workspace=ws, out=o, lse=lse)

        td = timed(dstep, max(args.steps, 200), args.warmup, torch, args.prewarm_s)
        msd = td["mean_ms"]
        kv_bytes = 2 * wd.B * wd.Nk * wd.Hkv * wd.d * 2
        # a plain device-to-device copy of 1 GiB in the same run: the attainable HBM rate
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        tc = timed(lambda i=0: dst.copy_(src), 20, 2, torch, 0.2)
        copy_gbps = 2 * src.numel() / (tc["median_ms"] * 1e-3) / 1e9   # read + write
        del src, dst
        result["decode"] = {"workload": wd.name, **stats_fields(td, 1e3, "us", 2),
                            "us_per_step": round(msd * 1e3, 2),
                            "kv_GBps": round(kv_bytes / (msd * 1e-3) / 1e9, 1),
                            "hbm_peak_frac": round(kv_bytes / (msd * 1e-3) / 1e9 / PEAK_HBM, 4),
                            "roofline_us": round(kv_bytes / (PEAK_HBM * 1e9) * 1e6, 2),
                            "copy_GBps": round(copy_gbps, 1),
                            "copy_frac": round(kv_bytes / (msd * 1e-3) / 1e9 / copy_gbps, 4),
                            "kv_sets_rotated": len(sets),
                            "kernels_us": kernel_times(dstep, 40, torch)}
        progress(f"decode: {result['decode']['us_per_step']} us/step")
        # the same step over a paged cache: 256-key pages in a scrambled block table
        from exact_tiled_attention_21_amd import decode_paged
        ps, mp = 256, wd.Nk // 256
        bt = torch.from_numpy(synthetic.block_table(wd.wid, wd.B, mp, wd.B * mp)).to(dev)
        lens = torch.full((wd.B,), wd.Nk, dtype=torch.int32, device=dev)
        # each KV set seen as a pool of B * Nk / 256 pages; the scrambled table makes every
        # sequence read pages scattered over the pool
        pools = [(qq, kk.view(wd.B * mp, ps, wd.Hkv, wd.d), vv.view(wd.B * mp, ps, wd.Hkv, wd.d))
                 for qq, kk, vv in sets]

        def pstep(i=0):
            qq, kk, vv = pools[i % len(pools)]
            decode_paged(qq, kk, vv, bt, lens, num_splits=wd.num_splits, scale=wd.scale, workspace=ws,
                         out=o, lse=lse)

        tp = timed(pstep, max(args.steps, 200), args.warmup, torch, args.prewarm_s)
        msp = tp["mean_ms"]
        result["decode_paged"] = {"workload": wd.name, "page_size": ps, **stats_fields(tp, 1e3, "us", 2),
                                  "us_per_step": round(msp * 1e3, 2),
                                  "kv_GBps": round(kv_bytes / (msp * 1e-3) / 1e9, 1),
                                  "hbm_peak_frac": round(kv_bytes / (msp * 1e-3) / 1e9 / PEAK_HBM, 4),
                                  "kernels_us": kernel_times(pstep, 40, torch)}
        del pools
        if "value" not in result:
            result.update({"value": round(msd * 1e3, 2), "unit": "us/step", "higher_is_better": False,
                           "ms_per_step": round(msd, 5), "vs_baseline": None, "dtype": "bf16",
                           "config": {"workload": wd.name}})
        del sets, ws, o, lse
        torch.cuda.empty_cache()

    # ---- backward at the pages' fwd+bwd benchmark setting (N 4096, 16 heads of 128, B 4)
    if args.only in ("bwd", "all"):
        from exact_tiled_attention_21_amd import attention_backward, bwd_workspace_bytes
        for name in ("bwd_bf16_4096_full", "bwd_bf16_4096_causal"):
            wb = synthetic.WORKLOADS[name]
            q, k, v = upload(wb, torch)
            dt = q.dtype
            do = torch.from_numpy(np.ascontiguousarray(wb.grad_out()).view(np.int16)).to(dev).view(dt)
            o, lse = attention(q, k, v, causal=wb.causal, scale=wb.scale)
            ws = torch.empty(bwd_workspace_bytes(wb.B, wb.Nq, wb.Hq), dtype=torch.uint8, device=dev)
            dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

            def bstep(i=0):
                attention_backward(q, k, v, o, lse, do, causal=wb.causal, scale=wb.scale, workspace=ws,
                                   dq=dq, dk=dk, dv=dv)

            tb_ = timed_auto(bstep, torch, args.prewarm_s)
            # the pages' convention: the backward does 2.5x the forward's matrix FLOPs
            # (five products of 2 N^2 d against two); these kernels execute seven
            fl = 2.5 * wb.flops()
            tb = fl / (tb_["mean_ms"] * 1e-3) / 1e12
            result["bwd_4096_" + ("causal" if wb.causal else "full")] = {
                "workload": wb.name, **stats_fields(tb_), "tflops": round(tb, 2),
                "tflops_executed": round(tb * 3.5 / 2.5, 2),
                "mfma_peak_frac": round(tb / PEAK_MFMA_F16, 4),
                "kernels_us": kernel_times(bstep, 10, torch)}
            progress(f"{wb.name}: {tb:.1f} TFLOP/s (pages' convention)")
            del q, k, v, do, o, lse, ws, dq, dk, dv
            torch.cuda.empty_cache()

    probe_s = args.power_probe if args.power_probe is not None else (3.0 if args.only == "all" else 0.0)
    if probe_s > 0:
        result["power_probe"] = power_probe(probe_s, torch, attention)
        progress(f"power probe: {result['power_probe']}")

    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(w)
        progress("cpu baseline (headline) done")
        if args.only == "all":
            names = (["tiny_f16_128"] + [n for n in synthetic.WORKLOADS if n.startswith("long_")]
                     + [n for n in synthetic.WORKLOADS if n.startswith("gqa_")] + ["decode_bf16_nq1"])
            result["cpu_baseline_sweep"] = cpu_baseline_sweep(names)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
