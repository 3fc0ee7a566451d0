#!/usr/bin/env python3
"""Benchmark of the exact-attention hot path on one MI355X.

One step = one forward pass over the pages' headline workload
[B=16, N=1024, H=32, d=128] fp16, non-causal (inputs resident in HBM). The line
also carries the split-KV decode step (split + combine kernels) at
B=8, Nq=1, Nk=8192, Hq=32, Hkv=8, d=128 bf16 with 16 splits, the forward at
N=4096, a packed variable-length batch, the backward pass, and a sweep over the
pages' other workloads (long sequences causal and not, the sharpened bf16 repeat,
the GQA head-dim sweep, decode with Nq=8; inputs drawn on the device), each timed
the same way. Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_F16 = 2500.0     # TFLOP/s, MI355X dense fp16/bf16 (published)
PEAK_HBM = 8000.0          # GB/s, MI355X HBM3E (published)
METRIC = "attention fwd TFLOP/s (4·B·H·N²·d) & % MFMA peak; split-KV decode µs/step"
PAGES_HEADLINE_TFLOPS_4X = 51.68   # RTX 3080 official FA2 at [16,1024,32,128], 5.32 ms (pages' table, x2)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fa_fwd_headline_traffic.json")
KERNEL_SOURCES = ("fa_fwd_kernel.h", "fa_device.h", "fa_launch.h")


def code_only(text: str) -> str:
    """C++ source with comments removed and whitespace collapsed: a comment edit
    leaves the kernel, and so its hash, unchanged."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


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


def time_steps(fn, steps, warmup, torch, warm_s=0.0):
    prewarm(fn, warm_s, torch)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        fn(i)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps   # ms per step


def upload(w, torch):
    """Seeded 16-bit inputs of workload w, copied to the GPU before any timing."""
    import numpy as np
    dt = torch.float16 if w.dtype == "f16" else torch.bfloat16
    return tuple(torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to("cuda:0").view(dt)
                 for x in w.inputs())


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


def cpu_baseline_decode(w, reps_budget_s=3.0):
    """The oracle on the whole decode workload (all batches, heads and keys), repeated
    for about reps_budget_s; reported as microseconds per decode step."""
    import oracle
    oracle.build(force=False)
    q, k, v = [oracle.widen(x, w.dtype) for x in w.inputs()]
    took, reps = 0.0, 0
    while took < reps_budget_s or reps == 0:
        t0 = time.perf_counter()
        oracle.attention(q, k, v, causal=w.causal, scale=w.scale)
        took += time.perf_counter() - t0
        reps += 1
    return {"value": round(took / reps * 1e6, 1), "unit": "us/step", "cores": oracle.num_threads(),
            "kind": "oracle", "sample": f"{w.name}: the whole step x{reps}, fp64 ({took:.1f} s)"}


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
        ms = time_steps(lambda i=0: attention(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse),
                        max(3, args.steps // 10), 2, torch, min(args.prewarm_s, 0.3))
        t = w.flops() / (ms * 1e-3) / 1e12
        row = {"workload": name, "ms": round(ms, 4), "tflops": round(t, 2),
               "tflops_pages_convention": round(t / 2, 2), "mfma_peak_frac": round(t / PEAK_MFMA_F16, 4)}
        if w.causal:   # the same time against the un-halved 4 B H N^2 d count
            row["tflops_unhalved_count"] = round(4.0 * w.B * w.Hq * w.Nq * w.Nk * w.d / (ms * 1e-3) / 1e12, 2)
        rows.append(row)
        del q, k, v, o, lse
        torch.cuda.empty_cache()
    wd = synthetic.WORKLOADS["decode_bf16_nq8"]
    sets = []
    for r in range(4):
        sets.append(device_inputs(dataclasses.replace(wd, wid=wd.wid + 1000 * r), torch, dev))
    ws = torch.empty(decode_workspace_bytes(wd.B, wd.Nq, wd.Hq, wd.d, wd.num_splits), dtype=torch.uint8, device=dev)
    o = torch.empty_like(sets[0][0])

    def dstep(i=0):
        qq, kk, vv = sets[i % len(sets)]
        decode(qq, kk, vv, num_splits=wd.num_splits, scale=wd.scale, workspace=ws, out=o)

    msd = time_steps(dstep, max(args.steps, 100), args.warmup, torch, min(args.prewarm_s, 0.3))
    kv_bytes = 2 * wd.B * wd.Nk * wd.Hkv * wd.d * 2
    rows.append({"workload": wd.name, "us_per_step": round(msd * 1e3, 2),
                 "kv_GBps": round(kv_bytes / (msd * 1e-3) / 1e9, 1), "kv_sets_rotated": len(sets)})
    del sets, ws, o
    torch.cuda.empty_cache()
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--only", choices=["fwd", "headline", "decode", "bwd", "all"], default="all")
    ap.add_argument("--prewarm-s", type=float, default=1.0,
                    help="seconds of untimed launches per workload before its warmup steps")
    ap.add_argument("--no-sweep", action="store_true", help="skip the sweep over the other workloads")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="also run a plain device copy of MIB MiB (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (the units "
              "(batch, KV head) are independent, so a sharded run is N copies of this one). "
              "Run with --gpus 1.", file=sys.stderr)
        return 2

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
    if args.only in ("fwd", "headline", "all"):
        q, k, v = upload(w, torch)
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device=dev)
        ms = time_steps(lambda i=0: attention(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse),
                        args.steps, args.warmup, torch, args.prewarm_s)
        tflops = w.flops() / (ms * 1e-3) / 1e12
        traffic = measured_traffic()
        result.update({
            "value": round(tflops, 2), "unit": "TFLOP/s", "ms_per_step": round(ms, 4),
            "vs_baseline": round(tflops / PAGES_HEADLINE_TFLOPS_4X, 2), "dtype": "f16",
            "config": {"workload": w.name, "B": w.B, "Nq": w.Nq, "Nk": w.Nk, "Hq": w.Hq, "Hkv": w.Hkv,
                       "d": w.d, "causal": w.causal},
            "tflops_pages_convention": round(tflops / 2, 2),
            "mfma_peak_frac": round(tflops / PEAK_MFMA_F16, 4),
            "roofline": {"bound": "mfma", "kernel": "fa_fwd_kernel<128,f16,noncausal>",
                         "achieved": round(tflops, 2), "peak": PEAK_MFMA_F16, "unit": "TFLOP/s",
                         "frac": round(tflops / PEAK_MFMA_F16, 4),
                         "traffic": traffic},
        })
        del q, k, v, o, lse
        torch.cuda.empty_cache()

    if args.only in ("fwd", "all"):
        # forward at N = 4096 (the 50%-of-peak target shape)
        w4 = synthetic.WORKLOADS["long_f16_4096_full"]
        q, k, v = upload(w4, torch)
        o = torch.empty_like(q)
        ms4 = time_steps(lambda i=0: attention(q, k, v, scale=w4.scale, out=o), max(5, args.steps // 5),
                         max(2, args.warmup // 5), torch, args.prewarm_s)
        t4 = w4.flops() / (ms4 * 1e-3) / 1e12
        result["fwd_4096"] = {"workload": w4.name, "ms": round(ms4, 4), "tflops": round(t4, 2),
                              "tflops_pages_convention": round(t4 / 2, 2),
                              "mfma_peak_frac": round(t4 / PEAK_MFMA_F16, 4)}
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
        msv = time_steps(lambda i=0: attention_varlen(qv, kv_, vv_, cu, cu, int(lens.max()), scale=w.scale,
                                                      out=ov), args.steps, args.warmup, torch, args.prewarm_s)
        fl = float(sum(4.0 * w.Hq * int(n) * int(n) * w.d for n in lens))
        result["fwd_varlen"] = {"workload": "16 packed sequences, lengths 256..2048 (seeded), Hq=Hkv=32, d=128, f16",
                                "tokens": tot, "ms": round(msv, 4), "tflops": round(fl / (msv * 1e-3) / 1e12, 2)}
        del qv, kv_, vv_, ov
        torch.cuda.empty_cache()

    if args.only in ("fwd", "all") and not args.no_sweep:
        result["sweep"] = sweep(args, torch, dev)

    # ---- split-KV decode, rotating over KV sets larger than the 256 MB infinity cache
    if args.only in ("decode", "all"):
        wd = synthetic.WORKLOADS["decode_bf16_nq1"]
        sets = []
        for r in range(4):
            wr = dataclasses.replace(wd, wid=wd.wid + 1000 * r)
            sets.append(upload(wr, torch))
        ws = torch.empty(decode_workspace_bytes(wd.B, wd.Nq, wd.Hq, wd.d, wd.num_splits), dtype=torch.uint8,
                         device=dev)
        o = torch.empty_like(sets[0][0])
        lse = torch.empty((wd.B, wd.Hq, wd.Nq), dtype=torch.float32, device=dev)

        def dstep(i=0):
            qq, kk, vv = sets[i % len(sets)]
            decode(qq, kk, vv, num_splits=wd.num_splits, scale=wd.scale, workspace=ws, out=o, lse=lse)

        msd = time_steps(dstep, max(args.steps, 100), args.warmup, torch, args.prewarm_s)
        kv_bytes = 2 * wd.B * wd.Nk * wd.Hkv * wd.d * 2
        # a plain device-to-device copy of 1 GiB in the same run: the attainable HBM rate
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        msc = time_steps(lambda i=0: dst.copy_(src), 10, 2, torch, 0.2)
        copy_gbps = 2 * src.numel() / (msc * 1e-3) / 1e9   # read + write
        del src, dst
        result["decode"] = {"workload": wd.name, "us_per_step": round(msd * 1e3, 2),
                            "kv_GBps": round(kv_bytes / (msd * 1e-3) / 1e9, 1),
                            "hbm_peak_frac": round(kv_bytes / (msd * 1e-3) / 1e9 / PEAK_HBM, 4),
                            "roofline_us": round(kv_bytes / (PEAK_HBM * 1e9) * 1e6, 2),
                            "copy_GBps": round(copy_gbps, 1),
                            "copy_frac": round(kv_bytes / (msd * 1e-3) / 1e9 / copy_gbps, 4),
                            "kv_sets_rotated": len(sets)}
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

        msp = time_steps(pstep, max(args.steps, 100), args.warmup, torch, args.prewarm_s)
        result["decode_paged"] = {"workload": wd.name, "page_size": ps, "us_per_step": round(msp * 1e3, 2),
                                  "kv_GBps": round(kv_bytes / (msp * 1e-3) / 1e9, 1),
                                  "hbm_peak_frac": round(kv_bytes / (msp * 1e-3) / 1e9 / PEAK_HBM, 4)}
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
            msb = time_steps(lambda i=0: attention_backward(q, k, v, o, lse, do, causal=wb.causal, scale=wb.scale,
                                                            workspace=ws, dq=dq, dk=dk, dv=dv),
                             max(5, args.steps // 5), max(2, args.warmup // 5), torch, args.prewarm_s)
            # the pages' convention: the backward does 2.5x the forward's matrix FLOPs
            # (five products of 2 N^2 d against two); these kernels execute seven
            fl = 2.5 * wb.flops()
            tb = fl / (msb * 1e-3) / 1e12
            result["bwd_4096_" + ("causal" if wb.causal else "full")] = {
                "workload": wb.name, "ms": round(msb, 4), "tflops": round(tb, 2),
                "tflops_executed": round(tb * 3.5 / 2.5, 2),
                "mfma_peak_frac": round(tb / PEAK_MFMA_F16, 4)}
            del q, k, v, do, o, lse, ws, dq, dk, dv
            torch.cuda.empty_cache()

    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(w)
        if args.only in ("decode", "all"):
            result["cpu_baseline_decode"] = cpu_baseline_decode(synthetic.WORKLOADS["decode_bf16_nq1"])
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
