#!/usr/bin/env python3
"""Benchmark of LongNet dilated attention on one MI355X (prints ONE JSON line).

A step is one pass of the whole operator path over one batch already
resident in HBM: dla_forward (attention over all patterns + merge) then
dla_backward (preprocess, attention backward over all patterns, sum of
the patterns' partial gradients), the operator's share of
a training step.  Default workload: bf16, B=2, N=32768, H=12, D=64, causal,
patterns w = 2048*2^i, r = 2^i for i = 0..4 (the 768-dim, 12-head model
settings of the gptget.net LongNet summary, section 实验设计, at 32K tokens).

Also reported, as extra fields of the same line:
  * forward-only throughput of every forward workload: fp32 N=2048 (B=1,
    non-causal, on the fp32 matrix cores, also against the fp32 peak), bf16
    N=8192 (B=4), N=32768 (B=1) and N=1,048,576 (B=1);
  * `shard_forward`: one device's share when the 1M-token sequence is split
    over 8 devices (the last shard, whose segments of the three coarsest
    patterns span 2, 4 and 8 devices): its exchange parts and its forward,
    and (`fwd_bwd`) forward plus backward, the collectives excluded;
  * in `forward_only`, also the N=32768 forward with FP8 E4M3 keys and values;
  * `layer`: the attention layer around the operator (hipBLASLt projections,
    768 dimensions, 12 heads, random weights) at 16 x 2K and 1 x 32K tokens,
    forward and forward plus backward;
  * `cold_cache` (the step, and each forward line): kernel time per step when
    512 MB are written between steps, so no input stays in the 256 MB
    last-level cache (`value` is the warm, back-to-back step);
  * `roofline` of the kernel family that takes most of the step, timed live
    with HIP events around its launches on the launch stream, in a second
    timed pass of the same steps (`ms_per_step_events` is that pass's wall
    time; `ms_per_step` and `value` come from the first pass, which records
    no events);
  * `cpu_baseline`: the CPU oracle (float32, thread pool) on a bounded
    sample of the same workload, scaled to the full workload.

The extra lines time their steps in three passes and keep the median pass;
the headline step is timed once, exactly `--steps` steps.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "tokens/s and % of bf16 MFMA peak, dilated attn fwd(+bwd), N=32K & 1M, 1 GPU"
BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3      # MI355X fp32 vector (the fp32 forward runs on the VALU)
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
FAMILIES = ("attn_fwd", "attn_fwd_f32", "attn_fwd_fp8", "combine", "bwd_prep", "attn_bwd",
            "bwd_finalize", "shard_gather", "shard_finish", "quantize_fp8")
KERNEL_SOURCES = {
    "attn_fwd": ["attn_fwd_bf16.hip", "dla_device.h"],
    "attn_bwd": ["attn_bwd_bf16.hip", "dla_device.h"],
    "combine": ["combine.hip", "dla_device.h"],
    "bwd_prep": ["bwd_misc.hip", "dla_device.h"],
    "bwd_finalize": ["bwd_misc.hip", "dla_device.h"],
}


def kernel_source_sha(family: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[family]:
        with open(os.path.join(ROOT, "sparse_long_sequence_dilated_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def gpu_inputs(wl, count, seed):
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    return [torch.randn((wl.B, wl.N, wl.H, wl.D), device="cuda", generator=g).to(dt)
            for _ in range(count)]


def family_work(family, wl, pairs):
    """Algorithmic work of one step of a kernel family: (amount, unit, bound)."""
    D = wl.D
    if family == "attn_bwd":
        return 10 * D * pairs, "flop", "mfma"
    if family in ("attn_fwd", "attn_fwd_f32"):
        return 4 * D * pairs, "flop", "mfma"
    rows = wl.B * wl.N * wl.H
    if family == "bwd_prep":
        # read O, dO (bf16) and LSE, write the (-LSE log2 e, -D) pair
        return rows * (2 * D * 2 + 4 + 8), "byte", "hbm"
    if family == "bwd_finalize":
        # rows kept by k >= 2 patterns: read k fp32 partial rows of dQ, dK, dV,
        # write the three bf16 gradient rows
        period = math.lcm(*[r for _, r in wl.patterns])
        total = 0
        for h in range(wl.H):
            for n_mod in range(period):
                kept = sum(1 for w, r in wl.patterns if n_mod % r == h % r)
                if kept >= 2:
                    total += 3 * (kept * D * 4 + D * 2) * (wl.N // period)
        return total * wl.B, "byte", "hbm"
    if family == "combine":
        # rows kept by the primary pattern and >= 1 other: read O, LSE and each
        # other pattern's partial (O_p bf16, LSE_p fp32); write O, LSE
        period = math.lcm(*[r for _, r in wl.patterns])
        total = 0
        for h in range(wl.H):
            for n_mod in range(period):
                kept = [p for p, (w, r) in enumerate(wl.patterns) if n_mod % r == h % r]
                if len(kept) < 2:
                    continue
                per = (2 * D * 2 + 8) + (len(kept) - 1) * (D * 2 + 4)
                total += per * (wl.N // period)
        return total * wl.B, "byte", "hbm"
    raise KeyError(family)


def traffic_for(family, launches_per_step):
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(family)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != kernel_source_sha(family):
        return None
    return rec["bytes_per_step"] / max(1, launches_per_step) if rec.get("per") == "step" else rec.get("bytes_per_launch")


def time_steps(step, steps, warmup, reps=1):
    """Time `steps` steps after `warmup` untimed ones, twice: first with the
    library's launch timing off (the wall time per step that is reported),
    then again with each library launch bracketed by HIP events on its own
    stream (per-family kernel times).  With reps > 1 (the extra lines, not
    the headline step) the first pass is repeated and its median kept, so
    that one host stall does not stand for the whole line.  Returns
    (ms per step, {family: (launches, total ms)}, ms per step with events)."""
    import torch
    from sparse_long_sequence_dilated_amd import dla
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    passes = []
    for _ in range(reps):
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        passes.append((time.perf_counter() - t0) * 1e3 / steps)
    ms = sorted(passes)[len(passes) // 2]
    # fill the library's event pool so the timed steps create no events
    dla.timing_enable(True)
    step()
    torch.cuda.synchronize()
    dla.timing_enable(False)
    for fam in FAMILIES:
        dla.timing_collect(fam)
    torch.cuda.synchronize()
    dla.timing_enable(True)
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    dla.timing_enable(False)
    fams = {}
    for fam in FAMILIES:
        n, fms = dla.timing_collect(fam)
        if n:
            fams[fam] = (n, fms)
    return ms, fams, (t1 - t0) * 1e3 / steps


def cold_kernel_ms(step, steps, flush_bytes=512 << 20):
    """Kernel time per step (the library's HIP-event-timed launches) when a
    write of `flush_bytes` between steps evicts the 256 MB last-level cache,
    so that every step starts with its inputs in HBM only."""
    import torch
    from sparse_long_sequence_dilated_amd import dla
    buf = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda")
    step()
    torch.cuda.synchronize()
    total = 0.0
    for i in range(steps):
        buf.fill_(i & 0xFF)
        torch.cuda.synchronize()
        dla.timing_enable(True)
        step()
        torch.cuda.synchronize()
        dla.timing_enable(False)
        for fam in FAMILIES:
            total += dla.timing_collect(fam)[1]
    del buf
    return total / steps


def forward_only(name, steps, warmup):
    import torch
    from sparse_long_sequence_dilated_amd import dla, inputs
    wl = inputs.WORKLOADS[name]
    q, k, v = gpu_inputs(wl, 3, 1000 + wl.seed)
    dt = dla.DLA_F32 if wl.dtype == "f32" else dla.DLA_BF16
    ws_f, _ = dla.plan_check(wl.patterns, wl.causal, wl.scale, wl.B, wl.N, wl.H, dtype=dt)
    ws = torch.empty(max(ws_f, 1), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((wl.B, wl.H, wl.N), dtype=torch.float32, device="cuda")

    def step():
        dla.forward(q, k, v, wl.patterns, wl.causal, wl.scale, out=o, lse=lse, workspace=ws)

    ms, fams, _ = time_steps(step, steps, warmup, reps=3)
    pairs = dla.pair_count(wl.patterns, wl.causal, wl.B, wl.N, wl.H)
    tflops = 4 * wl.D * pairs / (ms * 1e-3) / 1e12
    out = {"workload": wl.describe(), "tokens_per_s": wl.B * wl.N / (ms * 1e-3), "ms": ms,
           "useful_tflops": tflops, "pct_bf16_peak": 100.0 * tflops / BF16_PEAK_TFLOPS}
    if wl.dtype == "f32":
        # fp32 runs on the fp32 matrix cores: their peak is the one that bounds it
        out["pct_fp32_peak"] = 100.0 * tflops / FP32_PEAK_TFLOPS
    for fam, (n, fms) in fams.items():
        out[f"{fam}_us_per_launch"] = 1e3 * fms / n
        if fam in ("attn_fwd", "attn_fwd_f32"):
            kt = 4 * wl.D * pairs / (fms * 1e-3 / n) / 1e12
            out[f"{fam}_tflops"] = kt
            out[f"{fam}_frac_of_peak"] = kt / (FP32_PEAK_TFLOPS if fam == "attn_fwd_f32" else BF16_PEAK_TFLOPS)
    cold = cold_kernel_ms(step, min(steps, 10))
    out["cold_cache"] = {"kernel_ms": cold, "tokens_per_s": wl.B * wl.N / (cold * 1e-3),
                         "pct_bf16_peak": 100.0 * 4 * wl.D * pairs / (cold * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}
    del q, k, v, o, lse, ws
    torch.cuda.empty_cache()
    return out


def fp8_forward(name, steps, warmup):
    """Forward with FP8 E4M3 keys and values (quantized once, outside the
    timed step, as a cache of keys and values would hold them)."""
    import torch
    from sparse_long_sequence_dilated_amd import dla, inputs
    wl = inputs.WORKLOADS[name]
    q, k, v = gpu_inputs(wl, 3, 1000 + wl.seed)
    k8, ks = dla.quantize_fp8(k)
    v8, vs = dla.quantize_fp8(v)
    ws_f, _ = dla.plan_check(wl.patterns, wl.causal, wl.scale, wl.B, wl.N, wl.H)
    ws = torch.empty(max(ws_f, 1), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((wl.B, wl.H, wl.N), dtype=torch.float32, device="cuda")

    def step():
        dla.forward_fp8kv(q, k8, v8, ks, vs, wl.patterns, wl.causal, wl.scale, out=o, lse=lse,
                          workspace=ws)

    ms, fams, _ = time_steps(step, steps, warmup, reps=3)
    qms, _, _ = time_steps(lambda: dla.quantize_fp8(k), steps, warmup, reps=3)
    pairs = dla.pair_count(wl.patterns, wl.causal, wl.B, wl.N, wl.H)
    tflops = 4 * wl.D * pairs / (ms * 1e-3) / 1e12
    out = {"workload": wl.describe() + ", keys and values FP8 E4M3 with per-head scales",
           "tokens_per_s": wl.B * wl.N / (ms * 1e-3), "ms": ms, "useful_tflops": tflops,
           "pct_bf16_peak": 100.0 * tflops / BF16_PEAK_TFLOPS, "quantize_one_tensor_ms": qms}
    for fam, (n, fms) in fams.items():
        out[f"{fam}_us_per_launch"] = 1e3 * fms / n
    del q, k, v, k8, v8, ks, vs, o, lse, ws
    torch.cuda.empty_cache()
    return out


def shard_forward(name, devices, shard, steps, warmup):
    """One device's share of the sequence-split scheme: workload `name` cut into
    `devices` shards, the work of shard `shard` (its parts of the key/value
    exchange, then the shard's forward against the gathered segments).  The
    collective between the two is not part of a one-GPU step."""
    import torch
    from sparse_long_sequence_dilated_amd import dla, inputs
    wl = inputs.WORKLOADS[name]
    N = wl.N // devices
    start = shard * N
    g = torch.Generator(device="cuda")
    g.manual_seed(2000 + wl.seed)
    q, k, v = (torch.randn((wl.B, N, wl.H, wl.D), device="cuda", generator=g).bfloat16() for _ in range(3))
    span = [i for i, (w, r) in enumerate(wl.patterns) if w > N]
    ext_k = {i: torch.randn((wl.patterns[i][0] // N, wl.B, wl.H, N // wl.patterns[i][1], wl.D),
                            device="cuda", generator=g).bfloat16() for i in span}
    ext_v = {i: torch.randn_like(ext_k[i]) for i in span}
    part_k = {i: torch.empty((wl.B, wl.H, N // wl.patterns[i][1], wl.D), dtype=torch.bfloat16,
                             device="cuda") for i in span}
    part_v = {i: torch.empty_like(part_k[i]) for i in span}
    ws_f, _ = dla.plan_check_shard(wl.patterns, wl.causal, wl.scale, wl.B, N, wl.H, wl.N, start)
    ws = torch.empty(max(ws_f, 1), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((wl.B, wl.H, N), dtype=torch.float32, device="cuda")

    def step():
        for i in span:
            dla.shard_gather(k, wl.patterns, i, wl.N, start, wl.causal, out=part_k[i])
            dla.shard_gather(v, wl.patterns, i, wl.N, start, wl.causal, out=part_v[i])
        dla.forward_shard(q, k, v, wl.patterns, wl.N, start, ext_k, ext_v, wl.causal, wl.scale,
                          out=o, lse=lse, workspace=ws)

    ms, fams, _ = time_steps(step, steps, warmup, reps=3)
    pairs = dla.pair_count_shard(wl.patterns, wl.causal, wl.B, N, wl.H, wl.N, start)
    tflops = 4 * wl.D * pairs / (ms * 1e-3) / 1e12
    out = {"workload": f"{wl.describe()}, split over {devices} devices, shard {shard} "
                       f"(rows {start}..{start + N - 1}; {len(span)} patterns span devices)",
           "tokens_per_s": wl.B * N / (ms * 1e-3), "ms": ms, "useful_tflops": tflops,
           "pct_bf16_peak": 100.0 * tflops / BF16_PEAK_TFLOPS}
    for fam, (n, fms) in fams.items():
        out[f"{fam}_us_per_launch"] = 1e3 * fms / n

    # The backward of the same shard: its first half, then (after the
    # exchange, not part of a one-GPU step) the finish pass.
    dout = torch.randn_like(q)
    red_k = {i: torch.randn((wl.B, wl.H, N // wl.patterns[i][1], wl.D), device="cuda", generator=g)
             for i in span}
    red_v = {i: torch.randn_like(red_k[i]) for i in span}
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    _, ws_b = dla.plan_check_shard(wl.patterns, wl.causal, wl.scale, wl.B, N, wl.H, wl.N, start)
    wsb = torch.empty(max(ws_b, 1), dtype=torch.uint8, device="cuda")

    def bstep():
        step()
        dla.backward_shard(q, k, v, o, lse, dout, wl.patterns, wl.N, start, ext_k, ext_v, wl.causal,
                           wl.scale, dq=dq, dk=dk, dv=dv, workspace=wsb)
        dla.finish_shard(dk, dv, wl.patterns, wl.N, start, red_k, red_v, wsb, wl.causal, wl.scale)

    bms, bfams, _ = time_steps(bstep, steps, warmup, reps=3)
    btf = 14 * wl.D * pairs / (bms * 1e-3) / 1e12
    out["fwd_bwd"] = {"tokens_per_s": wl.B * N / (bms * 1e-3), "ms": bms, "useful_tflops": btf,
                      "pct_bf16_peak": 100.0 * btf / BF16_PEAK_TFLOPS}
    for fam, (n, fms) in bfams.items():
        out["fwd_bwd"][f"{fam}_us_per_step"] = 1e3 * fms / steps
    del q, k, v, o, lse, ws, ext_k, ext_v, part_k, part_v, dout, red_k, red_v, dq, dk, dv, wsb
    torch.cuda.empty_cache()
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, min_seconds=10.0, max_passes=30):
    """The oracle (float32, thread pool) on batch 0 of the workload, all heads,
    repeated until about `min_seconds` of CPU work have run.  One worker per
    CPU this process may run on, at most 16 (one GPU's share of the host)."""
    import numpy as np

    import oracle
    from sparse_long_sequence_dilated_amd import inputs
    host_cpus = os.cpu_count() or 1
    usable = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else host_cpus
    workers = max(1, min(16, usable))
    q, k, v, do = inputs.draw((1, wl.N, wl.H, wl.D), wl.seed, 4, wl.dtype)
    passes, t = 0, 0.0
    while passes < max_passes and (passes == 0 or t < min_seconds):
        t0 = time.perf_counter()
        o, lse = oracle.forward(q, k, v, wl.patterns, wl.causal, wl.scale, dtype=np.float32,
                                workers=workers)
        if wl.backward:
            oracle.backward(q, k, v, o, lse, do, wl.patterns, wl.causal, wl.scale, dtype=np.float32,
                            workers=workers)
        t += time.perf_counter() - t0
        passes += 1
    per_pass = t / passes
    return {"value": wl.B * wl.N / (per_pass * wl.B), "unit": "tokens/s", "cores": workers,
            "kind": "oracle", "threads": workers, "host_cpus": host_cpus, "usable_cpus": usable,
            "cpu_model": cpu_model(),
            "sample": (f"{'fwd+bwd' if wl.backward else 'fwd'} of batch 1 of {wl.B} (all {wl.H} heads, "
                       f"full N={wl.N}, all patterns), {passes} passes in {t:.1f} s; float32 NumPy "
                       f"oracle, one worker thread per usable CPU up to 16 ({workers} of "
                       f"{usable} usable, {host_cpus} on the host), BLAS at 1 thread each; "
                       f"scaled by {wl.B} to the full batch")}


def layer_bench(B, N, steps, warmup):
    """The attention layer (Q/K/V projections, dilated attention, output
    projection; random weights) at 768 dimensions and 12 heads with the 32K
    pattern set: forward, and forward plus backward, per step."""
    import torch
    from sparse_long_sequence_dilated_amd import dla, inputs
    H, D = 12, 64
    E = H * D
    pats = inputs.geometric_patterns(2048, 2, 5)
    scale = 1.0 / math.sqrt(D)
    g = torch.Generator(device="cuda")
    g.manual_seed(3000 + N)
    x = torch.randn((B, N, E), device="cuda", generator=g).bfloat16()
    dy = torch.randn_like(x)
    w_qkv = (torch.randn((E, 3 * E), device="cuda", generator=g) / math.sqrt(E)).bfloat16()
    w_o = (torch.randn((E, E), device="cuda", generator=g) / math.sqrt(E)).bfloat16()
    blas = dla.Blas()
    ws_f, ws_b = dla.layer_plan_check(pats, True, scale, B, N, H)
    wsf = torch.empty(ws_f, dtype=torch.uint8, device="cuda")
    wsb = torch.empty(ws_b, dtype=torch.uint8, device="cuda")
    saved = {}

    def fstep():
        saved["f"] = dla.layer_forward(x, w_qkv, w_o, pats, blas, True, scale, workspace=wsf)

    def bstep():
        fstep()
        _, qkv, attn, lse = saved["f"]
        dla.layer_backward(x, w_qkv, w_o, qkv, attn, lse, dy, pats, blas, True, scale, workspace=wsb)

    pairs = dla.pair_count(pats, True, B, N, H)
    gemm_flops = 8 * B * N * E * E
    out = {"workload": f"attention layer E={E} H={H} (random weights), bf16, B={B}, N={N}, "
                       f"causal, patterns {[list(p) for p in pats]}"}
    for name, fn, mult in (("forward", fstep, 1), ("fwd_bwd", bstep, 3)):
        ms, fams, _ = time_steps(fn, steps, warmup, reps=3)
        attn_ms = sum(t for _, t in fams.values()) / steps
        flops = mult * gemm_flops + (4 if mult == 1 else 14) * D * pairs
        out[name] = {"tokens_per_s": B * N / (ms * 1e-3), "ms": ms,
                     "useful_tflops": flops / (ms * 1e-3) / 1e12,
                     "attention_kernels_ms": attn_ms, "rest_ms": ms - attn_ms}
    blas.close()
    del x, dy, w_qkv, w_o, wsf, wsb, saved
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="C5")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-forward-lines", action="store_true")
    ap.add_argument("--layer-only", action="store_true",
                    help="only run the attention-layer legs (for profiling them)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path, so --gpus must be 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_long_sequence_dilated_amd import dla, inputs
    torch.cuda.set_device(0)

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 5}))
        return

    if args.layer_only:
        print(json.dumps({"layer": [layer_bench(16, 2048, args.steps, args.warmup),
                                    layer_bench(1, 32768, args.steps, args.warmup)]}), flush=True)
        return

    wl = inputs.WORKLOADS[args.workload]
    if wl.dtype != "bf16":
        raise SystemExit("the step benchmark runs the bf16 workloads")
    tensors = gpu_inputs(wl, 4, 1000 + wl.seed)
    q, k, v, do = tensors
    ws_f, ws_b = dla.plan_check(wl.patterns, wl.causal, wl.scale, wl.B, wl.N, wl.H)
    ws_fwd = torch.empty(max(ws_f, 1), dtype=torch.uint8, device="cuda")
    ws_bwd = torch.empty(max(ws_b, 1), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((wl.B, wl.H, wl.N), dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))

    def step():
        dla.forward(q, k, v, wl.patterns, wl.causal, wl.scale, out=o, lse=lse, workspace=ws_fwd)
        if wl.backward:
            dla.backward(q, k, v, o, lse, do, wl.patterns, wl.causal, wl.scale, dq=dq, dk=dk,
                         dv=dv, workspace=ws_bwd)

    ms, fams, ms_events = time_steps(step, args.steps, args.warmup)
    pairs = dla.pair_count(wl.patterns, wl.causal, wl.B, wl.N, wl.H)
    flops = (14 if wl.backward else 4) * wl.D * pairs
    tflops = flops / (ms * 1e-3) / 1e12

    dom = max(fams, key=lambda f: fams[f][1])
    n_launch, dom_ms = fams[dom]
    work, unit, bound = family_work(dom, wl, pairs)
    launches_per_step = n_launch / args.steps
    avg_launch_s = dom_ms * 1e-3 / n_launch
    per_launch = work / launches_per_step
    if unit == "flop":
        achieved, peak, runit = per_launch / avg_launch_s / 1e12, BF16_PEAK_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, runit = per_launch / avg_launch_s / 1e9, HBM_PEAK_GBS, "GB/s"
    roofline = {"bound": bound, "kernel": dom, "achieved": achieved, "peak": peak, "unit": runit,
                "frac": achieved / peak, "traffic": traffic_for(dom, launches_per_step),
                "launches_per_step": launches_per_step, "avg_launch_us": avg_launch_s * 1e6,
                "work_per_step": work, "work_unit": unit}
    kernels = {f: {"launches_per_step": n / args.steps, "us_per_step": 1e3 * t / args.steps}
               for f, (n, t) in fams.items()}
    cold = cold_kernel_ms(step, min(args.steps, 10))
    del tensors, q, k, v, do, ws_fwd, ws_bwd, o, lse, dq, dk, dv
    torch.cuda.empty_cache()

    extra = []
    if not args.no_forward_lines:
        extra.append(forward_only("C1", max(5, args.steps), args.warmup))
        extra.append(forward_only("C2", max(5, args.steps), args.warmup))
        extra.append(forward_only("C3", max(5, args.steps), args.warmup))
        extra.append(forward_only("C4", max(3, args.steps // 4), 1))
        extra.append(fp8_forward("C3", max(5, args.steps), args.warmup))
        shard = shard_forward("C4", 8, 7, max(3, args.steps // 2), 3)
        layers = [layer_bench(16, 2048, max(5, args.steps // 2), 2),
                  layer_bench(1, 32768, max(5, args.steps // 2), 2)]
    cpu = None if args.no_cpu_baseline else cpu_baseline(wl)

    line = {
        "metric": METRIC, "value": wl.B * wl.N / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.describe(), "B": wl.B, "N": wl.N, "H": wl.H, "D": wl.D,
                   "patterns": [list(p) for p in wl.patterns], "causal": wl.causal,
                   "step": "dla_forward + dla_backward" if wl.backward else "dla_forward"},
        "useful_tflops": tflops, "pct_bf16_peak": 100.0 * tflops / BF16_PEAK_TFLOPS,
        "ms_per_step_events": ms_events,
        "roofline": roofline, "kernels": kernels, "forward_only": extra, "cpu_baseline": cpu,
        "cold_cache": {"kernel_ms_per_step": cold, "tokens_per_s": wl.B * wl.N / (cold * 1e-3),
                       "note": "512 MB written between steps; kernel time only"},
    }
    if not args.no_forward_lines:
        line["shard_forward"] = shard
        line["layer"] = layers
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
