#!/usr/bin/env python3
"""Benchmark of the fused attention forward hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step = one mha_fwd_bf16 call on the headline workload (b1 hq128 hk128
8192^2 dqk192/dv128 causal, bf16), inputs resident in HBM.  The timed region is
exactly K steps bracketed by torch.cuda.synchronize(); the kernel's average
duration comes from HIP events recorded on the stream the kernel runs on.
The same run also times the quantised path on its own workloads (b1 h16 4096^2
d128 non-causal: k_smooth_mean + mha_fwd_fp8, and the same with mha_fwd_mxfp8)
and reports them under "fp8_call" and "mxfp8_call".

Prints ONE JSON line.  Extra modes used for HBM-traffic calibration:
    python bench.py --calibrate-copy BYTES   (a plain device copy of BYTES, for counter scaling)
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

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published
# The pages' own times for the same shapes: the retune page's tuned Triton kernel (gfx950) for
# the bf16 shapes, the gate page's eager mha_v4 call (MI355X) for the FP8 ones.
PAGES_BF16_US = {"mla_d192_d128_causal": 4083.2, "mla_d192_d128_noncausal": 7086.1,
                 "gqa_d128_8192_causal": 2686.6, "gqa_d64_causal": 333.0}
PAGES_FP8_CALL_US = {"fp8_ksmooth_d128": 219.2, "fp8_long_h5": 3857.2, "mxfp8_ksmooth_d128": 140.8}

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_bf16_mla_d192_d128_causal_traffic.json")
KERNEL_SOURCES = ["head_attention_forward_flash_amd/csrc/attn_fwd_bf16.hip",
                  "head_attention_forward_flash_amd/csrc/device_common.h"]


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_bytes():
    """HBM bytes per launch from the committed counter profile, or None if stale/missing."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_source_sha():
        return None
    return float(t["hbm_bytes_per_launch"])


def time_launches(fn, steps, warmup, stream, min_warm_s=0.3):
    """Average device time per call over exactly `steps` calls (HIP events on `stream`).

    Warm-up is at least `warmup` calls and at least `min_warm_s` seconds of calls, so
    that short kernels are timed at the clock the GPU settles to under load, not while
    it ramps up.
    """
    import torch
    t_warm = time.perf_counter()
    n = 0
    while n < warmup or time.perf_counter() - t_warm < min_warm_s:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / steps, wall


def cpu_baseline(w, q, k, v, budget_s=12.0, max_heads=64):
    """Time the float64 oracle on whole heads of the workload until ~budget_s of CPU work."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    import workloads
    grp = w.hq // w.hk
    sinks = workloads.make_sinks(w)
    ext = w.window_left >= 0 or w.window_right >= 0 or sinks is not None
    flops, elapsed, heads = 0.0, 0.0, 0
    for h in range(min(max_heads, w.hq)):
        g = h // grp
        qh = q[0:1, :, h:h + 1].float().numpy()
        kh = k[0:1, :, g:g + 1].float().numpy()
        vh = v[0:1, :, g:g + 1].float().numpy()
        t0 = time.perf_counter()
        if ext:
            oracle.attention_window_sink(qh, kh, vh, scale=w.scale, causal=w.causal, window_left=w.window_left,
                                         window_right=w.window_right,
                                         sinks=None if sinks is None else sinks[h:h + 1].double().numpy())
        else:
            oracle.attention_forward(qh, kh, vh, scale=w.scale, causal=w.causal)
        elapsed += time.perf_counter() - t0
        flops += w.flops() / (w.b * w.hq)
        heads += 1
        if elapsed >= budget_s:
            break
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{heads} of {w.hq} query heads (batch 0, all {w.sq} rows) of {w.name}, float64 NumPy; "
                      f"{elapsed:.1f} s",
            "seconds": round(elapsed, 2)}


def bench_fp8(steps, warmup, dev, name="fp8_ksmooth_d128"):
    """k_smooth_mean + the quantised call (mha_fwd_fp8, or mha_fwd_mxfp8 for an MXFP8 workload)."""
    import torch
    import head_attention_forward_flash_amd as mha
    import workloads
    w = workloads.WORKLOADS[name]
    q, k, v = (t.to(dev) for t in workloads.make_qkv(w))
    o = torch.empty((w.b, w.sq, w.hq, w.d_v), dtype=torch.bfloat16, device=dev)
    fwd = mha.mha_fwd_mxfp8 if w.mx else mha.mha_fwd_fp8
    ws_bytes = (mha.mha_fwd_mxfp8_workspace_bytes if w.mx else mha.mha_fwd_fp8_workspace_bytes)(
        w.b, w.hq, w.hk, w.sq, w.sk, w.d_qk)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    gws = torch.empty(max(256, mha.k_smooth_mean_workspace_bytes(w.b, w.hk, w.sk, w.d_qk)), dtype=torch.uint8,
                      device=dev)
    try:
        mean, _ = mha.k_smooth_mean(k, workspace=gws)
        fwd(q, k, v, k_mean=mean, out=o, workspace=ws, lse=False)
    except mha.MhaError as e:
        return {"available": False, "reason": str(e)}
    stream = torch.cuda.current_stream(dev)

    def call():
        m, _ = mha.k_smooth_mean(k, workspace=gws)
        fwd(q, k, v, k_mean=m, out=o, workspace=ws, lse=False)

    ms, _ = time_launches(call, steps, warmup, stream)
    tf = w.flops() / (ms * 1e-3) / 1e12
    return {"available": True, "workload": w.name, "us_per_call": round(ms * 1e3, 2), "tflops": round(tf, 1),
            "frac_of_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4), "pages_us_per_call": PAGES_FP8_CALL_US.get(w.name),
            "recipe": "mxfp8 (E8M0 per 32 channels)" if w.mx else "fp8 (fp32 scale per 128 tokens)",
            "includes": "k_smooth_mean (2 kernels) + quantisation + fp8 attention, device time by HIP events"}


def bench_varlen(steps, warmup, dev, name):
    """mha_fwd_bf16_varlen on a packed-sequence workload."""
    import itertools
    import torch
    import head_attention_forward_flash_amd as mha
    import workloads
    w = workloads.VARLEN_WORKLOADS[name]
    lens = w.lengths()
    q, k, v = (t.to(dev) for t in w.make_qkv())
    cu = torch.tensor([0] + list(itertools.accumulate(lens)), dtype=torch.int32, device=dev)
    o = torch.empty((q.shape[0], w.hq, w.d_v), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    def call():
        mha.mha_fwd_bf16_varlen(q, k, v, cu, cu, max(lens), max(lens), causal=w.causal, out=o, lse=False)

    ms, _ = time_launches(call, steps, warmup, stream)
    tf = w.flops() / (ms * 1e-3) / 1e12
    return {"workload": w.name, "sequences": len(lens), "tokens": sum(lens), "us_per_launch": round(ms * 1e3, 1),
            "tflops": round(tf, 1), "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mla_d192_d128_causal")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--fp8-workload", default="fp8_ksmooth_d128", help="FP8 workload of the fp8_call field")
    ap.add_argument("--fp8-only", action="store_true", help="time only the quantised call; print its JSON")
    ap.add_argument("--varlen-workload", default=None, help="time only this packed-sequence workload; print its JSON")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES")
    a = ap.parse_args()

    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (attention heads shard "
              "across GPUs without communication, so one GPU's share of the heads is the measured unit).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)

    if a.calibrate_copy:
        n = a.calibrate_copy
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n}))
        return

    import head_attention_forward_flash_amd as mha
    import workloads
    if a.varlen_workload:
        print(json.dumps(bench_varlen(a.steps, a.warmup, dev, a.varlen_workload)), flush=True)
        return
    if a.fp8_only:
        print(json.dumps(bench_fp8(max(20, a.steps), a.warmup, dev, a.fp8_workload)), flush=True)
        return
    w = workloads.WORKLOADS[a.workload]
    if w.fp8:
        print("--workload must be a bf16 workload", file=sys.stderr)
        sys.exit(2)
    qc, kc, vc = workloads.make_qkv(w)
    q, k, v = qc.to(dev), kc.to(dev), vc.to(dev)
    o = torch.empty((w.b, w.sq, w.hq, w.d_v), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.b, w.hq, w.sq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    sinks = workloads.make_sinks(w)
    if w.window_left >= 0 or w.window_right >= 0 or sinks is not None:
        sinks_d = None if sinks is None else sinks.to(dev)

        def step():
            mha.mha_fwd_bf16_window_sink(q, k, v, causal=w.causal, window_left=w.window_left,
                                         window_right=w.window_right, sinks=sinks_d, softmax_scale=w.scale, out=o)
    else:
        def step():
            mha.mha_fwd_bf16(q, k, v, causal=w.causal, softmax_scale=w.scale, out=o)

    torch.cuda.synchronize()
    ms, wall = time_launches(step, a.steps, a.warmup, stream)
    tflops = w.flops() / (ms * 1e-3) / 1e12

    traffic = traffic_bytes()
    roofline = {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                "traffic": None if traffic is None else int(traffic)}

    fp8 = None if a.no_fp8 else bench_fp8(max(20, a.steps), a.warmup, dev, a.fp8_workload)
    mxfp8 = None if a.no_fp8 else bench_fp8(max(20, a.steps), a.warmup, dev, "mxfp8_ksmooth_d128")
    cpu = None if a.no_cpu_baseline else cpu_baseline(w, qc, kc, vc)

    pages_tflops = w.flops() / (PAGES_BF16_US[w.name] * 1e-6) / 1e12 if w.name in PAGES_BF16_US else None
    out = {
        "metric": "attention fwd TFLOP/s (causal-halved) and % of MI355X MFMA peak per config",
        "value": round(tflops, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None if pages_tflops is None else round(tflops / pages_tflops, 3),
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 Q/K/V)",
        "config": {"workload": w.name, "b": w.b, "hq": w.hq, "hk": w.hk, "sq": w.sq, "sk": w.sk,
                   "d_qk": w.d_qk, "d_v": w.d_v, "causal": w.causal, "parallelism": "none (1 GPU)"},
        "frac_of_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "us_per_launch": round(ms * 1e3, 1),
        "timed_wall_s": round(wall, 3),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "fp8_call": fp8,
        "mxfp8_call": mxfp8,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
