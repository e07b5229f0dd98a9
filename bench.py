#!/usr/bin/env python3
"""Benchmark of the fused attention forward hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step = one mha_fwd_bf16 call on the headline workload (b1 hq128 hk128
8192^2 dqk192/dv128 causal, bf16), inputs resident in HBM.  The timed region is
exactly K steps bracketed by torch.cuda.synchronize(); the kernel's average
duration comes from HIP events recorded on the stream the kernel runs on.

The same run then times every config on its own (the "configs" block: the five
configs the metric is quoted on) and the further shapes (the "extra" block), each
with the pages' statistics over single dispatches: 200 dispatches after 20
warm-up calls (and at least 0.3 s of warm-up), each bracketed by its own pair of
HIP events, reported as the chronological middle-80 % trimmed mean (the first and
last 10 % of the dispatches in time order dropped), the median and the maximum.
Configs 1-5 also carry the float64 oracle's time on a bounded sample of the same
workload, on all BLAS threads and on one.

Prints ONE JSON line.  Other modes:
    python bench.py --calibrate-copy BYTES        a plain device copy of BYTES (counter scaling)
    python bench.py --summarize-trace CSV [RE]    per-kernel statistics of a rocprofv3 kernel trace
    python bench.py --summarize-counters CSV...   per-kernel counters of rocprofv3 --pmc passes
    python bench.py --fp8-only / --varlen-workload NAME / --workload NAME --configs none
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published
# The pages' own times for the same shapes: the retune page's tuned Triton kernel (gfx950) for
# the bf16 shapes (its "golden" column for the two TP8 d128 shapes, which it times only there),
# the gate page's eager mha_v4 call (MI355X) for the FP8 ones.
PAGES_BF16_US = {"mla_d192_d128_causal": 4083.2, "mla_d192_d128_noncausal": 7086.1,
                 "gqa_d128_8192_causal": 2686.6, "gqa_d64_causal": 333.0,
                 "gqa8_d128_tp8_noncausal": 330.0, "gqa5_d128_tp8_noncausal": 303.2}
PAGES_FP8_CALL_US = {"fp8_ksmooth_d128": 219.2, "fp8_long_h5": 3857.2, "mxfp8_ksmooth_d128": 140.8}

# The five configs the metric is quoted on, in order, and the further shapes timed beside them.
CONFIGS = [("c1", "tiny_d64"), ("c2", "gqa_d64_causal"), ("c3", "gqa_d128_causal"),
           ("c4", "mla_d192_d128_causal"), ("c5", "fp8_ksmooth_d128")]
EXTRA = ["gqa8_d128_tp8_noncausal", "gqa5_d128_tp8_noncausal", "gqa8_d128_tp8_causal", "gqa5_d128_tp8_causal",
         "mla_d192_d128_noncausal",
         "gqa_d128_8192_causal", "mla_d192_d128_tp8_causal", "gptoss_swa_sink_d64", "gptoss_sink_d64",
         "vd32_noncausal", "mxfp8_ksmooth_d128", "fp8_long_h5", "varlen:varlen_gqa_d128_causal"]

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


def _warm(fn, warmup, min_warm_s):
    import torch
    t_warm = time.perf_counter()
    n = 0
    while n < warmup or time.perf_counter() - t_warm < min_warm_s:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def time_launches(fn, steps, warmup, stream, min_warm_s=0.3):
    """Average device time per call over exactly `steps` calls (HIP events on `stream`).

    Warm-up is at least `warmup` calls and at least `min_warm_s` seconds of calls, so
    that short kernels are timed at the clock the GPU settles to under load, not while
    it ramps up.
    """
    import torch
    _warm(fn, warmup, min_warm_s)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / steps, wall


def trimmed_stats(us):
    """The pages' statistics of a chronological series of single-dispatch times (us)."""
    import numpy as np
    a = np.asarray(us, dtype=np.float64)
    cut = len(a) // 10
    mid = a[cut:len(a) - cut] if len(a) > 2 * cut else a
    return {"n": int(len(a)), "trimmed_mean_us": round(float(mid.mean()), 2),
            "median_us": round(float(np.median(a)), 2), "max_us": round(float(a.max()), 2),
            "min_us": round(float(a.min()), 2), "mean_us": round(float(a.mean()), 2)}


def time_dispatches(fn, stream, n=200, warmup=20, min_warm_s=0.3):
    """n single dispatches of fn, each between its own two HIP events on `stream`."""
    import torch
    _warm(fn, warmup, min_warm_s)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return trimmed_stats([a.elapsed_time(b) * 1e3 for a, b in ev])


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def _oracle_heads(w, q, k, v, heads):
    """Run the float64 oracle on whole query heads of batch 0 (and, for a quantised workload, the
    oracle's own gate and quantisation first); returns the seconds taken."""
    import numpy as np
    import oracle
    import workloads
    t0 = time.perf_counter()
    if w.fp8:
        kf = k.float().numpy()
        mu = oracle.k_smooth_mean(kf)["mean"].astype(np.float32)
        fwd = oracle.mxfp8_attention_forward if w.mx else oracle.fp8_attention_forward
        fwd(q.float().numpy(), kf, v.float().numpy(), mu=mu, scale=w.scale, causal=w.causal, heads=heads,
            batches=[0])
        return time.perf_counter() - t0
    grp = w.hq // w.hk
    sinks = workloads.make_sinks(w)
    ext = w.window_left >= 0 or w.window_right >= 0 or sinks is not None
    for h in heads:
        g = h // grp
        qh = q[0:1, :, h:h + 1].float().numpy()
        kh = k[0:1, :, g:g + 1].float().numpy()
        vh = v[0:1, :, g:g + 1].float().numpy()
        if ext:
            oracle.attention_window_sink(qh, kh, vh, scale=w.scale, causal=w.causal, window_left=w.window_left,
                                         window_right=w.window_right,
                                         sinks=None if sinks is None else sinks[h:h + 1].double().numpy())
        else:
            oracle.attention_forward(qh, kh, vh, scale=w.scale, causal=w.causal)
    return time.perf_counter() - t0


def oracle_timing(w, q, k, v, budget_s, budget_1core_s):
    """The oracle on whole heads of batch 0 until ~budget_s of CPU work (all BLAS threads), and
    again on one thread until ~budget_1core_s; FLOP rates count the workload's algorithmic FLOPs
    of the heads covered."""
    from threadpoolctl import threadpool_limits
    per_head = w.flops() / (w.b * w.hq)

    def run(budget):
        if w.fp8:   # the quantised oracle quantises every head of the tensors first: one run on 2 heads
            heads = min(2, w.hq)
            return heads, _oracle_heads(w, q, k, v, list(range(heads)))
        heads, secs = 0, 0.0
        while heads < w.hq and (heads == 0 or secs < budget):
            secs += _oracle_heads(w, q, k, v, [heads])
            heads += 1
        return heads, secs

    threads = blas_threads()
    heads, secs = run(budget_s)
    with threadpool_limits(1):
        heads1, secs1 = run(budget_1core_s)
    what = "gate + quantisation + attention, " if w.fp8 else ""
    return {"kind": "oracle", "threads": threads, "seconds": round(secs, 3),
            "sample": f"{heads} of {w.hq} query heads (batch 0, all {w.sq} rows) of {w.name}, {what}float64 NumPy",
            "tflops": per_head * heads / secs / 1e12, "seconds_1core": round(secs1, 3),
            "sample_1core": f"{heads1} of {w.hq} query heads on 1 thread",
            "tflops_1core": per_head * heads1 / secs1 / 1e12}


def _bf16_step(w, q, k, v, o):
    import torch
    import head_attention_forward_flash_amd as mha
    import workloads
    sinks = workloads.make_sinks(w)
    if w.window_left >= 0 or w.window_right >= 0 or sinks is not None:
        sinks_d = None if sinks is None else sinks.to(q.device)

        def step():
            mha.mha_fwd_bf16_window_sink(q, k, v, causal=w.causal, window_left=w.window_left,
                                         window_right=w.window_right, sinks=sinks_d, softmax_scale=w.scale, out=o)
    else:
        # the key-range split's plan and workspace are set up once, outside the timed calls
        n_split = mha.mha_fwd_bf16_split_plan(w.b, w.hq, w.hk, w.sq, w.sk, w.d_qk, w.d_v, w.causal)
        ws = None
        if n_split > 1:
            ws = torch.empty(mha.mha_fwd_bf16_split_workspace_bytes(w.b, w.hq, w.sq, w.d_qk, w.d_v, n_split),
                             dtype=torch.uint8, device=q.device)

        def step():
            mha.mha_fwd_bf16(q, k, v, causal=w.causal, softmax_scale=w.scale, out=o, n_split=n_split, workspace=ws)
        step.n_split = n_split
    return step


def _rates(stats_us, flops, peak):
    us = stats_us["trimmed_mean_us"]
    tf = flops / (us * 1e-6) / 1e12
    return round(tf, 1), round(tf / peak, 4)


def bench_bf16(w, dev, n, warmup, oracle_budget=None, tiny=False):
    """Single-dispatch statistics of one bf16 workload (and the oracle's time on a sample)."""
    import torch
    import workloads
    qc, kc, vc = workloads.make_qkv(w)
    q, k, v = qc.to(dev), kc.to(dev), vc.to(dev)
    o = torch.empty((w.b, w.sq, w.hq, w.d_v), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    step = _bf16_step(w, q, k, v, o)
    st = time_dispatches(step, stream, n, warmup)
    out = {"workload": w.name, "shape": w.description, "kernel": "attn_fwd_bf16", "dispatch_us": st}
    if getattr(step, "n_split", 1) > 1:
        out["n_split"] = step.n_split
        out["kernel"] = "attn_fwd_bf16 (key ranges) + attn_split_merge"
        out["note"] = "each query block's keys in n_split ranges, merged by a second kernel; timed as one call"
    del step
    if tiny:
        out["note"] = "launch-latency bound (8.4 MFLOP): reported in us only"
    else:
        out["tflops"], out["frac_of_bf16_peak"] = _rates(st, w.flops(), PEAK_BF16_TFLOPS)
    if w.name in PAGES_BF16_US:
        out["pages_us"] = PAGES_BF16_US[w.name]
        out["speedup_vs_pages"] = round(PAGES_BF16_US[w.name] / st["trimmed_mean_us"], 3)
    del q, k, v, o
    torch.cuda.empty_cache()
    if oracle_budget is not None:
        out["oracle"] = oracle_timing(w, qc, kc, vc, *oracle_budget)
    return out


def bench_quantised(w, dev, n, warmup, oracle_budget=None):
    """The quantised call three ways: the gate alone, quantisation + fp8 attention, and the whole
    call (gate + quantisation + attention), as in the gate page's per-call times."""
    import torch
    import head_attention_forward_flash_amd as mha
    import workloads
    qc, kc, vc = workloads.make_qkv(w)
    q, k, v = qc.to(dev), kc.to(dev), vc.to(dev)
    o = torch.empty((w.b, w.sq, w.hq, w.d_v), dtype=torch.bfloat16, device=dev)
    fwd = mha.mha_fwd_mxfp8 if w.mx else mha.mha_fwd_fp8
    ws_bytes = (mha.mha_fwd_mxfp8_workspace_bytes if w.mx else mha.mha_fwd_fp8_workspace_bytes)(
        w.b, w.hq, w.hk, w.sq, w.sk, w.d_qk)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    gws = torch.empty(max(256, mha.k_smooth_mean_workspace_bytes(w.b, w.hk, w.sk, w.d_qk)), dtype=torch.uint8,
                      device=dev)
    try:
        mean, _ = mha.k_smooth_mean(k, workspace=gws)
    except mha.MhaError as e:
        return {"available": False, "reason": str(e)}
    stream = torch.cuda.current_stream(dev)

    def gate():
        mha.k_smooth_mean(k, workspace=gws)

    def attn():
        fwd(q, k, v, k_mean=mean, out=o, workspace=ws, lse=True)

    def call():
        m, _ = mha.k_smooth_mean(k, workspace=gws)
        fwd(q, k, v, k_mean=m, out=o, workspace=ws, lse=True)

    g, a, c = (time_dispatches(f, stream, n, warmup) for f in (gate, attn, call))
    out = {"workload": w.name, "shape": w.description, "available": True,
           "recipe": "mxfp8 (E8M0 per 32 channels)" if w.mx else "fp8 (fp32 scale per 128 tokens)",
           "gate_us": g, "quant_attention_us": a, "whole_call_us": c, "lse": True,
           "note": "k_smooth_mean = k_moments + k_fold_gate; quant_attention = quant_fp8 + attn_fwd_fp8 "
                   "(the split between these two kernels is in the rocprofv3 trace)"}
    out["tflops_whole_call"], out["frac_of_fp8_peak_whole_call"] = _rates(c, w.flops(), PEAK_FP8_TFLOPS)
    out["tflops_quant_attention"], out["frac_of_fp8_peak_quant_attention"] = _rates(a, w.flops(), PEAK_FP8_TFLOPS)
    if w.name in PAGES_FP8_CALL_US:
        out["pages_us_per_call"] = PAGES_FP8_CALL_US[w.name]
        out["speedup_vs_pages"] = round(PAGES_FP8_CALL_US[w.name] / c["trimmed_mean_us"], 3)
    del q, k, v, o, ws
    torch.cuda.empty_cache()
    if oracle_budget is not None:
        out["oracle"] = oracle_timing(w, qc, kc, vc, *oracle_budget)
    return out


def bench_varlen(dev, name, n, warmup):
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
        mha.mha_fwd_bf16_varlen(q, k, v, cu, cu, max(lens), max(lens), causal=w.causal, out=o)

    st = time_dispatches(call, stream, n, warmup)
    out = {"workload": w.name, "shape": w.description, "kernel": "attn_fwd_bf16 (varlen)", "sequences": len(lens),
           "tokens": sum(lens), "dispatch_us": st}
    out["tflops"], out["frac_of_bf16_peak"] = _rates(st, w.flops(), PEAK_BF16_TFLOPS)
    del q, k, v, o
    torch.cuda.empty_cache()
    return out


def summarize_trace(path, pattern=None):
    """Per-kernel statistics of a rocprofv3 kernel trace (CSV), one row per (kernel, grid size)
    (so that workloads sharing a kernel instance stay apart): calls, mean, the chronological
    middle-80 % trimmed mean, median and max, plus the registers and LDS of the code object."""
    import csv
    rows = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            if pattern and not re.search(pattern, name):
                continue
            grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            wg = int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"])
            d = rows.setdefault((name, grid // max(wg, 1)), {"t": [], "meta": r})
            d["t"].append((int(r["Start_Timestamp"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    print("| kernel | workgroups | calls | mean us | trimmed mean us (middle 80 %) | median us | max us "
          "| VGPR | AGPR | SGPR | LDS B |")
    print("|---|---|---|---|---|---|---|---|---|---|---|")
    for (name, nwg), d in rows.items():
        st = trimmed_stats([t for _, t in sorted(d["t"])])
        m = d["meta"]
        print(f"| `{name}` | {nwg} | {st['n']} | {st['mean_us']} | {st['trimmed_mean_us']} | {st['median_us']} "
              f"| {st['max_us']} | {m.get('VGPR_Count')} | {m.get('Accum_VGPR_Count')} | {m.get('SGPR_Count')} "
              f"| {m.get('LDS_Block_Size')} |")


def summarize_counters(paths, pattern=None, simds=1024, xcds=8):
    """Mean per dispatch of every counter in rocprofv3 --pmc CSVs (one or more passes), per
    (kernel, grid size), and the derived figures: core clock, matrix-pipe busy fraction per
    SIMD, VALU-active and waiting fractions of wave time, instructions per MFMA, LDS bank
    conflicts.  GRBM_GUI_ACTIVE sums the XCDs' busy cycles; SQ_VALU_MFMA_BUSY_CYCLES sums the
    SIMDs'; SQ_WAVE_CYCLES, SQ_WAIT_INST_ANY and SQ_ACTIVE_INST_* count quad-cycles per wave;
    SQ_INSTS_VALU includes the MFMAs."""
    import csv
    import statistics
    acc = {}
    for path in paths:
        with open(path) as f:
            for r in csv.DictReader(f):
                name = r["Kernel_Name"]
                if pattern and not re.search(pattern, name):
                    continue
                d = acc.setdefault((name, int(r["Grid_Size"])), {"c": {}, "dur": {}})
                d["c"].setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
                key = (path, r["Dispatch_Id"])
                d["dur"][key] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    for (name, grid), d in acc.items():
        c = {k: sum(v) / len(v) for k, v in d["c"].items()}
        n = min(len(v) for v in d["c"].values())
        dur = statistics.median(d["dur"].values())
        print(f"### `{name}`, grid {grid} threads\n")
        print(f"Dispatches averaged: {n} or more per counter; median dispatch {dur:.1f} us.\n")
        print("| counter | mean per dispatch |\n|---|---|")
        for k in sorted(c):
            print(f"| {k} | {c[k]:.4g} |")
        print()
        g = c.get("GRBM_GUI_ACTIVE")
        if g:
            cyc = g / xcds
            print(f"* core clock: {cyc / dur / 1e3:.2f} GHz ({cyc:.4g} cycles per XCD)")
            if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
                print(f"* matrix pipe busy: {100 * c['SQ_VALU_MFMA_BUSY_CYCLES'] / (simds * cyc):.1f}% of cycles per SIMD")
        wc = c.get("SQ_WAVE_CYCLES")
        if wc:
            for k, label in (("SQ_ACTIVE_INST_VALU", "VALU active"), ("SQ_ACTIVE_INST_LDS", "LDS active"),
                             ("SQ_WAIT_INST_ANY", "waiting at s_waitcnt / dependencies")):
                if k in c:
                    print(f"* {label}: {100 * c[k] / wc:.1f}% of wave time")
        mf = c.get("SQ_INSTS_MFMA")
        if mf:
            for k, label in (("SQ_INSTS_VALU", "VALU (besides the MFMAs)"), ("SQ_INSTS_VALU_TRANS_F32", "of them exp"),
                             ("SQ_INSTS_LDS", "LDS"), ("SQ_INSTS_SALU", "SALU")):
                if k in c:
                    v = c[k] - mf if k == "SQ_INSTS_VALU" else c[k]
                    print(f"* {label}: {v / mf:.2f} per MFMA")
        if c.get("SQ_LDS_IDX_ACTIVE"):
            print(f"* LDS bank conflicts: {c.get('SQ_LDS_BANK_CONFLICT', 0):.4g} cycles "
                  f"({100 * c.get('SQ_LDS_BANK_CONFLICT', 0) / c['SQ_LDS_IDX_ACTIVE']:.2f}% of LDS-active cycles)")
        for k in ("FETCH_SIZE", "WRITE_SIZE"):
            if k in c:
                print(f"* {k}: {c[k]:.6g} KiB per dispatch")
        print()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mla_d192_d128_causal")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip every oracle timing")
    ap.add_argument("--configs", default="all", choices=["all", "main", "none"],
                    help="per-config blocks: all (configs and extra shapes), main (configs only), none")
    ap.add_argument("--no-fp8", action="store_true", help="same as --configs none (headline only)")
    ap.add_argument("--dispatches", type=int, default=200, help="single dispatches per config block")
    ap.add_argument("--fp8-workload", default="fp8_ksmooth_d128")
    ap.add_argument("--fp8-only", action="store_true", help="time only the quantised call; print its JSON")
    ap.add_argument("--varlen-workload", default=None, help="time only this packed-sequence workload; print its JSON")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES")
    ap.add_argument("--summarize-trace", nargs="+", metavar=("CSV", "REGEX"))
    ap.add_argument("--summarize-counters", nargs="+", metavar="CSV",
                    help="rocprofv3 --pmc counter CSVs (one per pass); --kernel-regex filters")
    ap.add_argument("--kernel-regex", default=None)
    a = ap.parse_args()
    if a.no_fp8:
        a.configs = "none"

    if a.summarize_trace:
        summarize_trace(a.summarize_trace[0], a.summarize_trace[1] if len(a.summarize_trace) > 1 else None)
        return
    if a.summarize_counters:
        summarize_counters(a.summarize_counters, a.kernel_regex)
        return

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

    import head_attention_forward_flash_amd as mha  # noqa: F401  (fails loudly without libmha.so)
    import workloads
    n, nw = a.dispatches, 20
    if a.varlen_workload:
        print(json.dumps(bench_varlen(dev, a.varlen_workload, n, nw)), flush=True)
        return
    if a.fp8_only:
        print(json.dumps(bench_quantised(workloads.WORKLOADS[a.fp8_workload], dev, n, nw)), flush=True)
        return
    w = workloads.WORKLOADS[a.workload]
    if w.fp8:
        print("--workload must be a bf16 workload", file=sys.stderr)
        sys.exit(2)

    # ---- the headline: exactly K timed steps of the workload
    qc, kc, vc = workloads.make_qkv(w)
    q, k, v = qc.to(dev), kc.to(dev), vc.to(dev)
    o = torch.empty((w.b, w.sq, w.hq, w.d_v), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    step = _bf16_step(w, q, k, v, o)
    torch.cuda.synchronize()
    ms, wall = time_launches(step, a.steps, a.warmup, stream)
    tflops = w.flops() / (ms * 1e-3) / 1e12
    del q, k, v, o
    torch.cuda.empty_cache()
    print(f"[bench] headline {w.name}: {ms * 1e3:.1f} us per step over {a.steps} steps", file=sys.stderr, flush=True)

    traffic = traffic_bytes() if w.name == "mla_d192_d128_causal" else None
    roofline = {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                "traffic": None if traffic is None else int(traffic)}

    # ---- per-config blocks (single-dispatch statistics; the oracle on bounded samples)
    budgets = {"c1": (1.0, 0.5), "c2": (2.0, 1.0), "c3": (2.0, 1.0), "c4": (12.0, 4.0), "c5": (3.0, 2.0)}
    configs, extra = {}, {}
    if a.configs != "none":
        for cname, wname in CONFIGS:
            cw = workloads.WORKLOADS[wname]
            ob = None if a.no_cpu_baseline else budgets[cname]
            if cw.fp8:
                configs[cname] = bench_quantised(cw, dev, n, nw, ob)
            else:
                configs[cname] = bench_bf16(cw, dev, n, nw, ob, tiny=(cname == "c1"))
            print(f"[bench] {cname} {wname} done", file=sys.stderr, flush=True)
    if a.configs == "all":
        for name in EXTRA:
            if name.startswith("varlen:"):
                extra[name[7:]] = bench_varlen(dev, name[7:], max(50, n // 4), 10)
            else:
                ew = workloads.WORKLOADS[name]
                m = max(50, n // 4)
                extra[name] = bench_quantised(ew, dev, m, 10) if ew.fp8 else bench_bf16(ew, dev, m, 10)
            print(f"[bench] extra {name} done", file=sys.stderr, flush=True)

    cpu = None
    c4o = configs.get("c4", {}).get("oracle") if w.name == "mla_d192_d128_causal" else None
    if c4o is not None:
        cpu = {"value": c4o["tflops"], "unit": "TFLOP/s", "cores": c4o["threads"], "kind": "oracle",
               "sample": c4o["sample"] + f"; {c4o['seconds']} s", "seconds": c4o["seconds"],
               "value_1core": c4o["tflops_1core"], "sample_1core": c4o["sample_1core"] + f"; {c4o['seconds_1core']} s"}
    elif not a.no_cpu_baseline:
        o_ = oracle_timing(w, qc, kc, vc, 12.0, 4.0)
        cpu = {"value": o_["tflops"], "unit": "TFLOP/s", "cores": o_["threads"], "kind": "oracle",
               "sample": o_["sample"] + f"; {o_['seconds']} s", "seconds": o_["seconds"],
               "value_1core": o_["tflops_1core"], "sample_1core": o_["sample_1core"]}

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
        "configs": configs,
        "extra": extra,
        "peaks": {"bf16_tflops": PEAK_BF16_TFLOPS, "fp8_tflops": PEAK_FP8_TFLOPS},
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
