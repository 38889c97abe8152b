#!/usr/bin/env python3
"""Benchmark: attention forward TFLOPS at B=2, H=32, N=4096, d=128, causal, bf16.

One step is one forward pass (one kernel launch) over the whole batch, with
Q/K/V resident in device memory before the timed region. FLOPs are counted as
4*B*H*N^2*d, halved for the causal mask (only the lower triangle is work).
Prints ONE JSON line.

Timing follows the method of the AIInfra FlashAttention note (dpshk.com,
§3.2): warm-up launches first, device synchronisation on both sides of the
timed region, a HIP event pair around each kernel launch on the stream the
kernel runs on, median reported alongside the mean. `value` is the wall-clock
throughput of the timed region. A second pass runs the same number of launches
back to back with one event pair around all of them; its per-launch time is
reported too (on this power-limited GPU, back-to-back launches can run a few
percent slower or faster than launches separated by the event records).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
WORKLOAD = "causal_bf16_b2_h32_n4096_d128"
METRIC = "attention fwd TFLOPS (and % of bf16 MFMA peak) at B=2,H=32,N=4096,d=128 causal"


def fwd_flops(B, H, N, d, causal):
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


def cpu_baseline(x, w, budget_s: float):
    """Time the fp64 CPU oracle on a bounded sample of the same workload: whole
    (b, h) heads, one after another, until about ``budget_s`` seconds are spent."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    done = 0
    t0 = time.perf_counter()
    for b, h in heads:
        oracle.attn_ref_head(x["q"][b, h], x["k"][b, h], x["v"][b, h], w.scale, w.causal)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    flops = fwd_flops(1, 1, w.N, w.d, w.causal) * done
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), model)
    except OSError:
        pass
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"fp64 numpy oracle (three-pass softmax, S and P materialised) on {done} of "
                      f"{len(heads)} (b,h) heads of {WORKLOAD}; {el:.1f} s; host cpu_count="
                      f"{os.cpu_count()} ({model}), BLAS threads={threads}"}


def max_sclk_mhz():
    """Highest shader-clock level the driver lists (amdgpu sysfs), or None."""
    import glob
    import re
    best = None
    for path in glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"):
        try:
            with open(path) as f:
                for m in re.finditer(r"(\d+)\s*[Mm][Hh]z", f.read()):
                    best = max(best or 0, int(m.group(1)))
        except OSError:
            continue
    return best


def device_info(torch):
    """Name, architecture, compute-unit count and top clock level as the
    runtime and driver report them."""
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", ""),
            "compute_units": p.multi_processor_count,
            "hbm_gib": round(p.total_memory / 2**30, 1),
            "max_sclk_mhz": max_sclk_mhz()}


COPY_BYTES = 256 << 20
PROFILE = "profiles/fwd_bf16_causal_b2_h32_n4096_d128.md"
FWD_SOURCES = ["exact_attention_24_amd/csrc/attn_fwd.hip", "exact_attention_24_amd/csrc/attn_common.h",
               "exact_attention_24_amd/csrc/attn_tile.h", "exact_attention_24_amd/csrc/attn_sched.h"]


def profiled_traffic():
    """HBM-side bytes per launch from the committed counter summary, or None when
    the forward kernel's sources changed after the counters were taken."""
    import hashlib
    import pathlib
    root = pathlib.Path(__file__).resolve().parent
    try:
        text = (root / PROFILE).read_text()
        h = hashlib.sha256()
        for s in FWD_SOURCES:
            h.update((root / s).read_bytes())
    except OSError:
        return None
    fields = dict(line.split(": ", 1) for line in text.splitlines()
                  if line.startswith(("traffic_bytes_per_launch: ", "source_sha256_16: ")))
    if fields.get("source_sha256_16", "").strip() != h.hexdigest()[:16]:
        return None
    return int(fields["traffic_bytes_per_launch"])


def copy_calibration(torch, steps):
    """Copy a 256 MiB buffer `steps` times (reads and writes 256 MiB per launch)."""
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"mode": "copy", "bytes_read_per_launch": COPY_BYTES,
                      "bytes_written_per_launch": COPY_BYTES, "launches": steps}), flush=True)


def gemm_reference(torch, steps, warmup):
    """A plain bf16 library GEMM (torch.matmul, 8192 x 8192 x 8192) timed the same
    way as the forward, once on seeded random operands and once on zeros: the
    dense-MFMA rate a vendor kernel reaches on this GPU under the same power
    limit, as context for the attention kernel's fraction of the nominal peak."""
    n = 8192
    g = torch.Generator("cpu").manual_seed(1234)
    a = torch.randn(n, n, generator=g).to(torch.bfloat16).to("cuda:0")
    b = torch.randn(n, n, generator=g).to(torch.bfloat16).to("cuda:0")
    c = torch.empty(n, n, dtype=torch.bfloat16, device="cuda:0")
    for kind in ("random", "zeros"):
        if kind == "zeros":
            a.zero_()
            b.zero_()
        for _ in range(warmup):
            torch.matmul(a, b, out=c)
        torch.cuda.synchronize()
        times = []
        for _ in range(steps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            torch.matmul(a, b, out=c)
            e1.record()
            e1.synchronize()
            times.append(e0.elapsed_time(e1))
        med = statistics.median(times)
        print(json.dumps({"mode": "gemm", "op": "torch.matmul bf16", "M": n, "N": n, "K": n,
                          "values": kind, "ms_median": round(med, 4),
                          "tflops": round(2.0 * n ** 3 / med / 1e9, 1)}), flush=True)


BWD_WORKLOAD = "causal_fwdbwd_bf16_b2_h16_n8192_d128"


def bench_backward(torch, ea, steps, warmup=3):
    """Time the recompute backward (delta, dK/dV and dQ kernels) on the causal
    B=2 H=16 N=8192 d=128 workload, with O and LSE from one forward pass.
    FLOPs follow the 5-GEMM convention, 10*B*H*N^2*d halved for causal; the
    kernels execute 7 GEMMs' worth (S and dP are recomputed for dQ)."""
    from attn_inputs import WORKLOADS, make_workload_inputs
    w = WORKLOADS[BWD_WORKLOAD]
    x = make_workload_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "do"))
    o, lse = ea.attn_fwd(q, k, v, scale=w.scale, causal=w.causal)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(ea.attn_bwd_workspace_bytes(w.B, w.H, w.N, w.d), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        ea.attn_bwd(q, k, v, o, do, lse, scale=w.scale, causal=w.causal, dq=dq, dk=dk, dv=dv,
                    workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in ev)
    mean_ms = sum(per) / len(per)
    flops = 10.0 * w.B * w.H * w.N * w.N * w.d / 2
    executed = 14.0 * w.B * w.H * w.N * w.N * w.d / 2
    return {"workload": BWD_WORKLOAD, "ms_mean": round(mean_ms, 4), "ms_median": round(per[len(per) // 2], 4),
            "tflops": round(flops / (mean_ms * 1e-3) / 1e12, 2),
            "tflops_executed": round(executed / (mean_ms * 1e-3) / 1e12, 2),
            "frac_of_bf16_peak": round(flops / (mean_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "flop_convention": "10*B*H*N^2*d/2 (5 GEMMs, causal half); executed = 14*B*H*N^2*d/2"}


SUITE_WORKLOADS = ["mha_bf16_b4_h16_n2048_d64", "causal_bf16_b2_h32_n4096_d128",
                   "varlen_bf16_b8_h16_n2048_d128", "causal_fwdbwd_bf16_b2_h16_n8192_d128",
                   "gqa_causal_bf16_b2_h32_hkv8_n4096_d128", "causal_f16_b2_h32_n4096_d128"]
SWEEP_N = [2048, 4096, 8192, 16384]
FLUSH_BYTES = 512 << 20  # larger than the 256 MiB Infinity Cache


def time_launches(torch, fn, stream, warmup, steps):
    """Per-launch HIP-event times (ms), sorted, after `warmup` untimed launches."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) for a, b in ev)


def bench_suite(torch, ea, steps, warmup):
    """Forward timings of every workload and of a context sweep (B=2 H=32 d=128
    causal, N = 2K..16K). A 512 MiB buffer is written before each case so no
    case starts with its inputs in the Infinity Cache. One JSON line per case:
    median and P90 launch times and TFLOPS at the median."""
    from attn_inputs import WORKLOADS, make_workload_inputs, Workload
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    cases = [(WORKLOADS[n], None) for n in SUITE_WORKLOADS]
    cases += [(Workload(f"sweep_causal_bf16_b2_h32_n{n}_d128", 2, 32, n, 128, "bf16", True, 2000 + n), n)
              for n in SWEEP_N]
    for w, sweep_n in cases:
        if sweep_n is None:
            x = make_workload_inputs(w)
            q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
            seqlens = x["seqlens"].to(dev) if x.get("seqlens") is not None else None
            lens = x["seqlens"].tolist() if seqlens is not None else [w.N] * w.B
        else:  # timing only: seeded normal inputs drawn on the device
            g = torch.Generator(device=dev)
            g.manual_seed(w.seed)
            q, k, v = (torch.randn((w.B, w.H, w.N, w.d), generator=g, device=dev).to(torch.bfloat16)
                       for _ in range(3))
            seqlens, lens = None, [w.N] * w.B
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
        flops = sum(fwd_flops(1, w.H, L, w.d, w.causal) for L in lens)
        flush.fill_(1)
        per = time_launches(torch, lambda: ea.attn_fwd(q, k, v, scale=w.scale, causal=w.causal,
                                                       seqlens=seqlens, out=o, lse=lse),
                            stream, warmup, steps)
        med, p90 = per[len(per) // 2], per[int(0.9 * (len(per) - 1))]
        print(json.dumps({"mode": "suite", "workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                          "causal": w.causal, "varlen": seqlens is not None,
                          "gflop": round(flops / 1e9, 2), "ms_median": round(med, 4),
                          "ms_p90": round(p90, 4), "tflops_median": round(flops / (med * 1e-3) / 1e12, 1),
                          "pct_of_bf16_peak": round(100 * flops / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 1)}),
              flush=True)
        del q, k, v, o, lse


DECODE_WORKLOADS = ["decode_bf16_b8_h64_hkv8_nq1_nk8192_d128", "decode_bf16_b8_h64_hkv8_nq8_nk8192_d128",
                    "decode_fp8kv_bf16_b8_h64_hkv8_nq1_nk8192_d128"]


def bench_decode(torch, ea, name, steps, warmup):
    """Time one split-KV decode call (split kernel + merge) on a decode
    workload. Decode is bound by HBM bandwidth ("Attention 算子优化..." §五), so the roofline
    is bytes: K and V over every valid cached position once, Q read, O and LSE
    written, divided by the median call time, against 8 TB/s."""
    from attn_inputs import WORKLOADS, fp8_cache, make_workload_inputs
    w = WORKLOADS[name]
    x = make_workload_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    if w.kv_fp8:  # FP8 (E4M3) cache with per-token scales, built once before timing
        k8, ks = (t.to(dev) for t in fp8_cache(x["k"]))
        v8, vs = (t.to(dev) for t in fp8_cache(x["v"]))
    kl = x["seqlens"].to(dev) if x["seqlens"] is not None else None
    lens = x["seqlens"].tolist() if x["seqlens"] is not None else [w.N] * w.B
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    ws = torch.empty(ea.attn_decode_workspace_bytes(w.B, w.H, w.kv_heads, w.Nq, w.N, w.d),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    flush.fill_(1)
    if w.kv_fp8:
        fn = lambda: ea.attn_decode_fp8kv(q, k8, v8, ks, vs, scale=w.scale, causal=w.causal,
                                          kv_lens=kl, out=o, lse=lse, workspace=ws)
    else:
        fn = lambda: ea.attn_decode(q, k, v, scale=w.scale, causal=w.causal, kv_lens=kl, out=o,
                                    lse=lse, workspace=ws)
    per = time_launches(torch, fn, stream, warmup, steps)
    med = per[len(per) // 2]
    # K and V: 2 bytes per element, or 1 byte plus a 4-byte scale per token
    kv_bytes = sum(lens) * w.kv_heads * 2 * ((w.d + 4) if w.kv_fp8 else w.d * 2)
    io_bytes = w.B * w.H * w.Nq * (w.d * 2 * 2 + 4)
    gbs = (kv_bytes + io_bytes) / (med * 1e-3) / 1e9
    return {"workload": name, "ms_median": round(med, 4), "ms_p90": round(per[int(0.9 * (len(per) - 1))], 4),
            "algorithmic_bytes": kv_bytes + io_bytes, "achieved_GBps": round(gbs, 1),
            "peak_GBps": PEAK_HBM_GBS, "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "kv_format": "fp8 e4m3 + per-token fp32 scale" if w.kv_fp8 else w.dtype,
            "bytes_convention": "K,V over every valid cached position + Q read + O, LSE written"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle time for the CPU baseline (0 disables it)")
    ap.add_argument("--bwd-steps", type=int, default=10,
                    help="timed backward passes on the causal B=2 H=16 N=8192 d=128 workload "
                         "(reported under \"bwd\"; 0 skips them)")
    ap.add_argument("--mode", choices=["fwd", "bwd", "copy", "suite", "decode", "gemm"], default="fwd",
                    help="fwd: the benchmark; bwd: the backward alone; suite: forward timings "
                         "of every workload plus a context sweep (one JSON line each); decode: "
                         "the split-KV decode workloads against the HBM roofline; copy: a "
                         "plain device copy of known size, whose FETCH_SIZE/WRITE_SIZE counters "
                         "calibrate the traffic figure; gemm: a library bf16 GEMM on random "
                         "and on zero operands, the dense-MFMA rate reachable under this "
                         "GPU's power limit (context only)")
    ap.add_argument("--values", choices=["random", "zeros"], default="random",
                    help="fwd mode only: 'zeros' runs the same launches on all-zero Q, K, V, "
                         "a diagnostic of data-dependent power (the clock the chip holds under "
                         "MFMA load depends on operand bit activity); never the benchmark line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.mode == "copy":
        copy_calibration(torch, args.steps)
        return
    if args.mode == "gemm":
        gemm_reference(torch, args.steps, args.warmup)
        return
    import exact_attention_24_amd as ea
    if args.mode == "bwd":
        print(json.dumps({"mode": "bwd", **bench_backward(torch, ea, args.steps, args.warmup)}), flush=True)
        return
    if args.mode == "suite":
        bench_suite(torch, ea, args.steps, args.warmup)
        return
    if args.mode == "decode":
        for name in DECODE_WORKLOADS:
            print(json.dumps({"mode": "decode", **bench_decode(torch, ea, name, args.steps, args.warmup)}),
                  flush=True)
        return
    from attn_inputs import WORKLOADS, make_workload_inputs

    w = WORKLOADS[WORKLOAD]
    x = make_workload_inputs(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    if args.values == "zeros":
        q, k, v = (torch.zeros_like(t) for t in (q, k, v))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        ea.attn_fwd(q, k, v, scale=w.scale, causal=w.causal, out=o, lse=lse)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = sorted(a.elapsed_time(b) for a, b in zip(starts, ends))  # ms per launch
    mean_ms = sum(per) / len(per)
    median_ms = per[len(per) // 2]
    ms_per_step = wall * 1e3 / args.steps
    # Second pass: the same launches back to back, one event pair around all.
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    b2b_ms = e0.elapsed_time(e1) / args.steps
    flops = fwd_flops(w.B, w.H, w.N, w.d, w.causal)
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (mean_ms * 1e-3) / 1e12

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal, "global_batch": w.B, "seq_len": w.N, "parallelism": "none"},
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "device": device_info(torch),
        "kernel_ms": {"mean": round(mean_ms, 4), "median": round(median_ms, 4),
                      "p90": round(per[int(0.9 * (len(per) - 1))], 4),
                      "back_to_back_per_launch": round(b2b_ms, 4)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": profiled_traffic(),
                     "kernel": "fwd_16_kernel<128, causal, bf16>",
                     "algorithmic": "4*B*H*N^2*d/2 FLOP per launch"},
    }
    if args.values == "zeros":
        out["data"] = "synthetic, all-zero Q/K/V (power diagnostic, not the benchmark)"
        out["roofline"]["traffic"] = None
        print(json.dumps(out), flush=True)
        return
    if args.bwd_steps > 0:
        out["bwd"] = bench_backward(torch, ea, args.bwd_steps)
        out["decode"] = bench_decode(torch, ea, DECODE_WORKLOADS[0], 20, 5)
    if args.cpu_budget > 0:
        out["cpu_baseline"] = cpu_baseline(x, w, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
