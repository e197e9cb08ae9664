#!/usr/bin/env python3
"""Decode benchmark of the OSCAR INT2 KV path on one MI355X.

One step = for every layer: append one token per sequence (rotate, clip,
INT2-quantize, pack, bf16 windows) then decode attention over the mixed cache
(q rotation, split-K INT2 flash-decode, bf16 window splits, LSE combine with
V un-rotation).  Default workload: Qwen3-8B-shaped attention, 36 layers,
batch 16, Hq 32, Hkv 8, head_dim 128, 32768 cached tokens per sequence, bf16
sink 64 + recent 256, group 128, clip K 0.96 / V 0.92.  Inputs are seeded
synthetic bf16 (N(0,1), 1% outlier channels x8) resident in HBM before timing.

Prints one JSON line (rank 0, one GPU).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "INT2-KV decode attention tokens/s + effective KV GB/s (% HBM peak) at 32k ctx"
HBM_PEAK_GBS = 8000.0

WORKLOADS = {
    # name: (layers, batch, Hq, Hkv, D, context, N, M, dist, outliers, v_dtype)
    "qwen3-8b-attn-32k": (36, 16, 32, 8, 128, 32768, 64, 256, "normal", "percent", 0),
    "qwen3-4b-attn-16k": (36, 1, 32, 8, 128, 16384, 512, 2048, "normal", "percent", 0),
    "qwen3-32b-attn-128k": (64, 8, 64, 8, 128, 131072, 64, 256, "student_t3", "none", 0),
    "wide-d512-attn-64k": (48, 4, 16, 8, 512, 65536, 512, 2048, "normal", "percent", 0),
    "wide-d512-attn-64k-vbf16": (48, 4, 16, 8, 512, 65536, 512, 2048, "normal", "percent", 1),
}


def prefill_summary(timings, B, Hkv, D):
    """The last fill chunk of every layer is a chunked-prefill append timed
    with HIP events: its rotation is a dense product (2 n B Hkv D^2 flops for K
    and the same for V) that runs on the matrix cores as three bf16 products
    (R held as three bf16 pieces)."""
    if not timings:
        return None
    n = timings[0][0]
    ms = sorted(t for _, t in timings)[len(timings) // 2]
    useful = 2 * 2 * n * B * Hkv * D * D / (ms / 1e3) / 1e12
    return {"tokens_per_chunk": n, "median_ms_per_layer": round(ms, 4), "layers": len(timings),
            "useful_TFLOPs": round(useful, 1), "mfma_TFLOPs": round(3 * useful, 1),
            "mfma_peak_TFLOPs": 2500.0, "mfma_util": round(3 * useful / 2500.0, 4),
            "kernel": "append_prefill_kernel"}


def measure_read_rate(torch, ok, nbytes, reps=5):
    """Best-of-reps rate of the library's read-only streaming kernel over a
    fresh nbytes buffer, timed with HIP events on the current stream."""
    src = torch.full((nbytes // 4,), 0x01020304, dtype=torch.int32, device="cuda")
    acc = torch.zeros(8192, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    ok.oscar_stream_read(src, nbytes, acc, stream)
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        ok.oscar_stream_read(src, nbytes, acc, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    del src
    torch.cuda.empty_cache()
    return {"GBps": round(nbytes / best / 1e6, 1), "bytes": nbytes, "best_ms": round(best, 4),
            "kernel": "stream_read_kernel", "reps": reps}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def fill_layer_device(cache, layer, B, Hkv, D, T, seed=0, dist="normal", outliers="percent", chunk=4096,
                      timings=None):
    """Append T synthetic tokens per sequence to `layer`, generated on the
    device.  With `timings` (a list), the last chunk's append is timed with HIP
    events and its (tokens, ms) appended."""
    import torch
    import synth
    mask = torch.from_numpy(synth.outlier_mask(D, Hkv, seed, layer, outliers)).cuda()
    t = 0
    ci = 0
    while t < T:
        n = min(chunk, T - t)
        k = synth.device_kv_fill((B, n, Hkv, D), synth.seed_of(seed, layer, "k", 1000 + ci), "cuda", mask, dist)
        v = synth.device_kv_fill((B, n, Hkv, D), synth.seed_of(seed, layer, "v", 1000 + ci), "cuda", mask, dist)
        last = t + n >= T
        if timings is not None and last:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            cache.append(layer, k, v)
            e1.record()
            torch.cuda.synchronize()
            timings.append((n, e0.elapsed_time(e1)))
        else:
            cache.append(layer, k, v)
        t += n
        ci += 1
    return mask


def prefill_attention_keys(T, n):
    """Keys the n queries of a chunk at the end of T cached positions attend to
    (query i at position T - n + i sees positions 0 .. T - n + i)."""
    return n * (T - n) + n * (n + 1) // 2


def time_prefill_attention(cache, B, Hq, Hkv, D, T, n, reps=3):
    """Chunked-prefill attention of the last n cached positions' queries
    (oscar_prefill_attn) on layer 0, timed with HIP events; median of reps.
    Useful flops: QK^T and PV over each query's causal prefix, 4 D per
    (query head, key); the matrix cores do twice that (q and p s_V each enter
    as two bf16 pieces).  head_dim 512 times at most 512 queries (a 4096-query
    chunk at 64k context is seconds of work)."""
    import torch
    if D == 512:
        n = min(n, 512)
    if D not in (128, 512) or n <= 0:
        return None
    g = torch.Generator(device="cuda")
    g.manual_seed(12345)
    q = torch.randn((B, n, Hq, D), generator=g, device="cuda").to(torch.bfloat16)
    out = torch.empty((B, n, Hq, D), dtype=torch.float32, device="cuda")
    ts = []
    for _ in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        cache.prefill_attn(0, q, out)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms = float(sorted(ts[1:])[len(ts[1:]) // 2])
    useful = 4.0 * D * B * Hq * prefill_attention_keys(T, n)
    return {"queries": n, "context": T, "median_ms": round(ms, 3),
            "useful_TFLOPs": round(useful / ms / 1e9, 1), "mfma_TFLOPs": round(2 * useful / ms / 1e9, 1),
            "mfma_peak_TFLOPs": 2500.0, "mfma_util": round(2 * useful / ms / 1e9 / 2500.0, 4),
            "kernel": "prefill_attn_kernel" if D == 128 else "prefill_attn_wide_kernel"}


def int2_bytes_per_token_head(D):
    return D // 4 + 4 * (D // 128)


def algorithmic_kv_bytes(B, Hkv, D, T, N, M, v_bf16):
    """Bytes one decode-attention call must read: INT2 K (+ INT2 or bf16 V) for
    the INT2 positions and bf16 K and V for the W = min(T, N+M) window tokens."""
    W = min(T, N + M)
    bk = int2_bytes_per_token_head(D)
    bv = 2 * D if v_bf16 else bk
    return B * Hkv * ((T - W) * (bk + bv) + W * 4 * D)


KERNEL_SOURCES = ("bit_attention_oscar_amd/csrc/decode.hip", "bit_attention_oscar_amd/csrc/append_impl.h",
                  "bit_attention_oscar_amd/csrc/common.h")


def kernel_sources_sha256() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def profiled_traffic(workload: str, kernel: str):
    """HBM bytes per launch of the dominant decode kernel from the committed
    rocprofv3 counter summary of this workload (FETCH_SIZE and WRITE_SIZE,
    each scaled by what the counter reads for the plain copy kernel), or None
    when there is none or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and line.startswith("- "):
                k, v = line[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel sources sha256") != kernel_sources_sha256():
        return None
    try:
        return int(fields["HBM bytes per launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(wl, budget_s=15.0):
    """The oracle, as it stands, on a bounded sample of the workload: one
    (layer, sequence) unit = append of one token + decode attention over the
    full context for all query heads of that sequence."""
    import oracle as orc
    import synth
    L, B, Hq, Hkv, D, T, N, M, dist, outl, vdt = wl
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = os.cpu_count() or 1
    cfg = orc.OracleConfig(num_layers=1, batch=1, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                           sink_tokens=N, recent_tokens=M, v_dtype=vdt)
    rk = synth.rotations(1, D, 0, "rot_k")
    rv = synth.rotations(1, D, 0, "rot_v")
    c = orc.OracleKVCache(cfg, rk, rv)
    mask = synth.outlier_mask(D, Hkv, 0, 0, outl)
    step = 4096
    t = 0
    while t < T:
        n = min(step, T - t)
        c.append(0, synth.kv_bits(1, n, Hkv, D, 0, 0, "k", mask, dist, 2000 + t),
                 synth.kv_bits(1, n, Hkv, D, 0, 0, "v", mask, dist, 2000 + t))
        t += n
    units = 0
    t0 = time.perf_counter()
    while True:
        kb = synth.kv_bits(1, 1, Hkv, D, 0, 0, "k", mask, dist, 9000 + units)
        vb = synth.kv_bits(1, 1, Hkv, D, 0, 0, "v", mask, dist, 9000 + units)
        c.append(0, kb, vb)
        q = synth.q_bits(1, Hq, Hkv, D, 0, 0, mask, dist, units)
        c.attend(0, q)
        units += 1
        el = time.perf_counter() - t0
        if el >= budget_s or units >= 64:
            break
    per_unit = el / units
    tok_s = 1.0 / (L * per_unit)          # B sequences x L layers units per B tokens
    cpu = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": tok_s, "unit": "tokens/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"{units} (layer, sequence) units of append(1 token) + decode attention at "
                      f"context {T}+, {el:.1f} s; tokens/s = 1/(layers x s per unit); cpu {cpu}; "
                      f"host cores {os.cpu_count()}"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen3-8b-attn-32k", choices=sorted(WORKLOADS))
    ap.add_argument("--splits", type=int, default=0, help="force INT2 splits (0 = auto)")
    ap.add_argument("--absorb-v", action="store_true",
                    help="V rotation absorbed into the caller's output projection: outputs stay in the "
                         "V-rotated basis (no un-rotation in the merge)")
    ap.add_argument("--separate", action="store_true",
                    help="append and attention as two calls per layer instead of the fused step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--read-calibration", action="store_true",
                    help="only measure the read-only streaming kernel and print its rate")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run the plain 16-byte copy kernel over MIB MiB ten times and print its "
                         "bandwidth (the reference for traffic counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this path runs on one GPU: the cache of one GPU's share is "
                                   "benchmarked at N=1; multi-GPU sharding is a design note, not built"}))
        sys.exit(2)

    import torch
    import synth
    from bit_attention_oscar_amd import oscar_kv as ok

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        ok.oscar_stream_copy(src, dst, n)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            ok.oscar_stream_copy(src, dst, n)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 10
        print(json.dumps({"copy_bytes": n, "avg_ms": ms, "read_plus_write_GBps": 2 * n / ms / 1e6,
                          "equal": bool(torch.equal(src, dst))}))
        return

    # achievable HBM read rate on this GPU: the read-only streaming kernel over
    # 4 GiB (well past the 256 MB last-level cache), best of five
    read_cal = measure_read_rate(torch, ok, 4 << 30)
    log(f"read-only streaming kernel: {read_cal['GBps']:.0f} GB/s")
    if args.read_calibration:
        print(json.dumps(read_cal))
        return

    wl = WORKLOADS[args.workload]
    L, B, Hq, Hkv, D, T0, N, M, dist, outl, vdt = wl
    W, K = args.warmup, args.steps
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    log(f"workload {args.workload}: L={L} B={B} Hq={Hq} Hkv={Hkv} D={D} T0={T0} N={N} M={M}")
    rk = synth.rotations(L, D, 0, "rot_k")
    rv = synth.rotations(L, D, 0, "rot_v")
    cap = T0 + W + 2 * K + 64
    cache = ok.KVCache(L, B, Hq, Hkv, D, cap, N, M, 128, 0.96, 0.92, ok.KV_INT2, vdt, rk, rv, 0,
                       1 if args.absorb_v else 0)
    if args.splits:
        cache.set_num_splits(args.splits)
    log(f"cache {cache.device_bytes() / 2**30:.2f} GiB; filling {T0} tokens x {L} layers")
    t_fill = time.perf_counter()
    masks = []
    prefill_t = []
    for l in range(L):
        masks.append(fill_layer_device(cache, l, B, Hkv, D, T0, seed=0, dist=dist, outliers=outl, timings=prefill_t))
    torch.cuda.synchronize()
    log(f"filled in {time.perf_counter() - t_fill:.1f} s")
    prefill_attn = time_prefill_attention(cache, B, Hq, Hkv, D, T0, min(4096, T0))
    if prefill_attn:
        log(f"prefill attention: {prefill_attn}")

    # per-step inputs, resident in HBM before timing
    steps_total = W + 2 * K
    g = torch.Generator(device=dev)
    g.manual_seed(synth.seed_of(0, 0, "step"))
    q_all = torch.randn((steps_total, L, B, Hq, D), generator=g, device=dev).to(torch.bfloat16)
    k_all = torch.randn((steps_total, L, B, 1, Hkv, D), generator=g, device=dev).to(torch.bfloat16)
    v_all = torch.randn((steps_total, L, B, 1, Hkv, D), generator=g, device=dev).to(torch.bfloat16)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        # one decode step of the whole model's attention: per layer, append the
        # new token's K/V and attend over the cache with the new q
        for l in range(L):
            if args.separate:
                cache.append(l, k_all[i, l], v_all[i, l], stream)
                cache.decode_attn(l, q_all[i, l], out, ok.OUT_F32, 0.0, stream)
            else:
                cache.decode_step(l, k_all[i, l], v_all[i, l], q_all[i, l], out, ok.OUT_F32, 0.0, stream)

    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    log("warmup done")

    # timed region: K steps, HIP events on the library's stream around them
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    e0.record(stream)
    for i in range(W, W + K):
        step(i)
    e1.record(stream)
    enqueue = time.perf_counter() - t_wall
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_total = e0.elapsed_time(e1)
    ms_per_step = ms_total / K
    tokens_s = B * K / (ms_total / 1e3)
    log(f"{K} steps: {ms_total:.2f} ms (wall {wall * 1e3:.1f} ms, host enqueue {enqueue * 1e3:.1f} ms), "
        f"{ms_per_step:.3f} ms/step")

    # the same K steps again (the cache keeps growing) with per-launch HIP
    # events that the library records on the stream it launches on: the
    # dominant kernel's average duration, live
    cache.profile_enable(True)
    torch.cuda.synchronize()
    for i in range(W + K, W + 2 * K):
        step(i)
    torch.cuda.synchronize()
    k_ms, k_n = cache.profile_read(0)
    call_ms, call_n = cache.profile_read(1)
    app_ms, app_n = cache.profile_read(2)
    cache.profile_enable(False)

    # bytes: every layer call of the profiled pass attends over
    # T = T0 + W + K + i + 1 tokens at its step i
    Ts = [T0 + W + K + i + 1 for i in range(K)]
    kv_bytes_calls = sum(algorithmic_kv_bytes(B, Hkv, D, T, N, M, vdt == 1) for T in Ts) * L
    # effective KV rate of the whole job: the timed pass's attention bytes
    # (steps W .. W + K - 1 attend over T0 + i + 1 tokens) over its wall time
    # on the GPU, appends included; the profiled pass's per-call events add a
    # launch gap per call and only give the per-call figure
    kv_bytes_timed = sum(algorithmic_kv_bytes(B, Hkv, D, T0 + i + 1, N, M, vdt == 1) for i in range(W, W + K)) * L
    kv_gbs = kv_bytes_timed / (ms_total / 1e3) / 1e9
    call_gbs = kv_bytes_calls / (call_ms / 1e3) / 1e9 if call_ms > 0 else None
    # dominant kernel: the decode attention launch (INT2 splits on matrix cores,
    # bf16 window blocks; at head_dim 128 also the last-block combine); it reads
    # every KV byte of the call.  Its duration comes from the HIP events the
    # library records around it on its launch stream (a q-record launch
    # before it, when there is one, and at head_dim 512 the merge launch after
    # it, are outside them and in the whole-job rate; a one-launch call at
    # head_dim 128 also rotates q and appends inside it)
    roof = None
    if k_n > 0:
        avg_ms = k_ms / k_n
        per_launch = kv_bytes_calls / k_n
        events_ms = avg_ms
        achieved = per_launch / (avg_ms / 1e3) / 1e9
        kname = "decode_wide" if D == 512 else "decode_mfma"
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": profiled_traffic(args.workload, kname),
                "kernel": kname + "_kernel",
                "avg_launch_us": round(avg_ms * 1e3, 3),
                "avg_launch_source": "per-launch HIP events",
                "avg_launch_us_events": round(events_ms * 1e3, 3),
                "algorithmic_bytes_per_launch": int(per_launch),
                "frac_of_measured_read": round(achieved / read_cal["GBps"], 4)}
    res = {
        "metric": METRIC,
        "value": round(tokens_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": args.workload, "layers": L, "batch": B, "q_heads": Hq, "kv_heads": Hkv,
                   "head_dim": D, "context": T0, "sink": N, "recent": M, "group": 128,
                   "k_clip": 0.96, "v_clip": 0.92, "v_cache": "bf16" if vdt else "int2",
                   "absorb_v_rotation": bool(args.absorb_v),
                   "parallelism": "none (1 GPU)"},
        "kv_gbps": round(kv_gbs, 1),
        "kv_hbm_frac": round(kv_gbs / HBM_PEAK_GBS, 4),
        "kv_gbps_per_call_events": None if call_gbs is None else round(call_gbs, 1),
        "step_mode": "separate" if args.separate else "fused",
        "attn_us_per_call": round(call_ms / max(call_n, 1) * 1e3, 3),
        "append_us_per_call": round(app_ms / max(app_n, 1) * 1e3, 3),
        "host_enqueue_ms_per_step": round(enqueue * 1e3 / K, 4),
        "hbm_read_measured": read_cal,
        "prefill": prefill_summary(prefill_t, B, Hkv, D),
        "prefill_attention": prefill_attn,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget)
    print(json.dumps(res), flush=True)
    cache.close()


if __name__ == "__main__":
    main()
