#!/usr/bin/env python3
"""Decode throughput of the compressed-KV library on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one decode step of the whole hot path on one batch: append the new
token's K/V to every layer's cache (kv_append) and attend over it (decode_attn).
Inputs are synthetic (seeded, synth/), already resident in HBM when the timed
region starts.  Prints ONE JSON line with steps/s, achieved HBM bandwidth of the
decode kernel (HIP events around every decode_attn launch, on the launch stream)
against the 8 TB/s peak, and the fp64 CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12  # B/s, MI355X HBM3E
METRIC = "decode steps/s + achieved HBM TB/s (% of peak); SnapKV compress ms"


def _parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default: per workload)")
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="llama2_7b_layer",
                    choices=["llama2_7b_layer", "gqa_long", "tiny_streaming"])
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="bound of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-snapkv", action="store_true", help="skip the SnapKV compression timing")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 1 GiB device copy (reference for HBM byte counters)")
    return ap.parse_args(argv)


def _copy_calibration():
    """A plain device-to-device copy of 1 GiB, three times (known bytes: 1 GiB read and
    1 GiB written per launch) so that profiler byte counters can be scaled."""
    import torch

    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def _streaming_bench(L, w, steps, warmup):
    import torch

    dev = "cuda"
    cfg = L.cache_config(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim,
                         L.LCD_F32 if w.dtype == "f32" else L.LCD_BF16, L.LCD_SINK_RING, n_layers=w.n_layers,
                         n_sink=w.n_sink, window=w.window, rope=1, rope_base=w.rope_base)
    cache = L.KVCache(cfg, device=dev)
    for layer in range(w.n_layers):
        if w.prefill:
            k = w.token_block_torch("k", layer, 0, w.prefill, dev)
            v = w.token_block_torch("v", layer, 0, w.prefill, dev)
            cache.append(layer, k, v)
            del k, v
    n_tok = warmup + steps
    t0 = w.prefill
    q = [w.token_major_torch("q", l, t0, t0 + n_tok, dev) for l in range(w.n_layers)]
    k = [w.token_major_torch("k", l, t0, t0 + n_tok, dev) for l in range(w.n_layers)]
    v = [w.token_major_torch("v", l, t0, t0 + n_tok, dev) for l in range(w.n_layers)]
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step(i, ev=None):
        for l in range(w.n_layers):
            cache.append(l, k[l][i].unsqueeze(2), v[l][i].unsqueeze(2))
            if ev is not None:
                ev[0][l].record()
            cache.decode(l, q[l][i], out)
            if ev is not None:
                ev[1][l].record()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # timed region 1: the steps alone
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(warmup, warmup + steps):
        step(i)
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    # timed region 2: the same number of steps again (continuing the stream), with an
    # event pair around every decode_attn launch for the kernel's own duration
    ev_steps = min(steps, 512)
    evs = [([torch.cuda.Event(enable_timing=True) for _ in range(w.n_layers)],
            [torch.cuda.Event(enable_timing=True) for _ in range(w.n_layers)]) for _ in range(ev_steps)]
    kq = [w.token_major_torch("q", l, t0 + n_tok, t0 + n_tok + ev_steps, dev) for l in range(w.n_layers)]
    kk = [w.token_major_torch("k", l, t0 + n_tok, t0 + n_tok + ev_steps, dev) for l in range(w.n_layers)]
    kv_ = [w.token_major_torch("v", l, t0 + n_tok, t0 + n_tok + ev_steps, dev) for l in range(w.n_layers)]
    torch.cuda.synchronize()
    for i in range(ev_steps):
        for l in range(w.n_layers):
            cache.append(l, kk[l][i].unsqueeze(2), kv_[l][i].unsqueeze(2))
            evs[i][0][l].record()
            cache.decode(l, kq[l][i], out)
            evs[i][1][l].record()
    torch.cuda.synchronize()
    kern_ms = [evs[i][0][l].elapsed_time(evs[i][1][l]) for i in range(ev_steps) for l in range(w.n_layers)]
    kern_ms.sort()
    avg_kernel_ms = sum(kern_ms) / len(kern_ms)
    C = w.n_sink + w.window
    kv_bytes = 2 * w.batch * w.n_kv_heads * C * w.head_dim * w.esize  # one layer, full cache
    io_bytes = w.batch * w.n_q_heads * w.head_dim * (w.esize + 4)     # q in, fp32 out
    launch_bytes = kv_bytes + io_bytes
    step_bytes = w.n_layers * (launch_bytes + 2 * w.batch * w.n_kv_heads * w.head_dim * w.esize)
    res = dict(
        steps_per_s=steps / (total_ms / 1e3),
        ms_per_step=total_ms / steps,
        avg_kernel_ms=avg_kernel_ms,
        median_kernel_ms=kern_ms[len(kern_ms) // 2],
        launch_bytes=launch_bytes,
        step_bytes=step_bytes,
        kernel_launches=len(kern_ms),
    )
    cache.close()
    return res


def _snapkv_bench(L, w, reps=20):
    """SnapKV compression of the 32k prompt: ms per compress (median of ``reps``)."""
    import torch

    B, H, D, N, Lo, K = w.batch, w.n_q_heads, w.head_dim, w.n_prompt, w.l_obs, w.k_keep
    dev = "cuda"
    p = L.snapkv_params(B, H, D, N, Lo, w.kernel_size, K)
    wsb = L.snapkv_sizes(p)
    q = w.snapkv_tensor_torch("q_obs", dev)
    k = w.snapkv_tensor_torch("k", dev)
    v = w.snapkv_tensor_torch("v", dev)
    ko = torch.empty((B, H, K + Lo, D), dtype=torch.bfloat16, device=dev)
    vo = torch.empty_like(ko)
    idx = torch.empty((B, H, K + Lo), dtype=torch.int32, device=dev)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    for _ in range(3):
        L.snapkv_compress(p, q, k, v, ko, vo, idx, None, ws, wsb)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        L.snapkv_compress(p, q, k, v, ko, vo, idx, None, ws, wsb)
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    times.sort()
    ms = times[len(times) // 2]
    # algorithmic: K read once, the kept K/V rows read and written, q, indices
    kbytes = B * H * N * D * 2
    gather = 2 * 2 * B * H * (K + Lo) * D * 2
    alg_bytes = kbytes + gather + B * H * Lo * D * 2 + B * H * (K + Lo) * 4
    flops = 2 * B * H * Lo * N * D  # one observation-window Q K^T
    return {"workload": w.title, "compress_ms": round(ms, 4), "reps": reps,
            "algorithmic_bytes": alg_bytes, "hbm_gb_s": round(alg_bytes / (ms / 1e3) / 1e9, 1),
            "hbm_frac": round(alg_bytes / (ms / 1e3) / HBM_PEAK, 4),
            "qk_tflops": round(flops / (ms / 1e3) / 1e12, 2),
            "mfma_frac_bf16": round(flops / (ms / 1e3) / 2.5e15, 5)}


def _cpu_baseline_streaming(w, budget_s):
    """The fp64 oracle on a bounded sample of one decode step (single thread)."""
    import numpy as np

    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    import oracle

    t = w.prefill + 7  # a decode step after the ring has wrapped
    toks = oracle.retained_tokens(t, w.n_sink, w.window)
    G = w.group
    heads_per_step = w.batch * w.n_kv_heads * w.n_layers
    done, elapsed = 0, 0.0
    limiter = threadpool_limits(1) if threadpool_limits else None
    try:
        for layer in range(w.n_layers):
            for b in range(w.batch):
                for g in range(w.n_kv_heads):
                    kk = w.token_block("k", layer, toks, batches=[b], heads=[g])[0]
                    vv = w.token_block("v", layer, toks, batches=[b], heads=[g])[0]
                    qq = w.token_block("q", layer, [t], batches=[b], heads=np.arange(g * G, g * G + G))[0, :, 0, :]
                    t1 = time.perf_counter()
                    oracle.streaming_decode(qq, lambda _t, kk=kk, vv=vv: (kk, vv), t, w.n_sink, w.window,
                                            w.rope_base)
                    elapsed += time.perf_counter() - t1
                    done += 1
                    if elapsed >= budget_s:
                        break
                if elapsed >= budget_s:
                    break
            if elapsed >= budget_s:
                break
    finally:
        if limiter is not None:
            limiter.restore_original_limits()
    steps_per_s = (done / heads_per_step) / elapsed
    return {"value": steps_per_s, "unit": "decode steps/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} of the {heads_per_step} (layer, batch row, KV head) slices of decode step t={t} "
                      f"({elapsed:.1f} s of fp64 numpy on one thread; input generation excluded)"}


def main(argv=None):
    a = _parse(argv)
    if a.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus_requested": a.gpus}))
        return 2
    import torch

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        return 2
    import long_context_decode_amd as L
    from synth import WORKLOADS

    if a.copy_calibration:
        _copy_calibration()
    w = WORKLOADS[a.workload]
    defaults = {"llama2_7b_layer": (8192, 64), "gqa_long": (128, 4), "tiny_streaming": (448, 64)}
    steps, warmup = defaults[a.workload]
    steps = a.steps if a.steps is not None else steps
    warmup = a.warmup if a.warmup is not None else warmup
    if a.workload == "tiny_streaming":
        warmup = min(warmup, w.steps)
    r = _streaming_bench(L, w, steps, warmup)
    achieved = r["launch_bytes"] / (r["avg_kernel_ms"] / 1e3)
    line = {
        "metric": METRIC,
        "value": round(r["steps_per_s"], 2),
        "unit": "decode steps/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.title, "batch": w.batch, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "n_layers": w.n_layers, "cache_slots": w.n_sink + w.window,
                   "n_sink": w.n_sink, "window": w.window},
        "hbm_tb_s": round(r["step_bytes"] * r["steps_per_s"] / 1e12, 3),
        "hbm_frac_of_peak": round(r["step_bytes"] * r["steps_per_s"] / HBM_PEAK, 4),
        "roofline": {"bound": "hbm", "kernel": "decode_split_kernel (lcd_decode_attn)",
                     "achieved": round(achieved / 1e9, 1), "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK, 4), "traffic": None,
                     "bytes_per_launch": r["launch_bytes"], "avg_launch_us": round(r["avg_kernel_ms"] * 1e3, 2),
                     "median_launch_us": round(r["median_kernel_ms"] * 1e3, 2),
                     "launches_timed": r["kernel_launches"]},
    }
    if not a.no_snapkv:
        line["snapkv"] = _snapkv_bench(L, WORKLOADS["snapkv_32k"])
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = _cpu_baseline_streaming(w, a.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
