#!/usr/bin/env python3
"""Decode throughput of the compressed-KV library on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--only]

A step is one decode step of the whole hot path on one batch: for every layer, the new
token's K/V appended and its query attended over the cache (one fused lcd_decode_step
launch per layer for the sink + ring caches; kv_append then decode_attn otherwise).
Inputs are synthetic (seeded, synth/) and already resident in HBM when the timed region
starts.  Prints ONE JSON line: the headline workload (the 16-layer GQA long cache: 24 / 4
heads, D = 256, 4 sinks + 32764 ring, B = 16) with steps/s, the decode kernel's achieved
HBM bandwidth against the 8 TB/s peak (HIP events on the launch stream around batches of
back-to-back launches) and its counter-measured HBM traffic when the record under
profiles/ matches the current kernel sources; the SnapKV compression time and the H2O
prompt-phase compression time and MFMA rate; the secondary decode workloads (the
Llama-2-7B-shaped layer, the Llama-3-shaped layer, the H2O 4096 budget with token- and
block-level eviction, the DuoAttention 128k mixed-head layer, the tiny fp32 stream)
unless --only; and the fp64 CPU oracle timed on all affinity cores (one process per core,
forked before any GPU work) on bounded samples of the headline step, the SnapKV
compression and the H2O budgeted decode step.
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
MFMA_BF16_PEAK = 2.5e15  # flop/s, dense
METRIC = "decode steps/s + achieved HBM TB/s (% of peak); SnapKV compress ms"
DEFAULTS = {"llama2_7b_layer": (8192, 64), "llama3_8b_layer": (1024, 32), "gqa_long": (64, 8), "h2o_128k": (1024, 32),
            "h2o_blocks_128k": (1024, 32), "duo_128k": (192, 16), "tiny_streaming": (448, 64)}
HEADLINE = "gqa_long"


def _parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps of the headline workload")
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(DEFAULTS) + ["snapkv_32k"],
                    help="decode workload to time (snapkv_32k: only with --counters)")
    ap.add_argument("--only", action="store_true", help="skip the secondary workloads and SnapKV")
    ap.add_argument("--no-snapkv", action="store_true", help="skip the SnapKV compression timing")
    ap.add_argument("--no-h2o-prompt", action="store_true", help="skip the H2O prompt-phase compression timing")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="bound of each oracle sample (oracle seconds per worker process)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--snapkv-only", action="store_true",
                    help="time the SnapKV compression alone and print its record (for profiling)")
    ap.add_argument("--l-obs", type=int, default=None,
                    help="with --snapkv-only: observation window of the 32k compression (default 32)")
    ap.add_argument("--mfma-counters", nargs="+", metavar="LOBS=CSV",
                    help="summarise rocprofv3 --pmc runs of 'bench.py --snapkv-only --l-obs LOBS' (MFMA and "
                         "activity counters, one CSV per observation window) into the SnapKV MFMA record "
                         "and exit (no GPU)")
    ap.add_argument("--counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of 'bench.py --only "
                         "--copy-calibration --workload NAME' into the traffic record of NAME and exit (no GPU)")
    return ap.parse_args(argv)


# HBM traffic of a decode kernel, from profiler counters.  A record is tied to the sources
# that decide the kernel's memory behaviour (the kernel and its launch plan); when any of
# them changes the record is stale and the bench reports traffic as null.
# workload -> (kernel instantiation as rocprofv3 names it, record file)
TRAFFIC = {
    "gqa_long": ("decode_twopass_kernel<lcd::bf16_t, 256, 6, 0>",
                 "decode_twopass_kernel_gqa32k_b16_traffic.md"),
    "llama2_7b_layer": ("decode_onepass_kernel<lcd::bf16_t, 128, 1, 0>",
                        "decode_onepass_kernel_llama2_b16_c2048_traffic.md"),
    "llama3_8b_layer": ("decode_twopass_kernel<lcd::bf16_t, 128, 4, 0>",
                        "decode_twopass_kernel_llama3_b16_c8192_traffic.md"),
    "h2o_128k": ("decode_twopass_kernel<lcd::bf16_t, 128, 4, 2>", "decode_twopass_kernel_h2o4096_b16_traffic.md"),
    "h2o_blocks_128k": ("decode_twopass_kernel<lcd::bf16_t, 128, 4, 3>",
                        "decode_twopass_kernel_h2o4096_blocks16_b16_traffic.md"),
    "duo_128k": ("decode_twopass_kernel<lcd::bf16_t, 128, 4, 1>", "decode_twopass_kernel_duo128k_b16_traffic.md"),
}
TRAFFIC_SOURCES = ("long_context_decode_amd/csrc/decode.hip", "long_context_decode_amd/csrc/lcd_internal.h",
                   "long_context_decode_amd/csrc/lcd_host.cpp")
COPY_BYTES = 1 << 30  # the calibration copy
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_FILTER = "decode_|copyBuffer"  # counters on the decode kernels and the calibration copies only


def _counter_run(workload):
    return (f"python3 bench.py --only --workload {workload} --copy-calibration --steps 16 --warmup 4 "
            "--no-cpu-baseline")


def _sources_digest():
    import hashlib

    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()


def _read_counter_csv(path, counter):
    """{dispatch id: (kernel name, grid size, value in KiB)} for one counter."""
    import csv

    out = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            d = int(row["Dispatch_Id"])
            name, grid, val = row["Kernel_Name"], int(row["Grid_Size"]), float(row["Counter_Value"])
            if d in out:  # one row per counter instance: sum them
                val += out[d][2]
            out[d] = (name, grid, val)
    return out


def _counter_summary(fetch_csv, write_csv, workload):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE of the workload's decode kernel, each scaled by
    what the counter reads for the 1 GiB calibration copy; writes the traffic record."""
    import statistics

    kernel, fname = TRAFFIC[workload]
    out = os.path.join(PROFILES, fname)
    res = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _read_counter_csv(path, counter)
        # the calibration copies are the process's first three device copies
        copies = [rows[d][2] for d in sorted(rows) if "copyBuffer" in rows[d][0]][:3]
        if len(copies) < 3 or max(copies) > 1.05 * min(copies):
            raise SystemExit(f"{path}: no consistent calibration copy (run the bench with --copy-calibration)")
        copy_kib = statistics.median(copies)
        dec = [v for (n, g, v) in rows.values() if kernel in n]
        if not dec:
            raise SystemExit(f"{path}: no {kernel} dispatch")
        res[counter] = dict(copy_kib=copy_kib, scale=COPY_BYTES / (copy_kib * 1024.0),
                            decode_kib=statistics.mean(dec), dispatches=len(dec))
    f, w = res["FETCH_SIZE"], res["WRITE_SIZE"]
    traffic = f["decode_kib"] * 1024.0 * f["scale"] + w["decode_kib"] * 1024.0 * w["scale"]
    from synth import WORKLOADS

    wl = WORKLOADS[workload]
    lines = [
        f"# `{kernel}` HBM traffic — {wl.title}",
        "",
        "Two rocprofv3 counter runs of the same command, one counter each, counters collected on the "
        "decode kernels and the calibration copies only:",
        "",
        "```",
        "cd /tmp && export TMPDIR=/tmp && cd $REPO",
        f"rocprofv3 --pmc FETCH_SIZE --kernel-include-regex '{KERNEL_FILTER}' --output-format csv "
        f"-d {os.path.dirname(fetch_csv)} -o run -- {_counter_run(workload)}",
        f"rocprofv3 --pmc WRITE_SIZE --kernel-include-regex '{KERNEL_FILTER}' --output-format csv "
        f"-d {os.path.dirname(write_csv)} -o run -- {_counter_run(workload)}",
        f"python3 bench.py --counters {fetch_csv} {write_csv} --workload {workload}",
        "```",
        "",
        "The calibration copy moves 1 GiB in each direction; each counter is scaled by "
        "1 GiB / (its reading for that copy).",
        "",
        "| counter | copy reads (KiB) | scale | decode kernel, mean per dispatch (KiB) | dispatches | scaled bytes |",
        "|---|---|---|---|---|---|",
    ]
    for name, r in (("FETCH_SIZE", f), ("WRITE_SIZE", w)):
        lines.append(f"| {name} | {r['copy_kib']:.1f} | {r['scale']:.4f} | {r['decode_kib']:.1f} | "
                     f"{r['dispatches']} | {r['decode_kib'] * 1024 * r['scale']:.0f} |")
    lines += ["", f"traffic-bytes-per-launch: {traffic:.0f}", f"sources-sha256: {_sources_digest()}",
              f"sources: {', '.join(TRAFFIC_SOURCES)}", ""]
    with open(out, "w") as fh:
        fh.write("\n".join(lines))
    print(f"traffic {traffic:.0f} B per launch -> {out}")
    return traffic


SNAPKV_FILTER = "snapkv_|copyBuffer"
MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE")
N_SIMD = 1024  # 256 CUs x 4 SIMDs
N_XCD = 8


def _snapkv_alg_bytes(w):
    B, H, D, N, Lo, K = w.batch, w.n_q_heads, w.head_dim, w.n_prompt, w.l_obs, w.k_keep
    return B * H * N * D * 2 + 2 * 2 * B * H * (K + Lo) * D * 2 + B * H * Lo * D * 2 + B * H * (K + Lo) * 4


def _snapkv_counter_summary(fetch_csv, write_csv):
    """FETCH_SIZE / WRITE_SIZE of the SnapKV kernels (mean per dispatch of each, summed over
    one compress), scaled by the calibration copy; writes the SnapKV traffic record."""
    import statistics
    from synth import WORKLOADS

    w = WORKLOADS["snapkv_32k"]
    per = {}
    scale = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _read_counter_csv(path, counter)
        copies = [rows[d][2] for d in sorted(rows) if "copyBuffer" in rows[d][0]][:3]
        if len(copies) < 3 or max(copies) > 1.05 * min(copies):
            raise SystemExit(f"{path}: no consistent calibration copy (run the bench with --copy-calibration)")
        scale[counter] = COPY_BYTES / (statistics.median(copies) * 1024.0)
        kern = {}
        for (n, g, v) in rows.values():
            if "snapkv_" in n:
                kern.setdefault(n, []).append(v)
        for n, vals in kern.items():
            per.setdefault(n, {})[counter] = (statistics.mean(vals) * 1024.0 * scale[counter], len(vals))
    total = sum(c.get("FETCH_SIZE", (0, 0))[0] + c.get("WRITE_SIZE", (0, 0))[0] for c in per.values())
    alg = _snapkv_alg_bytes(w)
    run = "python3 bench.py --snapkv-only --copy-calibration"
    lines = [f"# SnapKV compression kernels, HBM traffic — {w.title}", "",
             "Two rocprofv3 counter runs of the same command, one counter each, counters collected on the "
             "SnapKV kernels and the calibration copies only:", "", "```",
             "cd /tmp && export TMPDIR=/tmp && cd $REPO",
             f"rocprofv3 --pmc FETCH_SIZE --kernel-include-regex '{SNAPKV_FILTER}' --output-format csv "
             f"-d {os.path.dirname(fetch_csv)} -o run -- {run}",
             f"rocprofv3 --pmc WRITE_SIZE --kernel-include-regex '{SNAPKV_FILTER}' --output-format csv "
             f"-d {os.path.dirname(write_csv)} -o run -- {run}",
             f"python3 bench.py --counters {fetch_csv} {write_csv} --workload snapkv_32k", "```", "",
             f"Scales from the 1 GiB calibration copy: FETCH_SIZE x{scale['FETCH_SIZE']:.4f}, "
             f"WRITE_SIZE x{scale['WRITE_SIZE']:.4f}.", "",
             "| kernel | dispatches | read bytes (mean per dispatch) | written bytes (mean per dispatch) |",
             "|---|---:|---:|---:|"]
    for n in sorted(per, key=lambda n: -per[n].get("FETCH_SIZE", (0, 0))[0]):
        f_, w_ = per[n].get("FETCH_SIZE", (0, 0)), per[n].get("WRITE_SIZE", (0, 0))
        lines.append(f"| `{n}` | {f_[1]} | {f_[0]:.0f} | {w_[0]:.0f} |")
    lines += ["", f"Per compress (one dispatch of each kernel): {total:.0f} B against {alg} algorithmic bytes "
              f"(K read once, the kept K / V rows read and written, q and indices): {total / alg:.3f}x.",
              f"traffic-bytes-per-compress: {total:.0f}", ""]
    out = os.path.join(PROFILES, "snapkv_kernels_32k_traffic.md")
    with open(out, "w") as fh:
        fh.write("\n".join(lines))
    print(f"traffic {total:.0f} B per compress ({total / alg:.3f}x) -> {out}")
    return total


def _mfma_summary(entries):
    """MFMA counters of the two SnapKV scoring kernels over observation windows: per pass,
    flops (MOPS_BF16 x 512), the MFMA pipes' busy fraction (busy cycles over every SIMD's
    cycles) and the ceiling min(1, L_obs / 312) that K's bytes impose at 8 TB/s."""
    import csv
    import statistics

    lines = ["# SnapKV scoring kernels — MFMA counters over the observation window", "",
             "One rocprofv3 counter run per observation window L_obs (32-key prompt N=32768, 32 heads, "
             "D=128, bf16), counters on the SnapKV kernels only:", "", "```",
             "cd /tmp && export TMPDIR=/tmp && cd $REPO"]
    table = []
    for e in entries:
        lo, path = e.split("=", 1)
        lo = int(lo)
        lines.append(f"rocprofv3 --pmc {' '.join(MFMA_COUNTERS)} --kernel-include-regex 'snapkv_' "
                     f"--output-format csv -d {os.path.dirname(path)} -o run -- "
                     f"python3 bench.py --snapkv-only --l-obs {lo}")
        vals = {}
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                n = row["Kernel_Name"]
                kind = "rowstats" if "rowstats" in n else "colscore" if "colscore" in n else None
                if kind is None:
                    continue
                key = (kind, int(row["Dispatch_Id"]))
                vals.setdefault(key, {}).setdefault(row["Counter_Name"], 0.0)
                vals[key][row["Counter_Name"]] += float(row["Counter_Value"])
        for kind in ("rowstats", "colscore"):
            ds = [v for (k, _), v in vals.items() if k == kind and all(c in v for c in MFMA_COUNTERS)]
            if not ds:
                raise SystemExit(f"{path}: no complete {kind} dispatch")
            mops = statistics.mean(d["SQ_INSTS_VALU_MFMA_MOPS_BF16"] for d in ds)
            busy = statistics.mean(d["SQ_VALU_MFMA_BUSY_CYCLES"] for d in ds)
            gui = statistics.mean(d["GRBM_GUI_ACTIVE"] for d in ds)
            frac = busy / (N_SIMD * gui / N_XCD)
            table.append((lo, kind, len(ds), mops * 512, gui / N_XCD, frac, min(1.0, lo / 312.0)))
    lines += [f"python3 bench.py --mfma-counters {' '.join(entries)}", "```", "",
              "| L_obs | pass | dispatches | flops per dispatch | cycles (per XCD) | MFMA busy | ceiling min(1, L_obs/312) | busy / ceiling |",
              "|---:|---|---:|---:|---:|---:|---:|---:|"]
    for lo, kind, n, fl, cyc, frac, ceil in table:
        lines.append(f"| {lo} | {kind} | {n} | {fl:.4g} | {cyc:.0f} | {frac:.4f} | {ceil:.3f} | {frac / ceil:.3f} |")
    lines += ["", "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8 XCDs); a "
              "32x32x16 bf16 MFMA keeps its pipe busy 32 cycles for 32768 flops, so a busy fraction f "
              "is f x 2.5 PFLOP/s.  The ceiling: each pass reads K once, L_obs flop per byte, so at 8 TB/s "
              "it can use at most 8 L_obs TFLOP/s of the 2500.", ""]
    out = os.path.join(PROFILES, "snapkv_mfma_lobs_sweep.md")
    with open(out, "w") as fh:
        fh.write("\n".join(lines))
    print(f"-> {out}")


def _traffic(workload):
    """Scaled counter bytes per launch of the workload's decode kernel, or None when no
    record exists or the record was taken on other sources."""
    if workload not in TRAFFIC:
        return None
    try:
        with open(os.path.join(PROFILES, TRAFFIC[workload][1])) as f:
            kv = dict(line.split(": ", 1) for line in f.read().splitlines() if ": " in line and
                      line.split(": ", 1)[0] in ("traffic-bytes-per-launch", "sources-sha256"))
    except OSError:
        return None
    if kv.get("sources-sha256", "").strip() != _sources_digest():
        return None
    return int(float(kv["traffic-bytes-per-launch"]))


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


class _Stepper:
    """Owns a cache, its staged per-step inputs and the step function."""

    def __init__(self, L, w, n_tokens, dev="cuda"):
        import torch

        self.L, self.w, self.dev = L, w, dev
        dt = L.LCD_F32 if w.dtype == "f32" else L.LCD_BF16
        if w.kind == "streaming":
            cfg = L.cache_config(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, dt, L.LCD_SINK_RING,
                                 n_layers=w.n_layers, n_sink=w.n_sink, window=w.window, rope=1,
                                 rope_base=w.rope_base)
            self.cache = L.KVCache(cfg, device=dev)
            for layer in range(w.n_layers):
                if w.prefill:
                    k = w.token_block_torch("k", layer, 0, w.prefill, dev)
                    v = w.token_block_torch("v", layer, 0, w.prefill, dev)
                    self.cache.append(layer, k, v)
                    del k, v
            self.t0 = w.prefill
            self.slots = w.n_sink + w.window
        elif w.kind == "duo":
            cfg = L.cache_config(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, dt, L.LCD_DUO,
                                 n_layers=w.n_layers, n_sink=w.n_sink, window=w.window, capacity=w.capacity,
                                 retrieval=w.retrieval)
            self.cache = L.KVCache(cfg, device=dev)
            for layer in range(w.n_layers):
                for a in range(0, w.prefill, 8192):
                    e = min(w.prefill, a + 8192)
                    k = w.token_block_torch("k", layer, a, e, dev)
                    v = w.token_block_torch("v", layer, a, e, dev)
                    self.cache.append(layer, k, v)
                    del k, v
            self.t0 = w.prefill
            self.slots = w.prefill  # grows by one per step; launch_bytes counts the state at the end
        else:  # h2o
            from synth.workloads import h2o_state_torch

            cfg = L.cache_config(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, dt, L.LCD_H2O,
                                 capacity=w.budget, n_recent=w.n_recent, block_size=w.block_size)
            self.cache = L.KVCache(cfg, device=dev)
            K, V, P, S = h2o_state_torch(w, dev)
            kv, vv = self.cache.layer_tensors(0)
            pv, sv = self.cache.h2o_tensors(0)
            kv.copy_(K)
            vv.copy_(V)
            pv.copy_(P)
            sv.copy_(S)
            del K, V, P, S
            L.kv_set_filled(self.cache.handle, 0, w.budget, w.n_prompt)
            self.t0 = w.n_prompt
            self.slots = w.budget
        self.q = [w.token_major_torch("q", l, self.t0, self.t0 + n_tokens, dev) for l in range(w.n_layers)]
        self.k = [w.token_major_torch("k", l, self.t0, self.t0 + n_tokens, dev) for l in range(w.n_layers)]
        self.v = [w.token_major_torch("v", l, self.t0, self.t0 + n_tokens, dev) for l in range(w.n_layers)]
        self.out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device=dev)
        self.i = 0
        torch.cuda.synchronize()

    @property
    def fused(self):
        """Streaming and H2O caches run one lcd_decode_step launch per layer and token."""
        return self.w.kind in ("streaming", "h2o")

    def step(self):
        i = self.i
        for l in range(self.w.n_layers):
            if self.fused:
                self.cache.step(l, self.k[l][i], self.v[l][i], self.q[l][i], self.out)
            else:
                self.cache.append(l, self.k[l][i].unsqueeze(2), self.v[l][i].unsqueeze(2))
                self.cache.decode(l, self.q[l][i], self.out)
        self.i += 1

    def launch(self, j):
        """The decode launch alone, for timing: a fused step re-appending staged token
        j % staged (the ring advances; the data do not change the work), else decode_attn
        on the current state."""
        l = j % self.w.n_layers
        if self.fused:
            t = j % self.q[l].shape[0]
            self.cache.step(l, self.k[l][t], self.v[l][t], self.q[l][t], self.out)
        else:
            self.cache.decode(l, self.q[l][0], self.out)

    def launch_bytes(self):
        """Algorithmic bytes of one decode_attn launch (one layer)."""
        w = self.w
        io = w.batch * w.n_q_heads * w.head_dim * (w.esize + 4)  # q in, fp32 out
        if w.kind == "duo":
            n = self.t0 + self.i  # tokens held now (retrieval heads attend all of them)
            per_layer = []
            for gam in w.retrieval:
                r = sum(gam)
                slots = r * n + (w.n_kv_heads - r) * min(n, w.n_sink + w.window)
                per_layer.append(2 * w.batch * slots * w.head_dim * w.esize + io)
            return sum(per_layer) // len(per_layer)
        kv = 2 * w.batch * w.n_kv_heads * self.slots * w.head_dim * w.esize
        if w.kind == "h2o":
            logits = 2 * w.batch * w.n_q_heads * self.slots * 4  # written then read
            state = w.batch * w.n_kv_heads * self.slots * (4 + 4 + 4)  # score read+write, pos read
            if w.block_size > 1:
                state += w.batch * w.n_kv_heads * self.slots * 4  # positions read again to skip emptied slots
            new_rows = 2 * w.batch * w.n_kv_heads * w.head_dim * w.esize  # the fused append's rows written
            return kv + io + logits + state + new_rows
        if self.fused:  # the new rows are read from the input instead of the cache, then written
            return kv + io + 2 * w.batch * w.n_kv_heads * w.head_dim * w.esize
        return kv + io

    def step_bytes(self):
        w = self.w
        append = 0 if self.fused else 2 * w.batch * w.n_kv_heads * w.head_dim * w.esize
        return w.n_layers * (self.launch_bytes() + append)


def _decode_bench(L, w, steps, warmup, launch_batches=4, launch_batch=64):
    import torch

    st = _Stepper(L, w, warmup + steps)
    for _ in range(warmup):
        st.step()
    torch.cuda.synchronize()
    # timed region: the steps alone
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        st.step()
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    # decode kernel duration: batches of back-to-back decode launches (fused steps for
    # streaming caches) on the state the steps left (every launch reads the full cache),
    # one event pair per batch on the launch stream
    batch_ms = []
    for _ in range(launch_batches):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(launch_batch):
            st.launch(i)
        b.record()
        torch.cuda.synchronize()
        batch_ms.append(a.elapsed_time(b) / launch_batch)
    avg_kernel_ms = sum(batch_ms) / len(batch_ms)
    kind = "decode_onepass_kernel" if w.group <= 2 else "decode_twopass_kernel"
    res = dict(steps_per_s=steps / (total_ms / 1e3), ms_per_step=total_ms / steps, avg_kernel_ms=avg_kernel_ms,
               min_batch_kernel_ms=min(batch_ms), launch_bytes=st.launch_bytes(),
               step_bytes=st.step_bytes(), kernel_launches=launch_batches * launch_batch, kernel=kind,
               entry="lcd_decode_step" if st.fused else "lcd_decode_attn")
    st.cache.close()
    del st
    torch.cuda.empty_cache()
    return res


def _summary(w, r):
    achieved = r["launch_bytes"] / (r["avg_kernel_ms"] / 1e3)
    return {"workload": w.title, "steps_per_s": round(r["steps_per_s"], 2), "ms_per_step": round(r["ms_per_step"], 5),
            "hbm_tb_s": round(r["step_bytes"] * r["steps_per_s"] / 1e12, 3),
            "decode_launch_us": round(r["avg_kernel_ms"] * 1e3, 2),
            "decode_launch_gb_s": round(achieved / 1e9, 1), "decode_launch_frac": round(achieved / HBM_PEAK, 4),
            "bytes_per_launch": r["launch_bytes"]}


def _snapkv_bench(L, w, reps=20):
    """SnapKV compression of the 32k prompt: ms per compress (median of ``reps``, each
    started with the caches flushed by a read)."""
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
    # Read between calls, outside the timed region, so that each compress starts with none
    # of the prompt in the caches (256 MB memory-side cache included) and with clean lines:
    # a write flush would leave dirty lines whose write-back lands in the timed call.
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    for _ in range(3):
        L.snapkv_compress(p, q, k, v, ko, vo, idx, None, ws, wsb)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        flush.sum()
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
            "mfma_frac_bf16": round(flops / (ms / 1e3) / MFMA_BF16_PEAK, 5)}


def _h2o_prompt_bench(L, w, reps=2):
    """H2O prompt-phase compression of the 128k prompt: ms per compress (best of ``reps``
    after one warm-up) and the MFMA rate of its two causal score contractions."""
    import torch

    B, Hq, Hkv, D, N, C = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_prompt, w.budget
    dev = "cuda"
    p = L.h2o_prompt_params(B, Hq, Hkv, D, N, C, w.n_recent)
    wsb = L.h2o_prompt_sizes(p)
    q, k, v = (w.prompt_tensor_torch(t, dev) for t in ("q", "k", "v"))
    ko = torch.empty((B, Hkv, C, D), dtype=torch.bfloat16, device=dev)
    vo = torch.empty_like(ko)
    pos = torch.empty((B, Hkv, C), dtype=torch.int32, device=dev)
    sco = torch.empty((B, Hkv, C), dtype=torch.float32, device=dev)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    L.h2o_prompt_compress(p, q, k, v, ko, vo, pos, sco, None, ws, wsb)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        L.h2o_prompt_compress(p, q, k, v, ko, vo, pos, sco, None, ws, wsb)
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    ms = min(times)
    flops = 2 * B * Hq * (N * (N + 1) // 2) * D * 2  # two causal Q K^T passes
    del q, k, v, ko, vo, ws
    torch.cuda.empty_cache()
    return {"workload": w.title, "compress_ms": round(ms, 2), "reps": reps, "flops": flops,
            "tflops": round(flops / (ms / 1e3) / 1e12, 1),
            "mfma_frac_bf16": round(flops / (ms / 1e3) / MFMA_BF16_PEAK, 4)}


# ---------------------------------------------------------------- fp64 oracle on the host
# The oracle as it stands, timed on all affinity cores (at most 16, the host share of one
# GPU): a pool of worker processes forked before any GPU work, each with BLAS pinned to
# one thread (threadpoolctl), each timing oracle calls on its own share of a bounded
# sample; input generation is excluded from the timed calls.  Throughput = work units done
# / the longest worker's oracle time.


def _oracle_cores():
    return max(1, min(len(os.sched_getaffinity(0)), 16))


def _worker_streaming(args):
    """Oracle decode slices (layer, batch row, KV head) of consecutive steps of a streaming
    workload: the first `budget` seconds' worth of this worker's share."""
    name, worker, n_workers, t0, n_steps, budget = args
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    from synth import WORKLOADS

    w = WORKLOADS[name]
    G = w.group
    done, elapsed = 0, 0.0
    with threadpool_limits(1):
        i = 0
        for t in range(t0, t0 + n_steps):
            toks = oracle.retained_tokens(t, w.n_sink, w.window)
            for layer in range(w.n_layers):
                for b in range(w.batch):
                    for g in range(w.n_kv_heads):
                        i += 1
                        if (i - 1) % n_workers != worker:
                            continue
                        if elapsed >= budget:
                            return done, elapsed
                        kk = w.token_block("k", layer, toks, batches=[b], heads=[g])[0]
                        vv = w.token_block("v", layer, toks, batches=[b], heads=[g])[0]
                        qq = w.token_block("q", layer, [t], batches=[b], heads=np.arange(g * G, g * G + G))[0, :, 0, :]
                        t1 = time.perf_counter()
                        oracle.streaming_decode(qq, lambda _t, kk=kk, vv=vv: (kk, vv), t, w.n_sink, w.window,
                                                w.rope_base)
                        elapsed += time.perf_counter() - t1
                        done += 1
    return done, elapsed


def _worker_snapkv(args):
    """Oracle SnapKV compressions of this worker's heads of the 32k prompt."""
    name, worker, n_workers, budget = args
    from threadpoolctl import threadpool_limits

    import oracle
    from synth import WORKLOADS

    w = WORKLOADS[name]
    done, elapsed = 0, 0.0
    with threadpool_limits(1):
        for i, (b, h) in enumerate((b, h) for b in range(w.batch) for h in range(w.n_q_heads)):
            if i % n_workers != worker:
                continue
            if elapsed >= budget:
                break
            q, k, v = (w.snapkv_tensor(t, b, h) for t in ("q_obs", "k", "v"))
            t1 = time.perf_counter()
            oracle.snapkv_compress(q, k, v, w.k_keep, w.kernel_size)
            elapsed += time.perf_counter() - t1
            done += 1
    return done, elapsed


def _worker_h2o(args):
    """Oracle H2O decode steps (lockstep state of one (batch row, KV head) from the seeded
    budget state) on this worker's heads."""
    name, worker, n_workers, n_steps, budget = args
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    from synth import WORKLOADS

    w = WORKLOADS[name]
    G = w.group
    done, elapsed = 0, 0.0
    with threadpool_limits(1):
        for i, (b, g) in enumerate((b, g) for b in range(w.batch) for g in range(w.n_kv_heads)):
            if i % n_workers != worker:
                continue
            if elapsed >= budget:
                break
            pos, sc, _ = w.h2o_initial_state(b, g)
            head = oracle.H2OHead(w.budget, w.n_recent, pos, w.h2o_kv("k", b, g, pos), w.h2o_kv("v", b, g, pos), sc)
            for s in range(n_steps):
                t = w.n_prompt + s
                q = w.token_block("q", 0, [t], batches=[b], heads=np.arange(g * G, g * G + G))[0, :, 0, :]
                k = w.token_block("k", 0, [t], batches=[b], heads=[g])[0, 0, 0]
                v = w.token_block("v", 0, [t], batches=[b], heads=[g])[0, 0, 0]
                t1 = time.perf_counter()
                head.step(t, q, k, v)
                elapsed += time.perf_counter() - t1
                done += 1
    return done, elapsed


def _pool_map(fn, args):
    import multiprocessing as mp

    with mp.get_context("fork").Pool(len(args)) as pool:
        return pool.map(fn, args)


def _cpu_baselines(headline, budget_s):
    """The oracle's figures for the headline step, the SnapKV compression and the H2O
    budgeted decode step.  Runs before any GPU work (the pool is forked)."""
    from synth import WORKLOADS

    n = _oracle_cores()
    out = {}
    w = WORKLOADS[headline]
    if w.kind == "streaming":
        t0 = w.prefill + 7  # steps after the ring has wrapped
        per_step = w.batch * w.n_kv_heads * w.n_layers
        res = _pool_map(_worker_streaming, [(headline, i, n, t0, 4, budget_s) for i in range(n)])
        done, wall = sum(d for d, _ in res), max(e for _, e in res)
        out["cpu_baseline"] = {
            "value": (done / per_step) / wall, "unit": "decode steps/s", "cores": n, "kind": "oracle",
            "sample": f"{done} (layer, batch row, KV head) decode slices = {done / per_step:.3f} steps from t={t0} "
                      f"({per_step} slices per step) on {n} worker processes, BLAS pinned to 1 thread each; "
                      f"{wall:.1f} s of fp64 numpy on the busiest worker; input generation excluded"}
    sk = WORKLOADS["snapkv_32k"]
    res = _pool_map(_worker_snapkv, [("snapkv_32k", i, n, budget_s / 2) for i in range(n)])
    done, wall = sum(d for d, _ in res), max(e for _, e in res)
    heads = sk.batch * sk.n_q_heads
    # n workers each spent up to `wall` seconds; all `heads` at the measured rate done/wall
    out["snapkv_oracle"] = {"compress_ms": round(wall / done * heads * 1e3, 1), "cores": n, "kind": "oracle",
                            "sample": f"{done} of {heads} heads compressed on {n} worker processes "
                                      f"({wall:.1f} s on the busiest); ms per whole compress at that rate"}
    hw = WORKLOADS["h2o_128k"]
    res = _pool_map(_worker_h2o, [("h2o_128k", i, n, 4, budget_s / 2) for i in range(n)])
    done, wall = sum(d for d, _ in res), max(e for _, e in res)
    per_step = hw.batch * hw.n_kv_heads
    out["h2o_oracle"] = {"value": (done / per_step) / wall, "unit": "decode steps/s", "cores": n, "kind": "oracle",
                         "sample": f"{done} (batch row, KV head) H2O steps = {done / per_step:.3f} steps from "
                                   f"t={hw.n_prompt} on {n} worker processes ({wall:.1f} s on the busiest)"}
    return out


def main(argv=None):
    a = _parse(argv)
    if a.counters:
        if a.workload == "snapkv_32k":
            _snapkv_counter_summary(*a.counters)
        else:
            _counter_summary(*a.counters, workload=a.workload)
        return 0
    if a.mfma_counters:
        _mfma_summary(a.mfma_counters)
        return 0
    if a.workload not in DEFAULTS:
        print(json.dumps({"error": f"{a.workload} is not a decode workload (use --snapkv-only)"}))
        return 2
    if a.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only (one MI355X per box here); "
                                   "--gpus must be 1", "n_gpus_requested": a.gpus}))
        return 2
    # the oracle first: its worker processes are forked before anything touches the GPU
    cpu = {} if (a.no_cpu_baseline or a.snapkv_only) else _cpu_baselines(a.workload, a.cpu_seconds)
    import torch

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        return 2
    import long_context_decode_amd as L
    from synth import WORKLOADS

    if a.snapkv_only:
        from synth.workloads import scaled

        if a.copy_calibration:
            _copy_calibration()
        sk = WORKLOADS["snapkv_32k"]
        if a.l_obs:
            sk = scaled(sk, name=f"snapkv_32k_obs{a.l_obs}", l_obs=a.l_obs,
                        title=sk.title.replace("L_obs=32", f"L_obs={a.l_obs}"))
        print(json.dumps(_snapkv_bench(L, sk)), flush=True)
        return 0
    if a.copy_calibration:
        _copy_calibration()
    w = WORKLOADS[a.workload]
    steps, warmup = DEFAULTS[a.workload]
    steps = a.steps if a.steps is not None else steps
    warmup = a.warmup if a.warmup is not None else warmup
    r = _decode_bench(L, w, steps, warmup)
    achieved = r["launch_bytes"] / (r["avg_kernel_ms"] / 1e3)
    kernel = TRAFFIC.get(a.workload, (r["kernel"],))[0]
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
                   "head_dim": w.head_dim, "n_layers": w.n_layers,
                   "cache_slots": w.n_sink + w.window if w.kind == "streaming" else w.budget},
        "hbm_tb_s": round(r["step_bytes"] * r["steps_per_s"] / 1e12, 3),
        "hbm_frac_of_peak": round(r["step_bytes"] * r["steps_per_s"] / HBM_PEAK, 4),
        "roofline": {"bound": "hbm", "kernel": f"{kernel} ({r['entry']}, one launch per layer)",
                     "achieved": round(achieved / 1e9, 1), "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK, 4), "traffic": _traffic(a.workload),
                     "bytes_per_launch": r["launch_bytes"], "avg_launch_us": round(r["avg_kernel_ms"] * 1e3, 2),
                     "best_batch_launch_us": round(r["min_batch_kernel_ms"] * 1e3, 2),
                     "launches_timed": r["kernel_launches"]},
    }
    if not a.only and not a.no_snapkv:
        line["snapkv"] = _snapkv_bench(L, WORKLOADS["snapkv_32k"])
        if "snapkv_oracle" in cpu:
            line["snapkv"]["oracle"] = cpu["snapkv_oracle"]
        # the observation window swept: the scoring product grows with L_obs, K's bytes do not
        from synth.workloads import scaled

        sweep = []
        for lo in (64, 128, 256):
            rec = _snapkv_bench(L, scaled(WORKLOADS["snapkv_32k"], name=f"snapkv_32k_obs{lo}", l_obs=lo), reps=10)
            sweep.append({"l_obs": lo, "compress_ms": rec["compress_ms"], "qk_tflops": rec["qk_tflops"],
                          "mfma_frac_bf16": rec["mfma_frac_bf16"], "mfma_ceiling": round(min(1.0, lo / 312.0), 3)})
        line["snapkv"]["l_obs_sweep"] = sweep
    if not a.only and not a.no_h2o_prompt:
        line["h2o_prompt"] = _h2o_prompt_bench(L, WORKLOADS["h2o_prompt_128k"])
    if not a.only:
        others = []
        for name in ("llama2_7b_layer", "llama3_8b_layer", "h2o_128k", "h2o_blocks_128k", "duo_128k", "tiny_streaming"):
            if name == a.workload:
                continue
            s2, w2 = DEFAULTS[name]
            if name == "tiny_streaming":
                w2 = min(w2, WORKLOADS[name].steps - s2)
            rec = _summary(WORKLOADS[name], _decode_bench(L, WORKLOADS[name], s2, w2))
            rec["traffic"] = _traffic(name)
            if name == "h2o_128k" and "h2o_oracle" in cpu:
                rec["oracle"] = cpu["h2o_oracle"]
            others.append(rec)
        line["other_workloads"] = others
    if "cpu_baseline" in cpu:
        line["cpu_baseline"] = cpu["cpu_baseline"]
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
