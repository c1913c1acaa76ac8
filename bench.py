#!/usr/bin/env python
"""Benchmark of the exact-attention path on one MI355X; prints ONE JSON line.

A step is one pass of the whole path over resident synthetic inputs:
  1. fa_fwd    B=1 H=32 N=8192 d=128 bf16, causal, Q scaled x2
  2. fa_bwd    the same shape (dO ~ N(0,1)), consuming the forward's O and lse
  3. fa_decode B=64 H=32 Nkv=16384 d=128 bf16, 16 history chunks per head
value = (fwd + bwd useful FLOPs) / (fwd + bwd time), in TFLOP/s, with
useful FLOPs 4 B H N^2 d (forward) and 10 B H N^2 d (backward: five N x N x d
products), both halved for the causal mask.  Decode is reported in GB/s of
algorithmic HBM bytes (K + V + q + o).  Each entry point is timed live with
HIP events recorded on the stream its kernels run on (torch's current
stream, which the binding hands to the library).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--only fwd|bwd|decode|ext] [--no-ext]
--only runs a single entry point per step (for per-kernel profiling); the
JSON line then carries only that entry's figures.  --only ext runs only the
extension workloads.

After the timed steps, the extension entry points are timed on their own
workloads, outside the step (they do not enter value or ms_per_step):
  * fa_decode_ex, grouped key/value heads: B=64 H=32 H_kv=8 Nkv=16384 d=128
    bf16, 16 chunks; GB/s of algorithmic bytes, K and V counted once per
    key/value head;
  * fa_fwd_ex, causal sliding window of 1024 keys: B=1 H=32 N=8192 d=128
    bf16; TFLOP/s of useful work, 4 d FLOPs per visible (query, key) pair;
  * fa_decode_varlen, the grouped-head decode cache with ragged histories
    (lengths uniform in [1, 16384], seeded); GB/s of the bytes the lengths
    select (each sequence's K and V rows once per key/value head, q, o).
The other forward/backward configurations (tiny fp16 forward B1 H1 N256 d64;
B4 H16 N2048 d128 bf16 causal forward; B2 H16 N4096 d128 bf16 causal
backward) are timed the same way under "configs" (TFLOP/s of 4 B H N^2 d
forward and 10 B H N^2 d backward FLOPs, halved for causal, as the step).
--no-ext skips both (profiles of the step's kernels alone).
--copy-calibration BYTES only copies a BYTES-sized device buffer 5 times
(a plain copy kernel of known traffic, used to scale HBM byte counters).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E bandwidth (published)
CSRC = os.path.join(ROOT, "exact_io_aware_31_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
# Each entry point's kernel source and the device headers it includes.
KERNEL_SOURCES = {"fwd": ("fa_fwd.hip", "fa_tile.h", "fa_common.h"),
                  "bwd": ("fa_bwd.hip", "fa_tile.h", "fa_common.h"),
                  "decode": ("fa_decode.hip", "fa_common.h")}


def source_sha(entry: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[entry]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(entry: str):
    """HBM bytes per launch measured by rocprofv3 counters, if the kernel is unchanged since."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    for line in open(TRAFFIC_FILE):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        kv = dict(tok.split("=", 1) for tok in line.split() if "=" in tok)
        if kv.get("entry") == entry:
            if kv.get("source_sha256") != source_sha(entry):
                return None
            return float(kv["bytes_per_launch"])
    return None


def cpu_baseline(q, k, v, do, lse_unused, decode_inputs, heads: int, scale: float):
    """The float64 oracle, unmodified, on a bounded sample of the same workload."""
    import numpy as np
    import oracle

    n, d = q.shape[-2], q.shape[-1]
    t0 = time.perf_counter()
    for h in range(heads):
        qh, kh, vh, doh = (t[0, h].cpu() for t in (q, k, v, do))
        oracle.attn_fwd(qh, kh, vh, scale, True)
        oracle.attn_bwd(qh, kh, vh, doh, scale, True)
    secs = time.perf_counter() - t0
    flops = heads * (4 + 10) * n * n * d / 2
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": f"float64 oracle forward + backward on {heads} of 32 heads of the "
                      f"N={n} d={d} causal workload ({secs:.1f} s; useful-FLOP formula)"}


def time_calls(torch, call, reps: int, warmup: int = 2) -> float:
    """Average ms per call, HIP events on the current stream (the one the binding uses)."""
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        call()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / reps


def measure_extensions(fa, torch, dev, reps: int):
    """Grouped-head decode and sliding-window forward on their own workloads."""
    from synth_inputs import GQA_DECODE_16K, WINDOW_FWD_8K, workload_inputs
    out = []
    w = WINDOW_FWD_8K
    q, k, v = workload_inputs(w, dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    ms = time_calls(torch, lambda: fa.fa_fwd_ex(q, k, v, o, lse, w.scale, True, w.window), reps)
    pairs = w.window * (w.window + 1) // 2 + (w.N - w.window) * w.window
    tf = 4 * w.B * w.H * w.d * pairs / (ms * 1e-3) / 1e12
    out.append({"workload": w.name, "entry": "fa_fwd_ex", "bound": "mfma",
                "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tf / PEAK_BF16_TFLOPS, 4), "ms": round(ms, 4)})
    del q, k, v, o, lse
    w = GQA_DECODE_16K
    q, k, v = workload_inputs(w, dev)
    o = torch.empty((w.B, w.H, 1, w.d), dtype=w.dtype, device=dev)
    lse = torch.empty((w.B, w.H), dtype=torch.float32, device=dev)
    ws = fa.decode_workspace(k, w.splits, heads=w.H)
    ms = time_calls(torch, lambda: fa.fa_decode_ex(q, k, v, o, lse, w.scale, w.splits, ws), reps)
    nbytes = (2 * w.B * w.Hkv * w.Nkv * w.d + 2 * w.B * w.H * w.d) * 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    out.append({"workload": w.name, "entry": "fa_decode_ex", "bound": "hbm",
                "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "ms": round(ms, 4)})
    from synth_inputs import ragged_lengths
    lens_h = ragged_lengths(w.B, w.Nkv, w.seed)
    lens = lens_h.to(dev)
    ms = time_calls(torch, lambda: fa.fa_decode_varlen(q, k, v, lens, o, lse, w.scale, w.splits,
                                                       ws), reps)
    nbytes = (2 * w.Hkv * int(lens_h.sum()) * w.d + 2 * w.B * w.H * w.d) * 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    out.append({"workload": w.name + "_ragged", "entry": "fa_decode_varlen", "bound": "hbm",
                "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "ms": round(ms, 4)})
    del q, k, v, o, lse, ws, lens
    torch.cuda.empty_cache()
    return out


def measure_configs(fa, torch, dev, reps: int):
    """The forward and backward shapes the step does not time itself: the tiny fp16 forward,
    the B4 H16 N2048 causal forward and the B2 H16 N4096 causal backward (useful-FLOP rates)."""
    from synth_inputs import BWD_4K, FWD_2K, TINY_FWD, workload_inputs
    out = []
    for w in (TINY_FWD, FWD_2K, BWD_4K):
        ins = workload_inputs(w, dev)
        q, k, v = ins[:3]
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
        fa.fa_fwd(q, k, v, o, lse, w.scale, w.causal)
        pairs = w.N * w.N / 2 if w.causal else w.N * w.N  # halved for causal, as the step
        if w.kind == "fwd":
            ms = time_calls(torch, lambda: fa.fa_fwd(q, k, v, o, lse, w.scale, w.causal), reps)
            flops = 4 * w.B * w.H * w.d * pairs
        else:
            do = ins[3]
            dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
            ws = fa.bwd_workspace(q)
            ms = time_calls(torch, lambda: fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, w.scale,
                                                     w.causal), reps)
            flops = 10 * w.B * w.H * w.d * pairs
        tf = flops / (ms * 1e-3) / 1e12
        out.append({"workload": w.name, "entry": "fa_" + w.kind, "bound": "mfma",
                    "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tf / PEAK_BF16_TFLOPS, 4), "ms": round(ms, 4)})
        del ins, q, k, v, o, lse
    torch.cuda.empty_cache()
    return out


def copy_calibration(torch, nbytes: int, reps: int = 5):
    """Time a plain device-to-device copy of nbytes (reads nbytes, writes nbytes)."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        dst.copy_(src)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / reps
    print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written": src.numel() * 4,
                      "reps": reps, "ms_per_copy": round(ms, 4),
                      "gbs_read_plus_write": round(2 * src.numel() * 4 / (ms * 1e-3) / 1e9, 1)}),
          flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=16)
    ap.add_argument("--only", choices=("fwd", "bwd", "decode", "ext"), default=None)
    ap.add_argument("--no-ext", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this attention path runs on a single GPU "
              "(attention heads are independent, so N GPUs would each run their own share "
              "with no exchange).", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        copy_calibration(torch, args.copy_calibration)
        return

    import exact_io_aware_31_amd as fa
    from synth_inputs import DECODE_16K, FWD_8K, attention_inputs

    fa.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w, wd = FWD_8K, DECODE_16K
    if args.only == "ext":
        ext = measure_extensions(fa, torch, dev, args.steps)
        print(json.dumps({"metric": "extension entry points (grouped-head decode GB/s, "
                                    "sliding-window forward TFLOP/s)",
                          "value": ext[1]["achieved"], "unit": "GB/s", "n_gpus": 1,
                          "steps": args.steps, "warmup": 2, "higher_is_better": True,
                          "data": "synthetic", "extensions": ext, "only": "ext"}), flush=True)
        return

    # Inputs drawn on the GPU and resident in HBM before timing starts.
    q, k, v, do = attention_inputs(w.B, w.H, w.N, w.d, w.dtype, w.seed, dev, q_mult=w.q_mult,
                                   with_dout=True)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_b = fa.bwd_workspace(q)
    qd, kd, vd = attention_inputs(wd.B, wd.H, 1, wd.d, wd.dtype, wd.seed, dev, Nkv=wd.Nkv)
    od = torch.empty((wd.B, wd.H, 1, wd.d), dtype=wd.dtype, device=dev)
    lsed = torch.empty((wd.B, wd.H), dtype=torch.float32, device=dev)
    ws_d = fa.decode_workspace(kd, wd.splits)
    torch.cuda.synchronize()

    run = {e: args.only in (None, e) for e in ("fwd", "bwd", "decode")}
    if run["bwd"] and not run["fwd"]:  # the backward consumes a forward's O and lse
        fa.fa_fwd(q, k, v, o, lse, w.scale, w.causal)

    def step(ev):
        ev[0].record()
        if run["fwd"]:
            fa.fa_fwd(q, k, v, o, lse, w.scale, w.causal)
        ev[1].record()
        if run["bwd"]:
            fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, ws_b, w.scale, w.causal)
        ev[2].record()
        if run["decode"]:
            fa.fa_decode(qd, kd, vd, od, lsed, wd.scale, wd.splits, ws_d)
        ev[3].record()

    for _ in range(args.warmup):
        step([torch.cuda.Event(enable_timing=True) for _ in range(4)])
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record()
    for i in range(args.steps):
        step(events[i])
    end.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_step = start.elapsed_time(end) / args.steps
    ms = {name: sum(e[j].elapsed_time(e[j + 1]) for e in events) / args.steps
          for j, name in enumerate(("fwd", "bwd", "decode"))}

    nn = w.B * w.H * w.N * w.N * w.d
    fwd_flops = 4 * nn / 2
    bwd_flops = 10 * nn / 2
    elem = 2  # bf16 bytes
    dec_bytes = (2 * wd.B * wd.H * wd.Nkv * wd.d + 2 * wd.B * wd.H * wd.d) * elem
    def rate(amount, entry):
        return amount / (ms[entry] * 1e-3) if run[entry] and ms[entry] > 0 else 0.0

    fwd_tf = rate(fwd_flops, "fwd") / 1e12
    bwd_tf = rate(bwd_flops, "bwd") / 1e12
    dec_gbs = rate(dec_bytes, "decode") / 1e9
    if args.only is None:
        value = (fwd_flops + bwd_flops) / ((ms["fwd"] + ms["bwd"]) * 1e-3) / 1e12
    else:
        value = {"fwd": fwd_tf, "bwd": bwd_tf, "decode": dec_gbs}[args.only]

    def roof(entry, bound, achieved, peak, unit):
        return {"entry": entry, "bound": bound, "achieved": round(achieved, 2), "peak": peak,
                "unit": unit, "frac": round(achieved / peak, 4),
                "traffic": measured_traffic(entry), "ms": round(ms[entry], 4)}

    roofs = [roof("fwd", "mfma", fwd_tf, PEAK_BF16_TFLOPS, "TFLOP/s"),
             roof("bwd", "mfma", bwd_tf, PEAK_BF16_TFLOPS, "TFLOP/s"),
             roof("decode", "hbm", dec_gbs, PEAK_HBM_GBS, "GB/s")]
    roofs = [r for r in roofs if run[r["entry"]]]
    dominant = max(roofs, key=lambda r: r["ms"])

    out = {
        "metric": "fwd/bwd attention TFLOP/s (% MFMA peak) N=8192 d=128 bf16; decode HBM GB/s",
        "value": round(value, 2),
        "unit": "GB/s" if args.only == "decode" else "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "attention fwd+bwd B1 H32 N8192 d128 bf16 causal (Q x2) + "
                               "decode B64 H32 Nkv16384 d128 bf16 16 splits",
                   "global_batch": w.B, "seq_len": w.N, "heads": w.H, "head_dim": w.d,
                   "decode_batch": wd.B, "decode_kv_len": wd.Nkv, "decode_splits": wd.splits},
        "fwd_tflops": round(fwd_tf, 2),
        "bwd_tflops": round(bwd_tf, 2),
        "decode_gbs": round(dec_gbs, 2),
        "roofline": dominant,
        "rooflines": roofs,
        "wall_s_timed": round(t_wall, 3),
    }
    if args.only is None and not args.no_ext:
        out["configs"] = measure_configs(fa, torch, dev, max(5, args.steps // 2))
        out["extensions"] = measure_extensions(fa, torch, dev, max(5, args.steps // 2))
    if args.only is not None:
        out["only"] = args.only
    if not args.no_cpu_baseline and args.only is None:
        out["cpu_baseline"] = cpu_baseline(q, k, v, do, lse, None, args.cpu_heads, w.scale)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
