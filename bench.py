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
stream, which the binding hands to the library): the mean over the timed
steps enters value; the median and the minimum are reported beside it.
Within a step every call is bracketed by events (each event holds the
stream for about 10 us, under 1% of a step, which the step's figures
include); the workloads timed after the step are timed in batches of five
back-to-back calls with events only between batches.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--only ENTRY|WORKLOAD] [--no-ext] [--no-peaks]
--only fwd|bwd|decode runs a single entry point of the step; --only ext only
the extension workloads; --only <workload name> (tiny_fwd_b1h1n256d64_f16,
fwd_b4h16n2048d128_bf16_causal, bwd_b2h16n4096d128_bf16_causal) only that
workload, W warm-up and K timed calls.  These modes exist so that a profile
holds one workload's kernels; their JSON line carries only those figures.

After the timed steps (default run only):
  * configs: every workload of the specification in one list -- the tiny
    fp16 forward, the B4 H16 N2048 causal forward, the step's N=8192 forward,
    the B2 H16 N4096 causal backward, the step's decode, and (supplementary)
    the backward at the step's N=8192 shape.  The first two and the N=4096
    backward are timed after the step, the same way;
  * extensions: fa_fwd_ex with a causal window of 1024 keys (B1 H32 N8192),
    fa_decode_ex with grouped key/value heads (B64 H32 H_kv8 Nkv16384) and
    fa_decode_varlen over the same cache with ragged histories;
  * measured_peaks: the chip's own ceilings from libfa_probe (dense bf16
    matrix rate with the shader clock under that load; streaming read rate);
  * cpu_baseline / cpu_baselines: the float64 oracle timed on this host's
    cores on a bounded sample of each workload.
Every roofline entry reports its rate against the published peak (frac),
against the measured ceiling (frac_measured), and, from the committed
rocprofv3 counter summary of the same kernel sources (profiles/), the HBM
bytes per launch (traffic), the shader clock under that load (clock_ghz) and
the published peak scaled to that clock (frac_at_clock).
--copy-calibration BYTES only copies a BYTES-sized device buffer 5 times
(a plain copy kernel of known traffic, used to scale HBM byte counters).
"""
import argparse
import hashlib
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E bandwidth (published)
SPEC_CLOCK_GHZ = 2.4        # clock the published matrix peak assumes
CSRC = os.path.join(ROOT, "exact_io_aware_31_amd", "csrc")
INDEX_FILE = os.path.join(ROOT, "profiles", "roofline_index.txt")
# Each kernel family's source and the device headers it includes.
KERNEL_SOURCES = {"fwd": ("fa_fwd.hip", "fa_tile.h", "fa_common.h"),
                  "bwd": ("fa_bwd.hip", "fa_tile.h", "fa_common.h"),
                  "decode": ("fa_decode.hip", "fa_tile.h", "fa_common.h")}
FAMILY = {"fa_fwd": "fwd", "fa_fwd_ex": "fwd", "fa_bwd": "bwd", "fa_decode": "decode",
          "fa_decode_ex": "decode", "fa_decode_varlen": "decode"}
BWD_8K_NAME = "bwd_b1h32n8192d128_bf16_causal_q2"


def source_sha(family: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[family]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def profile_index():
    """Committed rocprofv3 figures per (workload, entry), kept only where the kernel sources
    are unchanged since the counters were taken."""
    out = {}
    if not os.path.exists(INDEX_FILE):
        return out
    for line in open(INDEX_FILE):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        kv = dict(tok.split("=", 1) for tok in line.split() if "=" in tok)
        fam = FAMILY.get(kv.get("entry", ""))
        if fam and kv.get("source_sha256") == source_sha(fam):
            out[(kv["workload"], kv["entry"])] = kv
    return out


def host_info(oracle_threads=None):
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    info = {"cpu_model": model or platform.processor() or None, "nproc": os.cpu_count()}
    try:
        info["affinity_cpus"] = len(os.sched_getaffinity(0))
    except AttributeError:
        pass
    if oracle_threads is not None:
        info["oracle_threads"] = oracle_threads
    return info


def stats(ms_list):
    return {"ms": round(statistics.fmean(ms_list), 4), "ms_median": round(statistics.median(ms_list), 4),
            "ms_min": round(min(ms_list), 4)}


def time_calls(torch, call, reps: int, warmup: int, batch: int = 5):
    """Milliseconds per call, one value per batch of `batch` back-to-back calls: HIP events on
    the current stream (the one the binding hands to the library) bracket each batch, not each
    call.  An event recorded between two calls holds the stream for about 10 us, which is 1.5%
    of a grouped decode and 6% of a window forward, so events only at batch boundaries leave
    the calls' own back-to-back rate.  reps calls in all (at least one batch)."""
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    batch = max(1, min(batch, reps))
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(max(1, reps // batch))]
    for a, b in ev:
        a.record()
        for _ in range(batch):
            call()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) / batch for a, b in ev]


def roofline(workload, entry, bound, amount, ms_list, index, peaks):
    """One roofline entry: amount is FLOP (bound mfma) or bytes (bound hbm) per call."""
    st = stats(ms_list)
    unit = "TFLOP/s" if bound == "mfma" else "GB/s"
    scale = 1e12 if bound == "mfma" else 1e9
    peak = PEAK_BF16_TFLOPS if bound == "mfma" else PEAK_HBM_GBS
    achieved = amount / (st["ms"] * 1e-3) / scale
    r = {"workload": workload, "entry": entry, "bound": bound, "achieved": round(achieved, 2),
         "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
         "achieved_at_median": round(amount / (st["ms_median"] * 1e-3) / scale, 2),
         "achieved_at_min": round(amount / (st["ms_min"] * 1e-3) / scale, 2)}
    r.update(st)
    mp = None
    if peaks:
        mp = peaks.get("mfma", {}).get("tflops") if bound == "mfma" else peaks.get("read", {}).get("gbs")
    r["peak_measured"] = mp
    r["frac_measured"] = round(achieved / mp, 4) if mp else None
    prof = index.get((workload, entry)) if index is not None else None
    r["traffic"] = float(prof["hbm_bytes"]) if prof and "hbm_bytes" in prof else None
    r["traffic_ratio"] = float(prof["ratio"]) if prof and "ratio" in prof else None
    r["profiled_ms"] = round(float(prof["kernel_us"]) / 1e3, 4) if prof else None
    clock = float(prof["clock_ghz"]) if prof and prof.get("clock_ghz") not in (None, "na") else None
    r["clock_ghz"] = clock
    # The published peak scaled to a clock under matrix load: the probe's, measured on this machine
    # in this run, else the profiled kernel's (another run, possibly another box).
    probe_clock = (peaks or {}).get("mfma", {}).get("clock_ghz")
    scale_clock, source = (probe_clock, "probe, this run") if probe_clock else (clock, "profile")
    if bound == "mfma" and scale_clock:
        pc = PEAK_BF16_TFLOPS * scale_clock / SPEC_CLOCK_GHZ
        r["peak_at_clock"] = round(pc, 1)
        r["frac_at_clock"] = round(achieved / pc, 4)
        r["clock_for_peak"] = {"ghz": scale_clock, "source": source}
    if prof and prof.get("mfma_busy") not in (None, "na"):
        r["mfma_busy"] = float(prof["mfma_busy"])
    return r


def fwd_flops(w):
    pairs = w.N * w.N / 2 if w.causal else w.N * w.N  # halved for causal
    return 4 * w.B * w.H * w.d * pairs


def bwd_flops(w):
    pairs = w.N * w.N / 2 if w.causal else w.N * w.N
    return 10 * w.B * w.H * w.d * pairs


def decode_bytes(w):
    hkv = w.Hkv or w.H
    return (2 * w.B * hkv * w.Nkv * w.d + 2 * w.B * w.H * w.d) * 2


# ------------------------------------------------------------------ oracle baseline
def _oracle_timed(fn):
    t0 = time.perf_counter()
    fn()
    return time.perf_counter() - t0


def cpu_baseline_step(q, k, v, do, heads: int, scale: float):
    """The float64 oracle, unmodified, forward + backward on `heads` heads of the step's
    N=8192 causal workload (the metric's workload)."""
    import oracle

    n, d = q.shape[-2], q.shape[-1]
    hs = [tuple(t[0, h].cpu() for t in (q, k, v, do)) for h in range(heads)]
    secs = _oracle_timed(lambda: [(oracle.attn_fwd(a, b, c, scale, True),
                                   oracle.attn_bwd(a, b, c, g, scale, True)) for a, b, c, g in hs])
    flops = heads * (4 + 10) * n * n * d / 2
    return {"value": round(flops / secs / 1e12, 5), "unit": "TFLOP/s",
            "cores": oracle.max_threads(), "kind": "oracle", "secs": round(secs, 2),
            "sample": f"float64 oracle forward + backward on {heads} of 32 heads of the N={n} "
                      f"d={d} causal workload ({secs:.1f} s; useful-FLOP formula)"}


def cpu_baselines_configs(dev, step_inputs, decode_inputs):
    """The oracle timed on a bounded sample of every workload (seconds, and GFLOP/s or GB/s
    with the same formulas as the GPU figures)."""
    import torch

    import oracle
    from synth_inputs import BWD_4K, DECODE_16K, FWD_2K, FWD_8K, TINY_FWD, attention_inputs

    out = []

    def rec(w, entry, secs, amount, unit, sample):
        scale = 1e9
        out.append({"workload": w if isinstance(w, str) else w.name, "entry": entry,
                    "value": round(amount / secs / scale, 4), "unit": unit, "secs": round(secs, 3),
                    "cores": oracle.max_threads(), "kind": "oracle", "sample": sample})

    w = TINY_FWD
    q, k, v = attention_inputs(w.B, w.H, w.N, w.d, w.dtype, w.seed, "cpu")
    secs = _oracle_timed(lambda: oracle.attn_fwd(q, k, v, w.scale, w.causal))
    rec(w, "fa_fwd", secs, fwd_flops(w), "GFLOP/s", "whole workload, forward")

    w, nh = FWD_2K, 8
    q, k, v = attention_inputs(1, nh, w.N, w.d, w.dtype, w.seed, "cpu")
    secs = _oracle_timed(lambda: oracle.attn_fwd(q, k, v, w.scale, w.causal))
    rec(w, "fa_fwd", secs, fwd_flops(w) * nh / (w.B * w.H), "GFLOP/s",
        f"forward on {nh} of {w.B * w.H} heads (same shape and generator)")

    w, nh = FWD_8K, 2
    q, k, v = (t[0, :nh].cpu() for t in step_inputs[:3])
    secs = _oracle_timed(lambda: oracle.attn_fwd(q, k, v, w.scale, w.causal))
    rec(w, "fa_fwd", secs, fwd_flops(w) * nh / (w.B * w.H), "GFLOP/s",
        f"forward on {nh} of {w.B * w.H} heads of the step's inputs")

    w, nh = BWD_4K, 2
    q, k, v, do = attention_inputs(1, nh, w.N, w.d, w.dtype, w.seed, "cpu", with_dout=True)
    secs = _oracle_timed(lambda: oracle.attn_bwd(q, k, v, do, w.scale, w.causal))
    rec(w, "fa_bwd", secs, bwd_flops(w) * nh / (w.B * w.H), "GFLOP/s",
        f"backward on {nh} of {w.B * w.H} heads (same shape and generator)")

    w, nb = DECODE_16K, 1
    qd, kd, vd = (t[:nb].cpu() for t in decode_inputs)
    secs = _oracle_timed(lambda: oracle.attn_decode(qd, kd, vd, w.scale))
    sample_bytes = (2 * nb * w.H * w.Nkv * w.d + 2 * nb * w.H * w.d) * 2
    rec(w, "fa_decode", secs, sample_bytes, "GB/s",
        f"decode of {nb} of {w.B} sequences (all {w.H} heads, {w.Nkv} keys; bytes of the "
        "bf16 K, V, q, o of the sample, float64 widening included)")
    del qd, kd, vd
    return out


# ------------------------------------------------------------------ workloads after the step
def measure_extensions(fa, torch, dev, reps, warmup, index, peaks):
    """Grouped-head decode, ragged decode and sliding-window forward on their own workloads."""
    from synth_inputs import GQA_DECODE_16K, WINDOW_FWD_8K, ragged_lengths, workload_inputs
    out = []
    w = WINDOW_FWD_8K
    q, k, v = workload_inputs(w, dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    ms = time_calls(torch, lambda: fa.fa_fwd_ex(q, k, v, o, lse, w.scale, True, w.window), reps,
                    warmup)
    pairs = w.window * (w.window + 1) // 2 + (w.N - w.window) * w.window
    out.append(roofline(w.name, "fa_fwd_ex", "mfma", 4 * w.B * w.H * w.d * pairs, ms, index, peaks))
    del q, k, v, o, lse
    w = GQA_DECODE_16K
    q, k, v = workload_inputs(w, dev)
    o = torch.empty((w.B, w.H, 1, w.d), dtype=w.dtype, device=dev)
    lse = torch.empty((w.B, w.H), dtype=torch.float32, device=dev)
    ws = fa.decode_workspace(k, w.splits, heads=w.H)
    ms = time_calls(torch, lambda: fa.fa_decode_ex(q, k, v, o, lse, w.scale, w.splits, ws), reps,
                    warmup)
    out.append(roofline(w.name, "fa_decode_ex", "hbm", decode_bytes(w), ms, index, peaks))
    lens_h = ragged_lengths(w.B, w.Nkv, w.seed)
    lens = lens_h.to(dev)
    ms = time_calls(torch, lambda: fa.fa_decode_varlen(q, k, v, lens, o, lse, w.scale, w.splits,
                                                       ws), reps, warmup)
    nbytes = (2 * w.Hkv * int(lens_h.sum()) * w.d + 2 * w.B * w.H * w.d) * 2
    out.append(roofline(w.name + "_ragged", "fa_decode_varlen", "hbm", nbytes, ms, index, peaks))
    del q, k, v, o, lse, ws, lens
    torch.cuda.empty_cache()
    return out


def measure_config(fa, torch, dev, w, reps, warmup, index, peaks):
    """One forward or backward workload of the specification, timed in batches of calls."""
    from synth_inputs import workload_inputs
    ins = workload_inputs(w, dev)
    q, k, v = ins[:3]
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    fa.fa_fwd(q, k, v, o, lse, w.scale, w.causal)
    if w.kind == "fwd":
        ms = time_calls(torch, lambda: fa.fa_fwd(q, k, v, o, lse, w.scale, w.causal), reps, warmup)
        r = roofline(w.name, "fa_fwd", "mfma", fwd_flops(w), ms, index, peaks)
    else:
        do = ins[3]
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = fa.bwd_workspace(q)
        ms = time_calls(torch, lambda: fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, w.scale,
                                                 w.causal), reps, warmup)
        r = roofline(w.name, "fa_bwd", "mfma", bwd_flops(w), ms, index, peaks)
    del ins, q, k, v, o, lse
    torch.cuda.empty_cache()
    return r


def copy_calibration(torch, nbytes: int, reps: int = 5):
    """Time a plain device-to-device copy of nbytes (reads nbytes, writes nbytes)."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    ms = statistics.median(time_calls(torch, lambda: dst.copy_(src), reps, 1))
    print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written": src.numel() * 4,
                      "reps": reps, "ms_per_copy": round(ms, 4),
                      "gbs_read_plus_write": round(2 * src.numel() * 4 / (ms * 1e-3) / 1e9, 1)}),
          flush=True)


def measure_peaks(torch):
    from exact_io_aware_31_amd import probe
    return {"mfma": probe.mfma_bf16_rate(torch), "read": probe.stream_read_rate(torch)}


METRIC = "fwd/bwd attention TFLOP/s (% MFMA peak) N=8192 d=128 bf16; decode HBM GB/s"


def main():
    from synth_inputs import BWD_4K, DECODE_16K, FWD_2K, FWD_8K, TINY_FWD, attention_inputs
    single = {w.name: w for w in (TINY_FWD, FWD_2K, BWD_4K)}

    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=8)
    ap.add_argument("--only", choices=["fwd", "bwd", "decode", "ext"] + sorted(single), default=None)
    ap.add_argument("--no-ext", action="store_true")
    ap.add_argument("--no-peaks", action="store_true")
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

    fa.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    index = profile_index()
    base = {"n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
            "data": "synthetic"}

    if args.only == "ext":
        ext = measure_extensions(fa, torch, dev, args.steps, args.warmup, index, None)
        print(json.dumps({"metric": "extension entry points (grouped-head decode GB/s, "
                                    "ragged decode GB/s, sliding-window forward TFLOP/s)",
                          "value": ext[1]["achieved"], "unit": "GB/s", **base,
                          "extensions": ext, "only": "ext"}), flush=True)
        return
    if args.only in single:
        r = measure_config(fa, torch, dev, single[args.only], args.steps, args.warmup, index, None)
        print(json.dumps({"metric": f"{r['entry']} {r['workload']}", "value": r["achieved"],
                          "unit": r["unit"], **base, "roofline": r, "only": args.only}), flush=True)
        return

    w, wd = FWD_8K, DECODE_16K
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
    per_call = {name: [e[j].elapsed_time(e[j + 1]) for e in events]
                for j, name in enumerate(("fwd", "bwd", "decode"))}

    peaks = None
    if args.only is None and not args.no_peaks:
        peaks = measure_peaks(torch)

    nn = w.B * w.H * w.N * w.N * w.d
    fwd_f, bwd_f, dec_b = 4 * nn / 2, 10 * nn / 2, decode_bytes(wd)
    roofs = []
    if run["fwd"]:
        roofs.append(roofline(w.name, "fa_fwd", "mfma", fwd_f, per_call["fwd"], index, peaks))
    if run["bwd"]:
        roofs.append(roofline(BWD_8K_NAME, "fa_bwd", "mfma", bwd_f, per_call["bwd"], index, peaks))
    if run["decode"]:
        roofs.append(roofline(wd.name, "fa_decode", "hbm", dec_b, per_call["decode"], index, peaks))
    by_entry = {r["entry"]: r for r in roofs}
    dominant = max(roofs, key=lambda r: r["ms"])
    if args.only is None:
        tf = statistics.fmean(per_call["fwd"]) + statistics.fmean(per_call["bwd"])
        value = (fwd_f + bwd_f) / (tf * 1e-3) / 1e12
    else:
        value = roofs[0]["achieved"]

    out = {
        "metric": METRIC,
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
        "fwd_tflops": by_entry["fa_fwd"]["achieved"] if run["fwd"] else 0.0,
        "bwd_tflops": by_entry["fa_bwd"]["achieved"] if run["bwd"] else 0.0,
        "decode_gbs": by_entry["fa_decode"]["achieved"] if run["decode"] else 0.0,
        "roofline": dominant,
        "rooflines": roofs,
        "wall_s_timed": round(t_wall, 3),
    }
    if args.only is not None:
        out["only"] = args.only
        print(json.dumps(out), flush=True)
        return
    if peaks is not None:
        out["measured_peaks"] = peaks
    if not args.no_ext:
        reps, wu = max(10, args.steps // 2), max(3, args.warmup // 2)
        cfg = [measure_config(fa, torch, dev, TINY_FWD, reps, wu, index, peaks),
               measure_config(fa, torch, dev, FWD_2K, reps, wu, index, peaks),
               by_entry["fa_fwd"],
               measure_config(fa, torch, dev, BWD_4K, reps, wu, index, peaks),
               by_entry["fa_decode"],
               dict(by_entry["fa_bwd"], note="supplementary: the backward at the N=8192 shape")]
        out["configs"] = cfg
        out["extensions"] = measure_extensions(fa, torch, dev, reps, wu, index, peaks)
    if not args.no_cpu_baseline:
        import oracle
        out["host"] = host_info(oracle.max_threads())
        out["cpu_baseline"] = cpu_baseline_step(q, k, v, do, args.cpu_heads, w.scale)
        cb = cpu_baselines_configs(dev, (q, k, v, do), (qd, kd, vd))
        out["cpu_baselines"] = cb
        if "configs" in out:
            by_wl = {c["workload"]: c for c in cb}
            for c in out["configs"]:
                o_ = by_wl.get(c["workload"])
                if o_ is not None:
                    c["oracle"] = {"value": o_["value"], "unit": o_["unit"], "secs": o_["secs"],
                                   "sample": o_["sample"]}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
