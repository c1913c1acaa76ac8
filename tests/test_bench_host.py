"""Host-side checks of bench.py's measurement bookkeeping (CPU only).

bench.py reads per-workload rocprofv3 figures (HBM bytes, clock, MFMA busy) from the committed
profiles/roofline_index.txt and keeps them only while the kernel sources are unchanged since the
counters were taken.  These tests pin that bookkeeping without a GPU:
  * every index line names a known entry point and an existing profile summary that carries
    the same source hash, and its traffic ratio is its HBM bytes over its algorithmic bytes;
  * the algorithmic bytes equal the tensor sizes each workload reads and writes once
    (Q, K, V, O and lse for a forward; also dO, dQ, dK, dV for a backward; K, V, q and o for a
    decode), recomputed here from the workload definitions;
  * the FLOP and byte formulas bench.py reports against match their closed forms;
  * the roofline arithmetic (mean, median, minimum, measured and clock-scaled peaks) and the
    source-hash gate.
"""
import os

import pytest

import bench
from synth_inputs import (BWD_4K, DECODE_16K, FWD_2K, FWD_8K, GQA_DECODE_16K, TINY_FWD,
                          WINDOW_FWD_8K, ragged_lengths)

PROFILES = os.path.join(os.path.dirname(bench.INDEX_FILE))


def index_rows():
    """Every line of the committed index, without the source-hash gate."""
    rows = []
    for line in open(bench.INDEX_FILE):
        line = line.split("#", 1)[0].strip()
        if line:
            rows.append(dict(tok.split("=", 1) for tok in line.split() if "=" in tok))
    return rows


def _bytes_fwd(w):
    elems = w.B * w.H * w.N * w.d
    return 4 * elems * 2 + w.B * w.H * w.N * 4          # Q, K, V, O in bf16/fp16; lse in fp32


def _bytes_bwd(w):
    elems = w.B * w.H * w.N * w.d
    return 8 * elems * 2 + w.B * w.H * w.N * 4          # Q, K, V, O, dO, dQ, dK, dV; lse


def _bytes_decode(w, keys_per_head):
    hkv = w.Hkv or w.H
    return (2 * hkv * keys_per_head * w.d + 2 * w.B * w.H * w.d) * 2   # K, V; q, o


def test_index_lines_name_known_entries_and_matching_profiles():
    rows = index_rows()
    assert len(rows) >= 9
    for r in rows:
        assert r["entry"] in bench.FAMILY, r["entry"]
        path = os.path.join(PROFILES, r["profile"])
        assert os.path.exists(path), path
        text = open(path).read()
        assert r["workload"] in text
        assert r["source_sha256"] in text
        hbm, alg = float(r["hbm_bytes"]), float(r["algorithmic_bytes"])
        assert abs(float(r["ratio"]) - hbm / alg) < 1e-3
        assert float(r["kernel_us"]) > 0


def test_algorithmic_bytes_are_the_tensor_sizes():
    lens = ragged_lengths(GQA_DECODE_16K.B, GQA_DECODE_16K.Nkv, GQA_DECODE_16K.seed)
    expected = {
        (FWD_8K.name, "fa_fwd"): _bytes_fwd(FWD_8K),
        (bench.BWD_8K_NAME, "fa_bwd"): _bytes_bwd(FWD_8K),
        (DECODE_16K.name, "fa_decode"): _bytes_decode(DECODE_16K, DECODE_16K.B * DECODE_16K.Nkv),
        (TINY_FWD.name, "fa_fwd"): _bytes_fwd(TINY_FWD),
        (FWD_2K.name, "fa_fwd"): _bytes_fwd(FWD_2K),
        (BWD_4K.name, "fa_bwd"): _bytes_bwd(BWD_4K),
        (WINDOW_FWD_8K.name, "fa_fwd_ex"): _bytes_fwd(WINDOW_FWD_8K),
        (GQA_DECODE_16K.name, "fa_decode_ex"):
            _bytes_decode(GQA_DECODE_16K, GQA_DECODE_16K.B * GQA_DECODE_16K.Nkv),
        (GQA_DECODE_16K.name + "_ragged", "fa_decode_varlen"):
            _bytes_decode(GQA_DECODE_16K, int(lens.sum())),
    }
    got = {(r["workload"], r["entry"]): int(r["algorithmic_bytes"]) for r in index_rows()}
    assert set(expected) <= set(got), set(expected) - set(got)
    for key, val in expected.items():
        assert got[key] == val, (key, got[key], val)
    # The decode's bytes as bench.py reports them (every history full).
    assert bench.decode_bytes(DECODE_16K) == expected[(DECODE_16K.name, "fa_decode")]
    assert bench.decode_bytes(GQA_DECODE_16K) == expected[(GQA_DECODE_16K.name, "fa_decode_ex")]


def test_flop_formulas():
    # 4 B H N^2 d (forward) and 10 B H N^2 d (backward: five N x N x d products), halved when causal.
    assert bench.fwd_flops(FWD_8K) == 4 * 1 * 32 * 128 * 8192 * 8192 / 2
    assert bench.bwd_flops(FWD_8K) == 2.5 * bench.fwd_flops(FWD_8K)
    assert bench.fwd_flops(TINY_FWD) == 4 * 1 * 1 * 64 * 256 * 256       # non-causal
    assert bench.bwd_flops(BWD_4K) == 10 * 2 * 16 * 128 * 4096 * 4096 / 2


def test_roofline_arithmetic():
    idx = {("w", "fa_fwd"): {"hbm_bytes": "1000", "ratio": "2.0", "kernel_us": "1500.0",
                             "clock_ghz": "1.8", "mfma_busy": "0.5"}}
    peaks = {"mfma": {"tflops": 2000.0}, "read": {"gbs": 7000.0}}
    r = bench.roofline("w", "fa_fwd", "mfma", 1e12, [1.0, 2.0, 3.0], idx, peaks)
    assert r["ms"] == 2.0 and r["ms_median"] == 2.0 and r["ms_min"] == 1.0
    assert r["achieved"] == 500.0 and r["frac"] == 0.2
    assert r["achieved_at_median"] == 500.0 and r["achieved_at_min"] == 1000.0
    assert r["peak_measured"] == 2000.0 and r["frac_measured"] == 0.25
    assert r["traffic"] == 1000.0 and r["traffic_ratio"] == 2.0 and r["profiled_ms"] == 1.5
    # without a probe clock the published peak is scaled to the profiled clock ...
    assert r["clock_ghz"] == 1.8 and r["peak_at_clock"] == 1875.0
    assert r["frac_at_clock"] == round(500.0 / 1875.0, 4) and r["mfma_busy"] == 0.5
    assert r["clock_for_peak"] == {"ghz": 1.8, "source": "profile"}
    # ... and with one, to the clock the probe measured in the same run
    peaks_clk = {"mfma": {"tflops": 2000.0, "clock_ghz": 1.92}, "read": {"gbs": 7000.0}}
    r = bench.roofline("w", "fa_fwd", "mfma", 1e12, [2.0], idx, peaks_clk)
    assert r["peak_at_clock"] == 2000.0 and r["frac_at_clock"] == 0.25
    assert r["clock_for_peak"] == {"ghz": 1.92, "source": "probe, this run"} and r["clock_ghz"] == 1.8
    # an HBM-bound entry against the measured read ceiling; no profile figures without an index
    r = bench.roofline("d", "fa_decode", "hbm", 8e9, [2.0], {}, peaks)
    assert r["achieved"] == 4000.0 and r["frac"] == 0.5 and r["frac_measured"] == round(4 / 7, 4)
    assert r["traffic"] is None and r["clock_ghz"] is None and "peak_at_clock" not in r


def test_profile_index_keeps_only_unchanged_sources(tmp_path, monkeypatch):
    good, stale = bench.source_sha("fwd"), "0" * 16
    f = tmp_path / "index.txt"
    f.write_text("# comment line\n"
                 f"workload=a entry=fa_fwd kernel_us=1 hbm_bytes=2 source_sha256={good}\n"
                 f"workload=b entry=fa_fwd kernel_us=1 hbm_bytes=2 source_sha256={stale}\n"
                 f"workload=c entry=unknown kernel_us=1 source_sha256={good}\n")
    monkeypatch.setattr(bench, "INDEX_FILE", str(f))
    idx = bench.profile_index()
    assert set(idx) == {("a", "fa_fwd")}
    monkeypatch.setattr(bench, "INDEX_FILE", str(tmp_path / "missing.txt"))
    assert bench.profile_index() == {}


@pytest.mark.parametrize("family", sorted(bench.KERNEL_SOURCES))
def test_source_hash_covers_existing_files(family):
    for name in bench.KERNEL_SOURCES[family]:
        assert os.path.exists(os.path.join(bench.CSRC, name)), name
    assert len(bench.source_sha(family)) == 16
