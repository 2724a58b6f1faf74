"""The algorithmic work counts behind the benchmark's roofline fractions.

FLOP = 4 * head_dim * q_heads * (number of unmasked query-key pairs); bytes
= Q + O + the K/V rows some query attends + sinks + offsets.  The pair count
is checked by enumeration of the mask (causal, optional window of W keys
including the query itself: the 128-token sliding-window layers of NVIDIA's
gpt-oss Blackwell announcement, model-description paragraph), the totals
against the figures these formulas give at the benchmark shapes.
"""

import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("length", [1, 2, 5, 127, 128, 129, 300])
@pytest.mark.parametrize("window", [0, 1, 2, 127, 128, 129, 400])
def test_visible_pairs_enumeration(length, window):
    b = _bench()
    brute = sum(1 for i in range(length) for j in range(i + 1) if window <= 0 or j > i - window)
    assert b.visible_pairs(length, window) == brute


def test_step_counts():
    b = _bench()
    # causal 8192: 8192 * 8193 / 2 pairs x 4 x 64 x 64
    assert b.prefill_flops([8192], 0) == 4 * 64 * 64 * (8192 * 8193 // 2)
    assert abs(b.prefill_flops([8192], 0) - 5.498e11) / 5.498e11 < 1e-3
    # window 128: 128 pairs for every query from 127 on, i + 1 before
    assert b.prefill_flops([8192], 128) == 4 * 64 * 64 * (128 * 8192 - 128 * 127 // 2)
    # Q + O: 2 x 8192 x 64 x 64 x 2 B; K + V: 2 x 8192 x 8 x 64 x 2 B
    assert b.prefill_bytes([8192], 0) == 2 * 8192 * 64 * 64 * 2 + 2 * 8192 * 8 * 64 * 2 + 64 * 4 + 2 * 4
    # decode 64 x 8192: the whole KV cache (1 GiB) plus Q and O
    kv = 2 * 64 * 8192 * 8 * 64 * 2
    assert kv == 1 << 30
    assert b.decode_bytes([8192] * 64, 0) == kv + 2 * 64 * 64 * 64 * 2 + 64 * 4 + 65 * 4
    # decode with a 128 window reads only the last 128 keys of each sequence
    assert b.decode_bytes([32768] * 16, 128) == 2 * 16 * 128 * 8 * 64 * 2 + 2 * 16 * 64 * 64 * 2 + 64 * 4 + 17 * 4
    assert b.decode_flops([32768] * 16, 128) == 4 * 64 * 64 * 16 * 128
    # short sequences under a window read all their keys
    assert b.decode_bytes([100], 128) == b.decode_bytes([100], 0)


def test_tiny_counts():
    b = _bench()
    assert b.prefill_flops([256], 0, hq=4) == 4 * 64 * 4 * (256 * 257 // 2)
    assert b.prefill_bytes([256], 0, 4, 1) == 2 * 256 * 4 * 64 * 2 + 2 * 256 * 64 * 2 + 4 * 4 + 2 * 4


def test_gpus_above_one_exits():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


@pytest.mark.parametrize("q_len,k_len", [(1, 1), (1, 9), (3, 9), (9, 9), (5, 300), (0, 7)])
@pytest.mark.parametrize("window", [0, 1, 4, 128])
def test_append_counts_by_enumeration(q_len, k_len, window):
    """Append pairs and attended K/V rows (bottom-right causal) by brute force."""
    b = _bench()
    pos = range(k_len - q_len, k_len)
    brute = sum(1 for p in pos for j in range(p + 1) if window <= 0 or j > p - window)
    assert b.append_pairs(q_len, k_len, window) == brute
    rows = {j for p in pos for j in range(p + 1) if window <= 0 or j > p - window}
    expect = 2 * q_len * 64 * 64 * 2 + 2 * len(rows) * 8 * 64 * 2 + 64 * 4 + 2 * 2 * 4
    assert b.append_bytes([q_len], [k_len], window) == expect


def _fake_full_record(b, n_others):
    """A full benchmark record with the structure gpu_bench and main build,
    filled with placeholder numbers (only the line's length is tested)."""
    st = {"median_ms": 0.123456789, "min_ms": 0.1111111, "mean_ms": 0.12345678, "max_ms": 0.2, "reps": 20}
    entry = dict(st, algorithmic_bytes=1.0748e9, gbs_median=6000.123456, gbs_best=6500.98765,
                 pct_hbm_peak=75.0123456, pct_mfma_peak=40.0123456, bound="hbm", shape="x" * 100)
    roof = {"kernel": "prefill_kernel (causal, L=8192, 64/8 heads)", "bound": "mfma", "achieved": 1234.56789,
            "peak": 2516.6, "unit": "TFLOP/s", "frac": 0.49056789, "traffic": 159465195.05569646,
            "ms": 0.558030778169632, "algorithmic_flop": 549822922752.0}
    splits = {k: dict(entry) for k in ("1", "4", "16")}
    return {
        "metric": b.METRIC, "value": 58.123456789, "unit": "% of MI355X peak (mean of prefill bf16-MFMA and "
        "decode HBM fractions)", "n_gpus": 1, "steps": 50, "warmup": 1000, "ms_per_step": 0.812345678,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) Q/K/V rounded to bf16, N(0,1) fp32 sinks",
        "config": {"workload": "w" * 220, "prefill": {}, "decode": {}},
        "prefill": {"causal_timing": st, "window_timing": st, "causal_tflops": 1234.5678, "window_gbs": 3456.789},
        "decode": {"timing": st, "gbs": 6000.1234, "by_splits": splits, "fp8_kv_by_splits": splits},
        "roofline": roof, "rooflines": [roof, roof, roof],
        "cpu_baseline": {"value": 0.0123456, "unit": "% of MI355X peak (same formula as value)", "cores": 16,
                         "affinity_cores": 128, "kind": "oracle", "sample": "s" * 300, "sample_short": "s" * 100,
                         "prefill_seconds": 12.3456, "prefill_tflops_f64": 0.0456789, "decode_seconds": 3.456789,
                         "decode_gbs_f64": 0.3456789, "other_configs": {"x": {"seconds": 1.0}}},
        "other_configs": {"workload_name_of_this_lengt_%02d_w128" % i: dict(entry) for i in range(n_others)},
        "bandwidth_reference": {"read": dict(st)}, "engine_clock": {"mhz_median": 2100, "samples": 40},
        "device": {"name": "AMD Instinct MI355X"},
    }


def test_compact_line_fits_a_short_log_tail():
    """The last stdout line carries the headline, the rooflines and the CPU
    baseline in a few KB (a long line loses its head in a short log tail),
    with every side workload named; here 46 side workloads (the benchmark has
    43) with names of 35 characters (the benchmark's average is 33)."""
    import json
    b = _bench()
    full = _fake_full_record(b, 46)
    line = json.dumps(b.compact_record(full, "gpurun_out/bench_detail.json"), separators=(",", ":"))
    assert len(line) < 4096, len(line)
    rec = json.loads(line)
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "dtype", "config",
                "roofline", "rooflines", "cpu_baseline", "legs"):
        assert rec[key] is not None, key
    assert set(rec["roofline"]) >= {"bound", "achieved", "peak", "unit", "frac", "traffic"}
    assert rec["cpu_baseline"]["cores"] == 16 and rec["cpu_baseline"]["affinity_cores"] == 128
    assert len(rec["other_pct_of_peak"]) == 46 and len(rec["rooflines"]) == 2
