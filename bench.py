"""Benchmark of the sink-attention hot path on one MI355X.

One step = one pass of the whole path over one batch of seeded synthetic
input with GPT-OSS attention shapes (64 query heads, 8 KV heads, head_dim
64, scale 1/8):
  * prefill, batch 1 x 8192 tokens: the causal full-context layer and the
    128-token sliding-window layer (varlen entry point, cu_seqlens);
  * split-KV decode, batch 64 x 8192 cached tokens, 16 splits, including
    the log-sum-exp merge.

Printed: ONE compact JSON line (a few KB; the full record with every
statistic goes to --detail-json, gpurun_out/bench_detail.json by default).
`value` is the mean of the two roofline fractions
(prefill FLOP/s over the bf16 MFMA peak, decode KV bytes/s over the HBM
peak) in percent; each leg is also reported on its own.  FLOP and byte
counts are algorithmic (unmasked query-key pairs; Q + O + the K/V rows
attended + sinks), measured with HIP events on the stream the kernels run
on; `value` uses each leg's mean interval, the rooflines its median.  Inputs are resident in HBM before timing; the prefill leg rotates three
input sets so that its 151 MB working set does not stay in the 256 MB
Infinity Cache between steps.  Each leg reports mean, median and min.

Also reported (not part of the step or of `value`): decode at 1, 4 and 16
splits, also against an FP8 (E4M3) cache with per-tensor scales; the tiny 256-token prefill; the long-context decode pair (16 x 32768
cached tokens, 32 splits, full then 128-window); the ragged 32-sequence
varlen prefill (causal and 128-window); the append prefill (the last
2048-token chunk of an 8192-token prompt; 64 x 4 draft tokens verified
against 8192 cached tokens, also through the multi-token-query decode at 1
and 4 splits; 8 draft tokens per sequence, and 4 or 8 against an E4M3
cache, through the multi-token decode alone); the 64 x 8192 decode against a paged cache (16- and 64-token
pages, shuffled), also with 4 draft tokens per sequence, over E4M3 pages, and
as the keys of a 2048-token prompt chunk (append prefill over pages); the fused rotary step (YaRN; Q out, K/V appended) for 8192
and 64 tokens; the output projection with bias (64 and 8192 rows, 4096 ->
2880); a streaming-read and a copy
bandwidth reference; the engine clock (sysfs pp_dpm_sclk) sampled during the warm-up and timed steps.
Small working sets are timed after a 512 MiB cache scrub.  The long-decode
and ragged inputs are drawn on the device from a seeded generator (same
distributions as the host-generated parity inputs) to keep start-up short.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extras]
                    [--detail-json PATH]
"""

from __future__ import annotations

import argparse
import gc
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sink-attn prefill TFLOP/s + decode KV GB/s, as % of MI355X peak (1 GPU)"
PEAK_BF16_TFLOPS = 2516.6     # 256 CU x 4096 flop/clk x 2.4 GHz (dense)
PEAK_HBM_GBS = 8000.0         # HBM3E

HQ, HKV, D = 64, 8, 64
PREFILL_LEN = 8192
WINDOW = 128
DEC_BATCH, DEC_CTX, DEC_SPLITS = 64, 8192, 16


# ---------------------------------------------------------------------------
# Algorithmic work counts
# ---------------------------------------------------------------------------

def visible_pairs(length: int, window: int) -> int:
    """Sum over queries i < length of |J(i)| (causal, optional window)."""
    if window <= 0 or window >= length:
        return length * (length + 1) // 2
    return window * length - window * (window - 1) // 2


def prefill_flops(lengths, window, hq=HQ) -> float:
    return 4.0 * D * hq * sum(visible_pairs(n, window) for n in lengths)


def prefill_bytes(lengths, window, hq=HQ, hkv=HKV) -> float:
    t = sum(lengths)
    qo = 2 * t * hq * D * 2
    kv = 2 * t * hkv * D * 2          # every key is attended by some query
    return float(qo + kv + hq * 4 + (len(lengths) + 1) * 4)


def decode_bytes(lengths, window, hq=HQ, hkv=HKV, kv_elem_bytes=2) -> float:
    """Q + O (bf16) + the K/V rows attended (kv_elem_bytes per element: 2 for
    bf16, 1 for an E4M3 cache) + sinks + offsets."""
    keys = sum(min(n, window) if window > 0 else n for n in lengths)
    return float(2 * len(lengths) * hq * D * 2 + 2 * keys * hkv * D * kv_elem_bytes + hq * 4
                 + (len(lengths) + 1) * 4)


def append_pairs(q_len: int, k_len: int, window: int) -> int:
    """Sum of |J(p)| over the query positions p = k_len - q_len .. k_len - 1
    (bottom-right causal, optional window)."""
    def upto(n):  # sum over p < n of |J(p)|
        return visible_pairs(n, window) if n > 0 else 0
    return upto(k_len) - upto(k_len - q_len)


def append_flops(q_lens, k_lens, window, hq=HQ) -> float:
    return 4.0 * D * hq * sum(append_pairs(a, b, window) for a, b in zip(q_lens, k_lens))


def append_bytes(q_lens, k_lens, window, hq=HQ, hkv=HKV) -> float:
    """Q + O + every K/V row some query sees + sinks + both offset arrays."""
    keys = 0
    for a, b in zip(q_lens, k_lens):
        first = max(0, b - a - window + 1) if window > 0 else 0
        keys += b - first if a > 0 else 0
    tq = sum(q_lens)
    return float(2 * tq * hq * D * 2 + 2 * keys * hkv * D * 2 + hq * 4 + 2 * (len(q_lens) + 1) * 4)


def rope_bytes(num_tokens: int, hq=HQ, hkv=HKV) -> float:
    """Fused rotary step: read qkv, positions and slots; write q, k and v."""
    row = D * 2
    return float(num_tokens * ((hq + 2 * hkv) * row * 2 + 8))


OPROJ_OUT = 2880  # synthetic output width of the projection


def oproj_bytes(num_rows: int, out_features: int = OPROJ_OUT, hq=HQ) -> float:
    """Output projection: o and W read once, y written, bias read."""
    k = hq * D
    return float(2 * (num_rows * k + out_features * k + num_rows * out_features) + 4 * out_features)


def decode_flops(lengths, window, hq=HQ) -> float:
    keys = sum(min(n, window) if window > 0 else n for n in lengths)
    return 4.0 * D * hq * keys


# ---------------------------------------------------------------------------
# CPU baseline: the oracle, timed on a bounded sample of the same workload
# ---------------------------------------------------------------------------

def _decode_one(args):
    from oracle import decode_ref
    q, k, v, sinks, length, scale = args
    return decode_ref(q, k, v, [0, length], sinks, 0, scale)


def affinity_cores() -> int:
    """Host cores this process may run on (its affinity mask)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _stop_process_helpers() -> None:
    """End the helper process that spawned pools leave behind (the
    multiprocessing resource tracker), so nothing outlives the benchmark."""
    try:
        from multiprocessing import resource_tracker
        resource_tracker._resource_tracker._stop()
    except Exception:  # pragma: no cover - private API, best effort
        pass


def cpu_baseline() -> dict:
    import multiprocessing as mp

    import numpy as np

    from attention_gqa_flash_amd import inputs
    from oracle import prefill_varlen_ref
    from oracle.sink_attention import _pool_init, default_workers

    cores = default_workers()
    # prefill leg: the whole 8192-token prefill step (causal layer and
    # 128-window layer, all 64 heads) on `cores` spawned processes
    p = inputs.gptoss_prefill(seed=0, length=PREFILL_LEN)
    qf, kf, vf = (inputs.bf16_bits_to_f32(x) for x in (p.q, p.k, p.v))
    t0 = time.perf_counter()
    for window in (0, WINDOW):
        prefill_varlen_ref(qf, kf, vf, p.sinks, p.cu_seqlens, window, p.scale, workers=cores)
    t_pre = time.perf_counter() - t0
    pre_flops = prefill_flops([PREFILL_LEN], 0) + prefill_flops([PREFILL_LEN], WINDOW)
    pre_tflops = pre_flops / t_pre / 1e12
    del qf, kf, vf, p

    # decode leg: the whole decode batch (64 sequences x 8192 keys), one
    # sequence per task
    d = inputs.make_decode([DEC_CTX] * DEC_BATCH, HQ, HKV, D, seed=0)
    qf, kf, vf = (inputs.bf16_bits_to_f32(x) for x in (d.q, d.k, d.v))
    tasks = [(qf[b:b + 1], kf[b * DEC_CTX:(b + 1) * DEC_CTX], vf[b * DEC_CTX:(b + 1) * DEC_CTX], d.sinks, DEC_CTX,
              d.scale) for b in range(DEC_BATCH)]
    ctx = mp.get_context("spawn")
    pool = ctx.Pool(processes=cores, initializer=_pool_init)
    try:
        pool.map(_decode_one, tasks[:cores], chunksize=1)  # start-up outside the timing
        t0 = time.perf_counter()
        pool.map(_decode_one, tasks, chunksize=1)
        t_dec = time.perf_counter() - t0
    finally:
        pool.close()
        pool.join()
    dec_gbs = decode_bytes([DEC_CTX] * DEC_BATCH, 0) / t_dec / 1e9
    value = 100.0 * 0.5 * (pre_tflops / PEAK_BF16_TFLOPS + dec_gbs / PEAK_HBM_GBS)
    others = _cpu_other_configs(cores)
    _stop_process_helpers()
    return {
        "value": value, "unit": "% of MI355X peak (same formula as value)", "cores": cores,
        "affinity_cores": affinity_cores(), "kind": "oracle",
        "sample": "one whole step: prefill 1 x 8192 tokens (causal + 128-window layers) and decode 64 x 8192 "
                  "keys, 64/8 heads, on %d spawned processes with 1 BLAS thread each (pool start-up included "
                  "for prefill, excluded for decode)" % cores,
        "sample_short": "whole step (prefill 1 x 8192 causal + w128, decode 64 x 8192), %d processes" % cores,
        "prefill_tflops_f64": pre_tflops, "prefill_seconds": t_pre,
        "decode_gbs_f64": dec_gbs, "decode_seconds": t_dec,
        "other_configs": others,
    }


def _cpu_other_configs(cores: int) -> dict:
    """The oracle on the other workloads, each on a bounded sample: the whole
    tiny prefill; 2 of the 16 long-decode sequences (both layers); for the
    ragged prefill, 3 of its sequences (the longest, a middle and a short
    one; all rows of the two shorter, 256 evenly spaced rows of the
    longest), both layers; 2 of the 64 decode sequences against the E4M3 and
    the paged cache; 256 query rows of the 2048-token append chunk (both
    layers); 2 of the 64 draft-token sequences; 1024 of the 8192 tokens of
    the fused rotary step; the whole 64-row output projection.  Rates are float64 GFLOP/s (or GB/s of the
    algorithmic bytes); `seconds_full` extrapolates to the whole workload."""
    import numpy as np

    from attention_gqa_flash_amd import inputs
    from oracle import decode_ref, prefill_varlen_ref

    out = {}
    p = inputs.tiny_prefill(seed=0)
    qf, kf, vf = (inputs.bf16_bits_to_f32(x) for x in (p.q, p.k, p.v))
    t0 = time.perf_counter()
    prefill_varlen_ref(qf, kf, vf, p.sinks, p.cu_seqlens, 0, p.scale)
    t = time.perf_counter() - t0
    f = prefill_flops([256], 0, hq=4)
    out["tiny_prefill_causal"] = {"seconds": t, "gflops_f64": f / t / 1e9, "sample": "whole workload, 1 process"}

    d = inputs.make_decode([32768] * 2, HQ, HKV, D, seed=0, sink_std=math.sqrt(2.0))
    qf, kf, vf = (inputs.bf16_bits_to_f32(x) for x in (d.q, d.k, d.v))
    for window in (0, WINDOW):
        t0 = time.perf_counter()
        decode_ref(qf, kf, vf, d.cu_seqlens_k, d.sinks, window, d.scale)
        t = time.perf_counter() - t0
        b = decode_bytes([32768] * 2, window)
        out["long_decode_%s" % ("full" if window == 0 else "w128")] = {
            "seconds": t, "gbs_f64": b / t / 1e9, "seconds_full": t * 8,
            "sample": "2 of 16 sequences x 32768 keys, 1 process"}

    lengths = sorted(inputs.ragged_lengths(np.random.default_rng(0), 32))
    pick = [lengths[-1], lengths[len(lengths) // 2], lengths[4]]
    p = inputs.make_prefill(pick, HQ, HKV, D, seed=0)
    qf, kf, vf = (inputs.bf16_bits_to_f32(x) for x in (p.q, p.k, p.v))
    rows = list(np.linspace(0, pick[0] - 1, 256).astype(np.int64)) + list(range(pick[0], sum(pick)))
    total_causal = prefill_flops(lengths, 0)
    total_window = prefill_flops(lengths, WINDOW)
    for window, total in ((0, total_causal), (WINDOW, total_window)):
        # flop of exactly the sampled rows
        fl = 0.0
        for r in rows:
            seq = 0 if r < pick[0] else (1 if r < pick[0] + pick[1] else 2)
            i = r - sum(pick[:seq])
            fl += 4.0 * D * HQ * (min(i + 1, window) if window > 0 else i + 1)
        t0 = time.perf_counter()
        prefill_varlen_ref(qf, kf, vf, p.sinks, p.cu_seqlens, window, p.scale, rows=rows, workers=cores)
        t = time.perf_counter() - t0
        out["ragged_prefill_%s" % ("causal" if window == 0 else "w128")] = {
            "seconds": t, "gflops_f64": fl / t / 1e9, "seconds_full": total / (fl / t),
            "sample": "%d rows of sequences of %s tokens, %d processes (pool start-up included)"
                      % (len(rows), pick, cores)}

    from oracle import decode_fp8_ref, decode_paged_ref, prefill_append_ref

    # FP8 (E4M3) decode and paged decode: 2 of the 64 sequences x 8192 keys
    f8 = inputs.make_decode_fp8([DEC_CTX] * 2, HQ, HKV, D, seed=0)
    t0 = time.perf_counter()
    decode_fp8_ref(inputs.bf16_bits_to_f32(f8.q), f8.k, f8.v, f8.k_scale, f8.v_scale, f8.cu_seqlens_k, f8.sinks, 0,
                   f8.scale)
    t = time.perf_counter() - t0
    out["fp8_decode"] = {"seconds": t, "gbs_f64": decode_bytes([DEC_CTX] * 2, 0, kv_elem_bytes=1) / t / 1e9,
                         "seconds_full": t * DEC_BATCH / 2, "sample": "2 of 64 sequences x 8192 keys, 1 process"}
    pg = inputs.make_paged_decode([DEC_CTX] * 2, 16, HQ, HKV, D, seed=0)
    kp, vp = inputs.bf16_bits_to_f32(pg.k_pages), inputs.bf16_bits_to_f32(pg.v_pages)
    t0 = time.perf_counter()
    decode_paged_ref(inputs.bf16_bits_to_f32(pg.q), kp, vp, pg.block_table, pg.seq_lens, 16, pg.sinks, 0, pg.scale)
    t = time.perf_counter() - t0
    out["paged_decode_ps16"] = {"seconds": t, "gbs_f64": decode_bytes([DEC_CTX] * 2, 0) / t / 1e9,
                                "seconds_full": t * DEC_BATCH / 2,
                                "sample": "2 of 64 sequences x 8192 keys, 16-token pages, 1 process"}
    del kp, vp

    # append prefill (last 2048 of 8192 tokens): 256 evenly spaced query rows;
    # draft verification: 2 of the 64 sequences x 4 queries x 8192 keys
    a = inputs.make_append([2048], [8192], HQ, HKV, D, seed=0)
    qf, kf, vf = (inputs.bf16_bits_to_f32(x) for x in (a.q, a.k, a.v))
    rows = list(np.linspace(0, 2047, 256).astype(np.int64))
    for window in (0, WINDOW):
        fl = sum(4.0 * D * HQ * (min(6144 + r + 1, window) if window > 0 else 6144 + r + 1) for r in rows)
        t0 = time.perf_counter()
        prefill_append_ref(qf, kf, vf, a.sinks, a.cu_seqlens_q, a.cu_seqlens_k, window, a.scale, rows=rows)
        t = time.perf_counter() - t0
        total = append_flops([2048], [8192], window)
        out["chunked_prefill_last_2048_of_8192_%s" % ("causal" if window == 0 else "w128")] = {
            "seconds": t, "gflops_f64": fl / t / 1e9, "seconds_full": total / (fl / t),
            "sample": "256 of 2048 query rows, 1 process"}
    a = inputs.make_append([4, 4], [DEC_CTX] * 2, HQ, HKV, D, seed=0)
    qf, kf, vf = (inputs.bf16_bits_to_f32(x) for x in (a.q, a.k, a.v))
    t0 = time.perf_counter()
    prefill_append_ref(qf, kf, vf, a.sinks, a.cu_seqlens_q, a.cu_seqlens_k, 0, a.scale)
    t = time.perf_counter() - t0
    # fused rotary step: 1024 of the 8192 prefill tokens
    from oracle import rope_qkv_append_ref, yarn_inv_freq_ref
    r = inputs.make_rope(1024, HQ, HKV, cache_rows=2048, seed=0)
    t0 = time.perf_counter()
    f_rope, m_rope = yarn_inv_freq_ref(D, 150000.0, 32.0, 4096, 32.0, 1.0)
    rope_qkv_append_ref(inputs.bf16_bits_to_f32(r.qkv), r.positions, HQ, HKV, f_rope, m_rope, r.slot_mapping,
                        inputs.bf16_bits_to_f32(r.k_cache), inputs.bf16_bits_to_f32(r.v_cache))
    t = time.perf_counter() - t0
    out["rope_qkv_append_8192"] = {"seconds": t, "gbs_f64": rope_bytes(1024) / t / 1e9, "seconds_full": t * 8,
                                   "sample": "1024 of 8192 tokens (cache copies included), 1 process"}
    # output projection with bias: the 64 rows of a decode step (whole)
    from oracle import oproj_ref
    rng = np.random.default_rng(0)
    o_rows = inputs.bf16_bits_to_f32(inputs.round_to_bf16_bits(rng.standard_normal((DEC_BATCH, HQ * D),
                                                                                   dtype=np.float32)))
    w_rows = inputs.bf16_bits_to_f32(inputs.round_to_bf16_bits(
        (rng.standard_normal((OPROJ_OUT, HQ * D)) / math.sqrt(HQ * D)).astype(np.float32)))
    t0 = time.perf_counter()
    oproj_ref(o_rows, w_rows, rng.standard_normal(OPROJ_OUT))
    t = time.perf_counter() - t0
    out["oproj_bias_64"] = {"seconds": t, "gbs_f64": oproj_bytes(DEC_BATCH) / t / 1e9,
                            "gflops_f64": 2.0 * DEC_BATCH * HQ * D * OPROJ_OUT / t / 1e9,
                            "sample": "whole workload (64 rows), 1 process"}
    out["draft_verify_64x4_ctx8192_causal"] = {
        "seconds": t, "gbs_f64": append_bytes([4, 4], [DEC_CTX] * 2, 0) / t / 1e9, "seconds_full": t * DEC_BATCH / 2,
        "sample": "2 of 64 sequences x 4 queries x 8192 keys, 1 process"}
    return out


# ---------------------------------------------------------------------------
# GPU leg
# ---------------------------------------------------------------------------

# The sources each counted kernel is built from (its own file and the shared
# device helpers).
_KERNEL_SOURCES = {"prefill": ("prefill.hip", "device_common.hpp"), "decode": ("decode.hip", "device_common.hpp"),
                   "merge": ("decode.hip", "device_common.hpp"), "oproj": ("oproj.hip", "device_common.hpp"),
                   "rope": ("rope.hip", "device_common.hpp")}


def _code_only(text: str) -> str:
    """Source text without its // comments, trailing blanks and empty lines:
    what a comment-only edit leaves unchanged."""
    lines = []
    for line in text.splitlines():
        cut = line.find("//")
        if cut >= 0 and line.count('"', 0, cut) % 2 == 0:  # not inside a string literal
            line = line[:cut]
        line = line.rstrip()
        if line:
            lines.append(line)
    return "\n".join(lines)


def kernel_source_hash(kernel: str) -> str:
    """Hash of the code (comments aside) of the sources of one counted kernel
    ('prefill_causal', 'decode_s16', ...)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "attention_gqa_flash_amd", "csrc")
    for name in _KERNEL_SOURCES[kernel.split("_")[0]]:
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode() + _code_only(f.read()).encode())
    return h.hexdigest()[:16]


def _traffic(kernel: str):
    """Measured HBM bytes per launch from the committed counter summary, if it
    was taken on the current sources of that kernel; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    ent = data.get(kernel)
    if not ent or ent.get("source_hash") != kernel_source_hash(kernel):
        return None
    return ent.get("bytes_per_launch")


class _ClockSampler:
    """Samples the engine clock of the GPU under test on a host thread while
    kernels run: the current level of sysfs pp_dpm_sclk (the line marked
    '*'), plus the hwmon power reading where present.  Best effort: None
    where the files are missing or unreadable."""

    def __init__(self, pci_bus: str):
        import glob
        cards = []
        for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
            if os.path.exists(os.path.join(dev, "pp_dpm_sclk")):
                cards.append(dev)
        match = [d for d in cards if os.path.realpath(d).lower().endswith(pci_bus.lower())]
        dev = match[0] if match else (cards[0] if len(cards) == 1 else None)
        self.sclk = os.path.join(dev, "pp_dpm_sclk") if dev else None
        power = sorted(glob.glob(os.path.join(dev, "hwmon", "hwmon*", "power1_input"))) if dev else []
        self.power = power[0] if power else None
        self.mhz, self.watts = [], []
        self._stop = None
        self._thread = None

    @staticmethod
    def _read(path):
        try:
            with open(path) as f:
                return f.read()
        except OSError:
            return None

    def _sample(self):
        text = self._read(self.sclk)
        if text:
            for line in text.splitlines():
                if line.rstrip().endswith("*"):
                    digits = "".join(ch for ch in line.split(":", 1)[-1] if ch.isdigit())
                    if digits:
                        self.mhz.append(int(digits))
        if self.power:
            text = self._read(self.power)
            if text and text.strip().isdigit():
                self.watts.append(int(text.strip()) / 1e6)

    def __enter__(self):
        import threading
        if self.sclk is None:
            return self
        self._stop = threading.Event()

        def run():
            while not self._stop.is_set():
                self._sample()
                self._stop.wait(0.02)

        self._thread = threading.Thread(target=run, daemon=True)
        self._thread.start()
        return self

    def __exit__(self, *exc):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()

    def summary(self):
        def med(xs):
            return sorted(xs)[len(xs) // 2] if xs else None
        return {"source": self.sclk, "mhz_median": med(self.mhz), "mhz_min": min(self.mhz) if self.mhz else None,
                "mhz_max": max(self.mhz) if self.mhz else None, "samples": len(self.mhz),
                "power_w_median": med(self.watts)}


def _stats(ms_list):
    import numpy as np
    a = np.asarray(ms_list, dtype=np.float64)
    return {"median_ms": float(np.median(a)), "min_ms": float(a.min()), "mean_ms": float(a.mean()),
            "max_ms": float(a.max()), "reps": int(a.size)}


def gpu_bench(steps: int, warmup: int, extras: bool = True) -> dict:
    import numpy as np
    import torch

    from attention_gqa_flash_amd import binding, inputs

    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    pci_bus = "%04x:%02x:%02x.0" % (props.pci_domain_id, props.pci_bus_id, props.pci_device_id)

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    sets = []
    for seed in range(3):
        p = inputs.gptoss_prefill(seed=seed, length=PREFILL_LEN)
        sets.append(dict(q=bf16(p.q), k=bf16(p.k), v=bf16(p.v), sinks=torch.from_numpy(p.sinks).to(dev),
                         cu=torch.from_numpy(p.cu_seqlens).to(dev), o=torch.empty_like(bf16(p.q))))
    scale = 0.125
    dd = inputs.gptoss_decode(seed=0, batch=DEC_BATCH, ctx=DEC_CTX)
    dq, dk, dv = bf16(dd.q), bf16(dd.k), bf16(dd.v)
    dsinks = torch.from_numpy(dd.sinks).to(dev)
    dcu = torch.from_numpy(dd.cu_seqlens_k).to(dev)
    del dd
    do = torch.empty_like(dq)
    ws = torch.empty(binding.decode_workspace_bytes(DEC_BATCH, HQ, D, 64), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    ev = {name: [] for name in ("causal", "window", "decode")}

    # events for every timed step exist before the timed loop starts
    all_marks = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]

    def step(i, record):
        # The window layer reads another input set than the causal layer of
        # the same step: set (i + 1) % 3 was last read two steps earlier, and
        # each step's 1 GiB decode has since streamed through the Infinity
        # Cache, so both layers start cold.
        s = sets[i % 3]
        sw = sets[(i + 1) % 3]
        marks = all_marks[i] if record else None
        if record:
            marks[0].record()
        binding.prefill_varlen(s["q"], s["k"], s["v"], s["sinks"], s["cu"], PREFILL_LEN, 0, scale, out=s["o"])
        if record:
            marks[1].record()
        binding.prefill_varlen(sw["q"], sw["k"], sw["v"], sw["sinks"], sw["cu"], PREFILL_LEN, WINDOW, scale,
                               out=sw["o"])
        if record:
            marks[2].record()
        binding.decode_splitkv(dq, dk, dv, dcu, DEC_CTX, dsinks, 0, scale, DEC_SPLITS, workspace=ws, out=do)
        if record:
            marks[3].record()
            ev["causal"].append((marks[0], marks[1]))
            ev["window"].append((marks[1], marks[2]))
            ev["decode"].append((marks[2], marks[3]))

    # The engine clock is sampled over the warm-up steps and the timed steps
    # together (the timed steps alone last tens of milliseconds).
    clock = _ClockSampler(pci_bus)
    with clock:
        for i in range(warmup):
            step(i, False)
        torch.cuda.synchronize()
        # No garbage-collector pass inside the timed loop: a full collection can
        # hold the host thread long enough for the GPU to run out of queued work.
        gc.collect()
        gc.disable()
        try:
            t0 = time.perf_counter()
            for i in range(steps):
                step(i, True)
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
        finally:
            gc.enable()

    leg = {name: _stats([a.elapsed_time(b) for a, b in ev[name]]) for name in ev}
    t_causal, t_window, t_decode = (leg[n]["mean_ms"] for n in ("causal", "window", "decode"))
    # The rooflines use the median interval of each kernel (the mean also
    # carries the occasional long gap between two launches).
    m_causal, m_window, m_decode = (leg[n]["median_ms"] for n in ("causal", "window", "decode"))

    # Infinity-Cache scrub for legs whose working set would otherwise stay
    # cached between repetitions: a 512 MiB write outside the timed region.
    scrub_buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    def scrub():
        scrub_buf.fill_(1)

    def timed(fn, reps=20, warm=5, scrub_each=False):
        for _ in range(warm):
            fn()
        pairs = []
        for _ in range(reps):
            if scrub_each:
                scrub()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            pairs.append((a, b))
        torch.cuda.synchronize()
        return _stats([a.elapsed_time(b) for a, b in pairs])

    def hbm_entry(st, nbytes, flops=None):
        gbs = nbytes / (st["median_ms"] * 1e-3) / 1e9
        e = dict(st, algorithmic_bytes=nbytes, gbs_median=gbs,
                 gbs_best=nbytes / (st["min_ms"] * 1e-3) / 1e9, pct_hbm_peak=100 * gbs / PEAK_HBM_GBS)
        if flops is not None:
            e["algorithmic_flop"] = flops
            e["tflops_median"] = flops / (st["median_ms"] * 1e-3) / 1e12
            e["pct_mfma_peak"] = 100 * e["tflops_median"] / PEAK_BF16_TFLOPS
        return e

    def mfma_entry(st, flops, nbytes):
        tf = flops / (st["median_ms"] * 1e-3) / 1e12
        return dict(st, algorithmic_flop=flops, algorithmic_bytes=nbytes, tflops_median=tf,
                    tflops_best=flops / (st["min_ms"] * 1e-3) / 1e12, pct_mfma_peak=100 * tf / PEAK_BF16_TFLOPS,
                    pct_hbm_peak=100 * nbytes / (st["median_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS)

    # decode at every split count of the 64 x 8192 workload (the step uses 16)
    per_split = {}
    for s_count in (1, 4, 16):
        st = timed(lambda: binding.decode_splitkv(dq, dk, dv, dcu, DEC_CTX, dsinks, 0, scale, s_count,
                                                  workspace=ws, out=do))
        e = hbm_entry(st, decode_bytes([DEC_CTX] * DEC_BATCH, 0))
        e["GB/s"] = e["gbs_median"]
        per_split[str(s_count)] = e

    # the same workload against an FP8 (E4M3) cache with per-tensor scales
    fp8 = _fp8_decode(torch, binding, dev, dq, dsinks, dcu, ws, do, timed, hbm_entry)

    other = {}
    if extras:
        sets.clear()
        other = _other_configs(torch, np, binding, inputs, dev, bf16, timed, hbm_entry, mfma_entry)

    f_causal = prefill_flops([PREFILL_LEN], 0)
    f_window = prefill_flops([PREFILL_LEN], WINDOW)
    b_prefill = prefill_bytes([PREFILL_LEN], 0)
    b_decode = decode_bytes([DEC_CTX] * DEC_BATCH, 0)
    causal_tflops = f_causal / (t_causal * 1e-3) / 1e12
    window_tflops = f_window / (t_window * 1e-3) / 1e12
    window_gbs = b_prefill / (t_window * 1e-3) / 1e9
    prefill_tflops = (f_causal + f_window) / ((t_causal + t_window) * 1e-3) / 1e12
    decode_gbs = b_decode / (t_decode * 1e-3) / 1e9
    value = 100.0 * 0.5 * (prefill_tflops / PEAK_BF16_TFLOPS + decode_gbs / PEAK_HBM_GBS)

    r_causal = f_causal / (m_causal * 1e-3) / 1e12
    r_window = b_prefill / (m_window * 1e-3) / 1e9
    r_decode = b_decode / (m_decode * 1e-3) / 1e9
    roof_causal = {"kernel": "prefill_kernel (causal, L=8192, 64/8 heads)", "bound": "mfma",
                   "achieved": r_causal, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                   "frac": r_causal / PEAK_BF16_TFLOPS, "traffic": _traffic("prefill_causal"),
                   "ms": m_causal, "stat": "median", "algorithmic_flop": f_causal}
    roof_window = {"kernel": "prefill_kernel (window 128, L=8192, 64/8 heads)", "bound": "hbm",
                   "achieved": r_window, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                   "frac": r_window / PEAK_HBM_GBS, "traffic": _traffic("prefill_window"),
                   "ms": m_window, "stat": "median", "algorithmic_bytes": b_prefill,
                   "tflops": f_window / (m_window * 1e-3) / 1e12}
    roof_decode = {"kernel": "decode_kernel + merge_kernel (B=64, ctx 8192, S=16)", "bound": "hbm",
                   "achieved": r_decode, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                   "frac": r_decode / PEAK_HBM_GBS, "traffic": _traffic("decode_s16"),
                   "ms": m_decode, "stat": "median", "algorithmic_bytes": b_decode}
    return {
        "value": value, "ms_per_step": wall * 1e3 / steps,
        "prefill": {"tflops": prefill_tflops, "pct_mfma_peak": 100 * prefill_tflops / PEAK_BF16_TFLOPS,
                    "causal_ms": t_causal, "window_ms": t_window, "causal_tflops": causal_tflops,
                    "window_tflops": window_tflops, "window_gbs": window_gbs,
                    "causal_timing": leg["causal"], "window_timing": leg["window"]},
        "decode": {"gbs": decode_gbs, "pct_hbm_peak": 100 * decode_gbs / PEAK_HBM_GBS, "ms": t_decode,
                   "splits": DEC_SPLITS, "timing": leg["decode"], "by_splits": per_split,
                   "fp8_kv_by_splits": fp8},
        "roofline": roof_causal, "rooflines": [roof_causal, roof_window, roof_decode],
        "other_configs": other.get("configs"), "bandwidth_reference": other.get("bandwidth"),
        "engine_clock": clock.summary(),
        "device": {"name": props.name, "cus": props.multi_processor_count, "arch": props.gcnArchName,
                   "pci_bus": pci_bus},
    }


def _fp8_decode(torch, binding, dev, dq, dsinks, dcu, ws, do, timed, hbm_entry) -> dict:
    """64 x 8192 decode against an E4M3 cache (K = k_scale * e4m3(code), V
    likewise), S = 1, 4, 16: the codes are N(0,1) / scale rounded to E4M3 on
    the device from a seeded generator (timing-only inputs; parity runs on
    host-generated codes).  Bytes count one byte per cached element."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(3)
    k_scale, v_scale = 1.0 / 16, 1.0 / 16
    shape = (DEC_BATCH * DEC_CTX, HKV, D)

    def codes(s):
        x = torch.randn(shape, generator=gen, device=dev, dtype=torch.float32).mul_(1.0 / s)
        c = x.to(torch.float8_e4m3fn).view(torch.uint8)
        del x
        return c

    fk, fv = codes(k_scale), codes(v_scale)
    out = {}
    for s_count in (1, 4, 16):
        st = timed(lambda: binding.decode_splitkv_fp8(dq, fk, fv, k_scale, v_scale, dcu, DEC_CTX, dsinks, 0, 0.125,
                                                      s_count, workspace=ws, out=do))
        e = hbm_entry(st, decode_bytes([DEC_CTX] * DEC_BATCH, 0, kv_elem_bytes=1))
        e["shape"] = "B=64, ctx 8192, 64/8 heads, E4M3 K/V, S=%d" % s_count
        out[str(s_count)] = e
    del fk, fv
    torch.cuda.synchronize()
    return out


def _device_normal_bf16(torch, shape, gen, dev, std=1.0):
    """N(0, std^2) drawn in fp32 on the device from a seeded generator and
    rounded to bf16 (round to nearest even): timing-only inputs with the
    distribution of the host-generated parity inputs."""
    x = torch.randn(shape, generator=gen, device=dev, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(torch.bfloat16)


def _other_configs(torch, np, binding, inputs, dev, bf16, timed, hbm_entry, mfma_entry) -> dict:
    """The workloads besides the step: the tiny prefill, the long-context
    decode pair (full then 128-window, 32 splits) and the ragged 32-sequence
    varlen prefill (causal and 128-window), plus an achievable-bandwidth
    reference.  Each is timed alone with HIP events around the one call:
    5 warm-ups, 20 repetitions, median and min."""
    out = {}
    scale = 0.125

    # tiny: 1 x 256 tokens, 4 q heads / 1 KV head, causal (host inputs, seed 0)
    p = inputs.tiny_prefill(seed=0)
    tq, tk, tv = bf16(p.q), bf16(p.k), bf16(p.v)
    ts, tcu = torch.from_numpy(p.sinks).to(dev), torch.from_numpy(p.cu_seqlens).to(dev)
    to = torch.empty_like(tq)
    st = timed(lambda: binding.prefill_varlen(tq, tk, tv, ts, tcu, 256, 0, scale, out=to), scrub_each=True)
    out["tiny_prefill_causal"] = dict(mfma_entry(st, prefill_flops([256], 0, hq=4), prefill_bytes([256], 0, 4, 1)),
                                      bound="launch latency", shape="B=1, L=256, 4/1 heads")

    gen = torch.Generator(device=dev)

    # long decode: 16 x 32768 cached tokens, sinks std sqrt(2), 32 splits
    gen.manual_seed(1)
    nb, ctx, splits = 16, 32768, 32
    lq = _device_normal_bf16(torch, (nb, HQ, D), gen, dev)
    lk = _device_normal_bf16(torch, (nb * ctx, HKV, D), gen, dev)
    lv = _device_normal_bf16(torch, (nb * ctx, HKV, D), gen, dev)
    lsinks = torch.randn(HQ, generator=gen, device=dev, dtype=torch.float32) * math.sqrt(2.0)
    lcu = torch.arange(0, (nb + 1) * ctx, ctx, dtype=torch.int32, device=dev)
    lo = torch.empty_like(lq)
    lws = torch.empty(binding.decode_workspace_bytes(nb, HQ, D, splits), dtype=torch.uint8, device=dev)
    pair = []
    for window in (0, WINDOW):
        st = timed(lambda: binding.decode_splitkv(lq, lk, lv, lcu, ctx, lsinks, window, scale, splits,
                                                  workspace=lws, out=lo), scrub_each=(window > 0))
        e = hbm_entry(st, decode_bytes([ctx] * nb, window), decode_flops([ctx] * nb, window))
        e["shape"] = "B=16, ctx 32768, 64/8 heads, S=32, window %d" % window
        out["long_decode_%s" % ("full" if window == 0 else "w128")] = e
        pair.append(e)
    pb = sum(e["algorithmic_bytes"] for e in pair)
    pms = sum(e["median_ms"] for e in pair)
    out["long_decode_pair"] = {"median_ms": pms, "algorithmic_bytes": pb,
                               "gbs_median": pb / (pms * 1e-3) / 1e9,
                               "pct_hbm_peak": 100 * pb / (pms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    del lq, lk, lv, lo, lws

    # ragged varlen prefill: 32 sequences with the log-uniform lengths of
    # seed 0, heads 0, 9, 18, 27 without sink
    lengths = inputs.ragged_lengths(np.random.default_rng(0), 32)
    total, lmax = int(sum(lengths)), int(max(lengths))
    gen.manual_seed(2)
    rq = _device_normal_bf16(torch, (total, HQ, D), gen, dev)
    rk = _device_normal_bf16(torch, (total, HKV, D), gen, dev)
    rv = _device_normal_bf16(torch, (total, HKV, D), gen, dev)
    rs = torch.randn(HQ, generator=gen, device=dev, dtype=torch.float32)
    rs[list(inputs.NO_SINK_HEADS)] = -math.inf
    rcu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32), device=dev)
    ro = torch.empty_like(rq)
    for window in (0, WINDOW):
        st = timed(lambda: binding.prefill_varlen(rq, rk, rv, rs, rcu, lmax, window, scale, out=ro),
                   reps=20 if window else 10)
        f, b = prefill_flops(lengths, window), prefill_bytes(lengths, window)
        e = mfma_entry(st, f, b) if window == 0 else hbm_entry(st, b, f)
        e["shape"] = "32 sequences, T=%d, max L=%d, 64/8 heads, window %d" % (total, lmax, window)
        e["bound"] = "mfma" if window == 0 else "hbm"
        out["ragged_prefill_%s" % ("causal" if window == 0 else "w128")] = e
    del rq, rk, rv, ro
    torch.cuda.synchronize()

    # paged cache: the 64 x 8192 decode with 16- and 64-token pages in a
    # shuffled physical order (page table from a seeded host permutation)
    gen.manual_seed(5)
    pq = _device_normal_bf16(torch, (DEC_BATCH, HQ, D), gen, dev)
    psinks = torch.randn(HQ, generator=gen, device=dev, dtype=torch.float32)
    plens = torch.full((DEC_BATCH,), DEC_CTX, dtype=torch.int32, device=dev)
    po = torch.empty_like(pq)
    pws = torch.empty(binding.decode_workspace_bytes(DEC_BATCH, HQ, D, 16), dtype=torch.uint8, device=dev)
    pm_lens = [4] * DEC_BATCH
    pmq = _device_normal_bf16(torch, (sum(pm_lens), HQ, D), gen, dev)
    pmcq = torch.tensor(np.concatenate([[0], np.cumsum(pm_lens)]).astype(np.int32), device=dev)
    pmo = torch.empty_like(pmq)
    pmws = torch.empty(binding.decode_workspace_bytes(sum(pm_lens), HQ, D, 4), dtype=torch.uint8, device=dev)
    for page_size in (16, 64):
        per_seq = DEC_CTX // page_size
        n_pages = DEC_BATCH * per_seq
        kp = _device_normal_bf16(torch, (n_pages, page_size, HKV, D), gen, dev)
        vp = _device_normal_bf16(torch, (n_pages, page_size, HKV, D), gen, dev)
        perm = np.random.default_rng(page_size).permutation(n_pages).astype(np.int32)
        table = torch.tensor(perm.reshape(DEC_BATCH, per_seq), device=dev)
        for s_count in (1, 4, 16):
            st = timed(lambda: binding.decode_paged(pq, kp, vp, table, plens, DEC_CTX, psinks, 0, scale, s_count,
                                                    workspace=pws, out=po))
            e = hbm_entry(st, decode_bytes([DEC_CTX] * DEC_BATCH, 0))
            e["shape"] = "B=64, ctx 8192, 64/8 heads, %d-token pages (shuffled), S=%d" % (page_size, s_count)
            out["paged_decode_ps%d_s%d" % (page_size, s_count)] = e
        # draft-token verification against the same paged cache: the 4
        # newest tokens of each sequence are its queries
        for window in (0, WINDOW):
            f, b = append_flops(pm_lens, [DEC_CTX] * DEC_BATCH, window), append_bytes(pm_lens, [DEC_CTX] * DEC_BATCH,
                                                                                      window)
            for s_count in (1, 4):
                st = timed(lambda: binding.decode_paged_multi(pmq, kp, vp, table, plens, pmcq, 4, DEC_CTX, psinks,
                                                              window, scale, s_count, workspace=pmws, out=pmo),
                           scrub_each=(window > 0))
                e = hbm_entry(st, b, f)
                e["bound"] = "hbm"
                e["shape"] = "64 sequences, 4 queries, ctx 8192, 64/8 heads, %d-token pages (shuffled), window %d, " \
                             "S=%d" % (page_size, window, s_count)
                out["paged_draft_verify_64x4_ps%d_s%d_%s" % (page_size, s_count,
                                                              "causal" if window == 0 else "w128")] = e
        if page_size == 16:
            # the last 2048-token chunk of an 8192-token prompt whose keys
            # are the first sequence's pages
            cq2 = torch.tensor([0, 2048], dtype=torch.int32, device=dev)
            q2 = _device_normal_bf16(torch, (2048, HQ, D), gen, dev)
            o2 = torch.empty_like(q2)
            for window in (0, WINDOW):
                st = timed(lambda: binding.prefill_append_paged(q2, kp, vp, table[:1], plens[:1], cq2, 2048, DEC_CTX,
                                                                psinks, window, scale, out=o2),
                           scrub_each=(window > 0))
                f, b = append_flops([2048], [DEC_CTX], window), append_bytes([2048], [DEC_CTX], window)
                e = mfma_entry(st, f, b) if window == 0 else hbm_entry(st, b, f)
                e["bound"] = "mfma" if window == 0 else "hbm"
                e["shape"] = "last 2048 of 8192 tokens, keys in 16-token pages (shuffled), 64/8 heads, window %d" % window
                out["paged_chunked_prefill_last_2048_of_8192_%s" % ("causal" if window == 0 else "w128")] = e
            del q2, o2
            # the same table over pages of E4M3 codes (N(0,1) / scale rounded
            # on the device; one byte per cached element)
            fkp = (torch.randn(kp.shape, generator=gen, device=dev) * 16.0).to(torch.float8_e4m3fn).view(torch.uint8)
            fvp = (torch.randn(kp.shape, generator=gen, device=dev) * 16.0).to(torch.float8_e4m3fn).view(torch.uint8)
            for s_count in (1, 4, 16):
                st = timed(lambda: binding.decode_paged_fp8(pq, fkp, fvp, 1.0 / 16, 1.0 / 16, table, plens, DEC_CTX,
                                                            psinks, 0, scale, s_count, workspace=pws, out=po))
                e = hbm_entry(st, decode_bytes([DEC_CTX] * DEC_BATCH, 0, kv_elem_bytes=1))
                e["shape"] = "B=64, ctx 8192, 64/8 heads, E4M3 K/V in 16-token pages (shuffled), S=%d" % s_count
                out["paged_fp8_decode_ps16_s%d" % s_count] = e
            del fkp, fvp
        del kp, vp
    del pq, po, pws, pmq, pmo, pmws, pmcq
    torch.cuda.synchronize()

    # fused rotary step (YaRN, theta 150000, factor 32 over a 4096-token
    # original context, beta 32 / 1): the 8192 tokens of the prefill and the
    # 64 tokens of one decode step, K/V appended to distinct cache rows
    gen.manual_seed(6)
    for n_tok, rows_cache in ((PREFILL_LEN, 2 * PREFILL_LEN), (DEC_BATCH, DEC_BATCH * DEC_CTX)):
        rqkv = _device_normal_bf16(torch, (n_tok, HQ + 2 * HKV, D), gen, dev)
        rpos = torch.randint(0, 131072, (n_tok,), generator=gen, device=dev, dtype=torch.int32)
        rslots = torch.randperm(rows_cache, generator=gen, device=dev)[:n_tok].to(torch.int32)
        rkc = torch.empty((rows_cache, HKV, D), dtype=torch.bfloat16, device=dev)
        rvc = torch.empty_like(rkc)
        rq = torch.empty((n_tok, HQ, D), dtype=torch.bfloat16, device=dev)
        st = timed(lambda: binding.rope_qkv_append(rqkv, rpos, rslots, HQ, HKV, rkc, rvc, rope_theta=150000.0,
                                                   yarn_factor=32.0, yarn_original_max_position=4096,
                                                   yarn_beta_fast=32.0, yarn_beta_slow=1.0, q_out=rq),
                   scrub_each=(n_tok < 1024))
        nbytes = rope_bytes(n_tok)
        e = hbm_entry(st, nbytes)
        e["bound"] = "hbm"
        e["shape"] = "%d tokens, 64/8 heads, YaRN, K/V to distinct rows of a %d-row cache" % (n_tok, rows_cache)
        out["rope_qkv_append_%d" % n_tok] = e
        del rqkv, rkc, rvc, rq
    torch.cuda.synchronize()

    # output projection with bias (synthetic 2880-wide projection of the
    # 64 x 64 concatenated heads): the 64 rows of a decode step and the 8192
    # rows of the prefill
    gen.manual_seed(7)
    ow = (torch.randn((OPROJ_OUT, HQ * D), generator=gen, device=dev) / math.sqrt(HQ * D)).to(torch.bfloat16)
    ob = torch.randn(OPROJ_OUT, generator=gen, device=dev, dtype=torch.float32)
    for n_rows in (DEC_BATCH, PREFILL_LEN):
        oo = _device_normal_bf16(torch, (n_rows, HQ * D), gen, dev)
        oy = torch.empty((n_rows, OPROJ_OUT), dtype=torch.bfloat16, device=dev)
        st = timed(lambda: binding.oproj_bias(oo, ow, ob, out=oy), scrub_each=True)
        f = 2.0 * n_rows * HQ * D * OPROJ_OUT
        b = oproj_bytes(n_rows)
        if n_rows == DEC_BATCH:
            e = hbm_entry(st, b, f)
            e["bound"] = "hbm"
        else:
            e = mfma_entry(st, f, b)
            e["bound"] = "mfma"
        e["shape"] = "%d rows x 4096 -> 2880, bias" % n_rows
        out["oproj_bias_%d" % n_rows] = e
        del oo, oy
    del ow, ob
    torch.cuda.synchronize()

    # append prefill: the last 2048-token chunk of an 8192-token prompt, and
    # draft-token verification (64 sequences x 4 queries against 8192 cached)
    gen.manual_seed(4)
    for name, q_lens, k_lens in (("chunked_prefill_last_2048_of_8192", [2048], [8192]),
                                 ("draft_verify_64x4_ctx8192", [4] * 64, [8192] * 64)):
        aq = _device_normal_bf16(torch, (sum(q_lens), HQ, D), gen, dev)
        ak = _device_normal_bf16(torch, (sum(k_lens), HKV, D), gen, dev)
        av = _device_normal_bf16(torch, (sum(k_lens), HKV, D), gen, dev)
        asinks = torch.randn(HQ, generator=gen, device=dev, dtype=torch.float32)
        acq = torch.tensor(np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32), device=dev)
        ack = torch.tensor(np.concatenate([[0], np.cumsum(k_lens)]).astype(np.int32), device=dev)
        ao = torch.empty_like(aq)
        for window in (0, WINDOW):
            st = timed(lambda: binding.prefill_append(aq, ak, av, asinks, acq, ack, max(q_lens), max(k_lens), window,
                                                      scale, out=ao), scrub_each=(sum(k_lens) < 100000))
            f, b = append_flops(q_lens, k_lens, window), append_bytes(q_lens, k_lens, window)
            mfma_bound = name.startswith("chunked") and window == 0
            e = mfma_entry(st, f, b) if mfma_bound else hbm_entry(st, b, f)
            e["bound"] = "mfma" if mfma_bound else "hbm"
            e["shape"] = "%d sequences, %s queries, %s keys, 64/8 heads, window %d" % (
                len(q_lens), sorted(set(q_lens)), sorted(set(k_lens)), window)
            out["%s_%s" % (name, "causal" if window == 0 else "w128")] = e
            if name.startswith("draft"):
                # the same verification through the multi-token-query decode
                for s_count in (1, 4):
                    aws = torch.empty(binding.decode_workspace_bytes(sum(q_lens), HQ, D, s_count), dtype=torch.uint8,
                                      device=dev)
                    st = timed(lambda: binding.decode_splitkv_multi(aq, ak, av, acq, ack, max(q_lens), max(k_lens),
                                                                    asinks, window, scale, s_count, workspace=aws,
                                                                    out=ao), scrub_each=(window > 0))
                    e = hbm_entry(st, b, f)
                    e["bound"] = "hbm"
                    e["shape"] = "64 sequences, 4 queries, 8192 keys, 64/8 heads, window %d, S=%d" % (window, s_count)
                    out["%s_multi_decode_s%d_%s" % (name, s_count, "causal" if window == 0 else "w128")] = e
        del aq, ak, av, ao
    torch.cuda.synchronize()

    # a short chunk over a long cache: 256 new tokens after 32512 cached
    # (32768 keys), causal, unsplit and with each query tile's keys split 8
    # ways (sinkattn_prefill_append_splitkv)
    gen.manual_seed(9)
    q_lens, k_lens = [256], [32768]
    aq = _device_normal_bf16(torch, (256, HQ, D), gen, dev)
    ak = _device_normal_bf16(torch, (32768, HKV, D), gen, dev)
    av = _device_normal_bf16(torch, (32768, HKV, D), gen, dev)
    asinks = torch.randn(HQ, generator=gen, device=dev, dtype=torch.float32)
    acq = torch.tensor([0, 256], dtype=torch.int32, device=dev)
    ack = torch.tensor([0, 32768], dtype=torch.int32, device=dev)
    ao = torch.empty_like(aq)
    aws = torch.empty(binding.decode_workspace_bytes(256, HQ, D, 8), dtype=torch.uint8, device=dev)
    for s_count in (1, 8):
        st = timed(lambda: binding.prefill_append(aq, ak, av, asinks, acq, ack, 256, 32768, 0, scale, out=ao,
                                                  num_splits=s_count, workspace=aws), scrub_each=True)
        e = mfma_entry(st, append_flops(q_lens, k_lens, 0), append_bytes(q_lens, k_lens, 0))
        e["bound"] = "mfma"
        e["shape"] = "1 sequence, 256 queries, 32768 keys, 64/8 heads, causal, S=%d" % s_count
        out["chunked_prefill_256_of_32768_s%d" % s_count] = e
    del aq, ak, av, ao, aws
    torch.cuda.synchronize()

    # draft tokens through the multi-token decode only: 8 per sequence (64
    # columns per KV head), against the bf16 cache and against E4M3 caches
    # (4 and 8 per sequence); causal, 1 and 4 splits
    gen.manual_seed(8)
    k_lens = [DEC_CTX] * DEC_BATCH
    ak = _device_normal_bf16(torch, (sum(k_lens), HKV, D), gen, dev)
    av = _device_normal_bf16(torch, (sum(k_lens), HKV, D), gen, dev)
    fk = (torch.randn((sum(k_lens), HKV, D), generator=gen, device=dev) * 16.0).to(torch.float8_e4m3fn).view(torch.uint8)
    fv = (torch.randn((sum(k_lens), HKV, D), generator=gen, device=dev) * 16.0).to(torch.float8_e4m3fn).view(torch.uint8)
    asinks = torch.randn(HQ, generator=gen, device=dev, dtype=torch.float32)
    ack = torch.tensor(np.concatenate([[0], np.cumsum(k_lens)]).astype(np.int32), device=dev)
    for n_tok, fp8 in ((8, False), (4, True), (8, True)):
        q_lens = [n_tok] * DEC_BATCH
        aq = _device_normal_bf16(torch, (sum(q_lens), HQ, D), gen, dev)
        acq = torch.tensor(np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32), device=dev)
        ao = torch.empty_like(aq)
        f = append_flops(q_lens, k_lens, 0)
        b = append_bytes(q_lens, k_lens, 0)
        if fp8:  # one byte per cached K / V element
            b -= 2 * DEC_BATCH * DEC_CTX * HKV * D
        for s_count in (1, 4):
            aws = torch.empty(binding.decode_workspace_bytes(sum(q_lens), HQ, D, s_count), dtype=torch.uint8, device=dev)
            if fp8:
                st = timed(lambda: binding.decode_splitkv_multi_fp8(aq, fk, fv, 1.0 / 16, 1.0 / 16, acq, ack, n_tok,
                                                                    DEC_CTX, asinks, 0, scale, s_count, workspace=aws,
                                                                    out=ao))
            else:
                st = timed(lambda: binding.decode_splitkv_multi(aq, ak, av, acq, ack, n_tok, DEC_CTX, asinks, 0, scale,
                                                                s_count, workspace=aws, out=ao))
            e = hbm_entry(st, b, f)
            e["bound"] = "hbm"
            e["shape"] = "64 sequences, %d queries, 8192 keys (%s), 64/8 heads, causal, S=%d" % (
                n_tok, "E4M3" if fp8 else "bf16", s_count)
            out["%sdraft_verify_64x%d_multi_decode_s%d" % ("fp8_" if fp8 else "", n_tok, s_count)] = e
        del aq, ao
    del ak, av, fk, fv
    torch.cuda.synchronize()

    # one GPU's share of the heads under 4-way tensor parallelism (16 query /
    # 2 KV heads, the decode layout of the cost section), same batch, context
    # and sequence length: decode at 1, 4 and 16 splits and the causal
    # prefill; the quarter-size cache is read after a scrub
    gen.manual_seed(8)
    thq, thkv = HQ // 4, HKV // 4
    tq = _device_normal_bf16(torch, (DEC_BATCH, thq, D), gen, dev)
    tk = _device_normal_bf16(torch, (DEC_BATCH * DEC_CTX, thkv, D), gen, dev)
    tv = _device_normal_bf16(torch, (DEC_BATCH * DEC_CTX, thkv, D), gen, dev)
    tsinks = torch.randn(thq, generator=gen, device=dev, dtype=torch.float32)
    tcu = torch.arange(0, (DEC_BATCH + 1) * DEC_CTX, DEC_CTX, dtype=torch.int32, device=dev)
    to_ = torch.empty_like(tq)
    tws = torch.empty(binding.decode_workspace_bytes(DEC_BATCH, thq, D, 16), dtype=torch.uint8, device=dev)
    for s_count in (1, 4, 16):
        st = timed(lambda: binding.decode_splitkv(tq, tk, tv, tcu, DEC_CTX, tsinks, 0, scale, s_count,
                                                  workspace=tws, out=to_), scrub_each=True)
        e = hbm_entry(st, decode_bytes([DEC_CTX] * DEC_BATCH, 0, thq, thkv))
        e["shape"] = "B=64, ctx 8192, 16/2 heads (the 4-way tensor-parallel share), S=%d" % s_count
        out["tp4_share_decode_s%d" % s_count] = e
    del tq, tk, tv, to_, tws
    pq4 = _device_normal_bf16(torch, (PREFILL_LEN, thq, D), gen, dev)
    pk4 = _device_normal_bf16(torch, (PREFILL_LEN, thkv, D), gen, dev)
    pv4 = _device_normal_bf16(torch, (PREFILL_LEN, thkv, D), gen, dev)
    pcu4 = torch.tensor([0, PREFILL_LEN], dtype=torch.int32, device=dev)
    po4 = torch.empty_like(pq4)
    st = timed(lambda: binding.prefill_varlen(pq4, pk4, pv4, tsinks, pcu4, PREFILL_LEN, 0, scale, out=po4),
               scrub_each=True)
    e = mfma_entry(st, prefill_flops([PREFILL_LEN], 0, hq=thq), prefill_bytes([PREFILL_LEN], 0, thq, thkv))
    e["bound"] = "mfma"
    e["shape"] = "B=1, L=8192, 16/2 heads (the 4-way tensor-parallel share), causal"
    out["tp4_share_prefill_causal"] = e
    del pq4, pk4, pv4, po4
    torch.cuda.synchronize()

    # achievable bandwidth: a 2 GiB streaming read (torch sum over fp32) and a
    # 2 GiB device-to-device copy (4 GiB moved)
    n = (2 << 30) // 4
    a = torch.ones(n, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    acc = torch.empty((), dtype=torch.float32, device=dev)
    st_read = timed(lambda: torch.sum(a, dim=0, out=acc), reps=10, warm=3)
    st_copy = timed(lambda: b.copy_(a), reps=10, warm=3)
    bw = {"read_2GiB": dict(st_read, gbs_median=(n * 4) / (st_read["median_ms"] * 1e-3) / 1e9,
                            gbs_best=(n * 4) / (st_read["min_ms"] * 1e-3) / 1e9, kernel="torch.sum fp32"),
          "copy_2GiB": dict(st_copy, gbs_median=(2 * n * 4) / (st_copy["median_ms"] * 1e-3) / 1e9,
                            gbs_best=(2 * n * 4) / (st_copy["min_ms"] * 1e-3) / 1e9,
                            kernel="torch copy_ (read + write counted)")}
    del a, b
    torch.cuda.synchronize()
    return {"configs": out, "bandwidth": bw}


def _r(x, nd=4):
    """Round a float for the compact line (None stays None)."""
    return None if x is None else float("%.*g" % (nd, x))


def _leg(st, extra=None):
    out = {"median_ms": _r(st["median_ms"]), "min_ms": _r(st["min_ms"]), "mean_ms": _r(st["mean_ms"])}
    if extra:
        out.update(extra)
    return out


def _pct(entry):
    """The fraction of the peak an entry reports (MFMA for MFMA-bound
    workloads, else HBM), in percent."""
    if entry is None:
        return None
    key = "pct_mfma_peak" if entry.get("bound") == "mfma" and "pct_mfma_peak" in entry else "pct_hbm_peak"
    return _r(entry.get(key), 3)


def compact_record(full: dict, detail_path) -> dict:
    """The benchmark's last stdout line: the headline, each leg of the step,
    the rooflines, the CPU baseline and one figure per side workload, kept to
    a few KB so that it survives a short log tail.  Everything else (every
    statistic of every side workload, the bandwidth reference, the engine
    clock samples) is in the detail file."""
    pre, dec = full["prefill"], full["decode"]

    def roof(rf, named=True):
        if rf is None:
            return None
        out = {"kernel": rf.get("kernel")} if named else {}
        out.update({"bound": rf["bound"], "achieved": _r(rf["achieved"]), "peak": rf["peak"], "unit": rf["unit"],
                    "frac": _r(rf["frac"]), "traffic": _r(rf.get("traffic")), "ms": _r(rf.get("ms"))})
        return out

    cpu = full.get("cpu_baseline")
    cpu_c = None
    if cpu is not None:
        cpu_c = {"value": _r(cpu["value"]), "unit": cpu["unit"], "cores": cpu["cores"],
                 "affinity_cores": cpu.get("affinity_cores"), "kind": cpu["kind"], "sample": cpu.get("sample_short", cpu["sample"]),
                 "prefill_seconds": _r(cpu["prefill_seconds"]), "prefill_tflops_f64": _r(cpu["prefill_tflops_f64"]),
                 "decode_seconds": _r(cpu["decode_seconds"]), "decode_gbs_f64": _r(cpu["decode_gbs_f64"])}
    others = full.get("other_configs") or {}
    clock = full.get("engine_clock") or {}
    return {
        "metric": full["metric"], "value": _r(full["value"], 5), "unit": full["unit"], "n_gpus": full["n_gpus"],
        "steps": full["steps"], "warmup": full["warmup"], "ms_per_step": _r(full["ms_per_step"], 5),
        "higher_is_better": full["higher_is_better"], "scaling": full["scaling"], "vs_baseline": full["vs_baseline"],
        "dtype": full["dtype"], "data": full["data"], "config": {"workload": full["config"]["workload"]},
        "legs": {
            "prefill_causal": _leg(pre["causal_timing"], {"tflops": _r(pre["causal_tflops"])}),
            "prefill_w128": _leg(pre["window_timing"], {"gbs": _r(pre["window_gbs"])}),
            "decode_s16": _leg(dec["timing"], {"gbs": _r(dec["gbs"])}),
        },
        "decode_pct_hbm_by_splits": {k: _r(v["pct_hbm_peak"], 3) for k, v in dec["by_splits"].items()},
        "fp8_decode_pct_hbm_by_splits": {k: _r(v["pct_hbm_peak"], 3) for k, v in (dec.get("fp8_kv_by_splits") or {}).items()},
        "roofline": roof(full["roofline"]),
        # the step's other two legs: window prefill, decode (the causal
        # prefill is `roofline`)
        "rooflines": [roof(r, named=False) for r in full["rooflines"][1:]],
        "cpu_baseline": cpu_c,
        "other_pct_of_peak": {k: _pct(v) for k, v in others.items()},
        "engine_clock_mhz": clock.get("mhz_median"), "clock_samples": clock.get("samples"),
        "detail": detail_path,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the other workloads and the bandwidth reference (the step only)")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="also run one plain device-to-device copy of this many MiB (a reference "
                         "for HBM byte counters)")
    ap.add_argument("--detail-json", default=os.path.join("gpurun_out", "bench_detail.json"),
                    help="where the full record goes (the last stdout line is its compact form)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(the hot path needs no collective); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline()   # before the GPU is touched
    if args.calibration_copy_mib > 0:
        import torch
        n = args.calibration_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    g = gpu_bench(args.steps, args.warmup, extras=not args.no_extras)
    full = {
        "metric": METRIC, "value": g["value"],
        "unit": "% of MI355X peak (mean of prefill bf16-MFMA and decode HBM fractions)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": g["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) Q/K/V rounded to bf16, N(0,1) fp32 sinks",
        "config": {"workload": "GPT-OSS attention, 64 q / 8 KV heads, head_dim 64, scale 1/8: prefill of "
                               "1 x 8192 tokens (causal layer + 128-window layer) and split-KV decode of "
                               "64 x 8192 cached tokens (16 splits + LSE merge)",
                   "prefill": {"batch": 1, "seq_len": PREFILL_LEN, "windows": [0, WINDOW]},
                   "decode": {"batch": DEC_BATCH, "context": DEC_CTX, "splits": DEC_SPLITS}},
        "prefill": g["prefill"], "decode": g["decode"], "roofline": g["roofline"], "rooflines": g["rooflines"],
        "cpu_baseline": cpu, "other_configs": g["other_configs"],
        "bandwidth_reference": g["bandwidth_reference"], "engine_clock": g["engine_clock"], "device": g["device"],
    }
    detail = None
    if args.detail_json:
        try:
            d = os.path.dirname(args.detail_json)
            if d:
                os.makedirs(d, exist_ok=True)
            with open(args.detail_json, "w") as f:
                json.dump(full, f, indent=1)
            detail = args.detail_json
        except OSError as e:
            print("could not write %s: %s" % (args.detail_json, e), file=sys.stderr)
    sys.stdout.flush()
    print(json.dumps(compact_record(full, detail), separators=(",", ":")), flush=True)


if __name__ == "__main__":
    main()
