"""Benchmark of the sink-attention hot path on one MI355X.

One step = one pass of the whole path over one batch of seeded synthetic
input with GPT-OSS attention shapes (64 query heads, 8 KV heads, head_dim
64, scale 1/8):
  * prefill, batch 1 x 8192 tokens: the causal full-context layer and the
    128-token sliding-window layer (varlen entry point, cu_seqlens);
  * split-KV decode, batch 64 x 8192 cached tokens, 16 splits, including
    the log-sum-exp merge.

Printed: ONE JSON line.  `value` is the mean of the two roofline fractions
(prefill FLOP/s over the bf16 MFMA peak, decode KV bytes/s over the HBM
peak) in percent; each leg is also reported on its own.  FLOP and byte
counts are algorithmic (unmasked query-key pairs; Q + O + the K/V rows
attended + sinks), measured with HIP events on the stream the kernels run
on.  Inputs are resident in HBM before timing; the prefill leg rotates three
input sets so that its 151 MB working set does not stay in the 256 MB
Infinity Cache between steps.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
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


def prefill_flops(lengths, window) -> float:
    return 4.0 * D * HQ * sum(visible_pairs(n, window) for n in lengths)


def prefill_bytes(lengths, window) -> float:
    t = sum(lengths)
    qo = 2 * t * HQ * D * 2
    kv = 2 * t * HKV * D * 2          # every key is attended by some query
    return float(qo + kv + HQ * 4 + (len(lengths) + 1) * 4)


def decode_bytes(lengths, window) -> float:
    keys = sum(min(n, window) if window > 0 else n for n in lengths)
    return float(2 * len(lengths) * HQ * D * 2 + 2 * keys * HKV * D * 2 + HQ * 4 + (len(lengths) + 1) * 4)


def decode_flops(lengths, window) -> float:
    keys = sum(min(n, window) if window > 0 else n for n in lengths)
    return 4.0 * D * HQ * keys


# ---------------------------------------------------------------------------
# CPU baseline: the oracle, timed on a bounded sample of the same workload
# ---------------------------------------------------------------------------

def _decode_one(args):
    from oracle import decode_ref
    q, k, v, sinks, length, scale = args
    return decode_ref(q, k, v, [0, length], sinks, 0, scale)


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
    with ctx.Pool(processes=cores, initializer=_pool_init) as pool:
        pool.map(_decode_one, tasks[:cores], chunksize=1)  # start-up outside the timing
        t0 = time.perf_counter()
        pool.map(_decode_one, tasks, chunksize=1)
        t_dec = time.perf_counter() - t0
    dec_gbs = decode_bytes([DEC_CTX] * DEC_BATCH, 0) / t_dec / 1e9
    value = 100.0 * 0.5 * (pre_tflops / PEAK_BF16_TFLOPS + dec_gbs / PEAK_HBM_GBS)
    return {
        "value": value, "unit": "% of MI355X peak (same formula as value)", "cores": cores, "kind": "oracle",
        "sample": "one whole step: prefill 1 x 8192 tokens (causal + 128-window layers) and decode 64 x 8192 "
                  "keys, 64/8 heads, on %d spawned processes with 1 BLAS thread each (pool start-up included "
                  "for prefill, excluded for decode)" % cores,
        "prefill_tflops_f64": pre_tflops, "prefill_seconds": t_pre,
        "decode_gbs_f64": dec_gbs, "decode_seconds": t_dec,
    }


# ---------------------------------------------------------------------------
# GPU leg
# ---------------------------------------------------------------------------

def _kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "attention_gqa_flash_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def _traffic(kernel: str):
    """Measured HBM bytes per launch from the committed counter summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    ent = data.get(kernel)
    if not ent or ent.get("source_hash") != _kernel_source_hash():
        return None
    return ent.get("bytes_per_launch")


def gpu_bench(steps: int, warmup: int) -> dict:
    import numpy as np
    import torch

    from attention_gqa_flash_amd import binding, inputs

    dev = torch.device("cuda:0")

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

    def step(i, record):
        s = sets[i % 3]
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(4)] if record else None
        if record:
            marks[0].record()
        binding.prefill_varlen(s["q"], s["k"], s["v"], s["sinks"], s["cu"], PREFILL_LEN, 0, scale, out=s["o"])
        if record:
            marks[1].record()
        binding.prefill_varlen(s["q"], s["k"], s["v"], s["sinks"], s["cu"], PREFILL_LEN, WINDOW, scale,
                               out=s["o"])
        if record:
            marks[2].record()
        binding.decode_splitkv(dq, dk, dv, dcu, DEC_CTX, dsinks, 0, scale, DEC_SPLITS, workspace=ws, out=do)
        if record:
            marks[3].record()
            ev["causal"].append((marks[0], marks[1]))
            ev["window"].append((marks[1], marks[2]))
            ev["decode"].append((marks[2], marks[3]))

    for i in range(warmup):
        step(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    def mean_ms(name):
        return float(np.mean([a.elapsed_time(b) for a, b in ev[name]]))

    t_causal, t_window, t_decode = mean_ms("causal"), mean_ms("window"), mean_ms("decode")

    # decode at the other split counts (reported; not part of the step)
    per_split = {}
    for s_count in (1, 4, 16):
        for _ in range(3):
            binding.decode_splitkv(dq, dk, dv, dcu, DEC_CTX, dsinks, 0, scale, s_count, workspace=ws, out=do)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(10):
            binding.decode_splitkv(dq, dk, dv, dcu, DEC_CTX, dsinks, 0, scale, s_count, workspace=ws, out=do)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / 10
        per_split[str(s_count)] = {"ms": ms, "GB/s": decode_bytes([DEC_CTX] * DEC_BATCH, 0) / (ms * 1e-3) / 1e9}

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

    roof_causal = {"kernel": "prefill_kernel (causal, L=8192, 64/8 heads)", "bound": "mfma",
                   "achieved": causal_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                   "frac": causal_tflops / PEAK_BF16_TFLOPS, "traffic": _traffic("prefill_causal"),
                   "ms": t_causal, "algorithmic_flop": f_causal}
    roof_window = {"kernel": "prefill_kernel (window 128, L=8192, 64/8 heads)", "bound": "hbm",
                   "achieved": window_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                   "frac": window_gbs / PEAK_HBM_GBS, "traffic": _traffic("prefill_window"),
                   "ms": t_window, "algorithmic_bytes": b_prefill, "tflops": window_tflops}
    roof_decode = {"kernel": "decode_kernel + merge_kernel (B=64, ctx 8192, S=16)", "bound": "hbm",
                   "achieved": decode_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                   "frac": decode_gbs / PEAK_HBM_GBS, "traffic": _traffic("decode_s16"),
                   "ms": t_decode, "algorithmic_bytes": b_decode}
    props = torch.cuda.get_device_properties(dev)
    return {
        "value": value, "ms_per_step": wall * 1e3 / steps,
        "prefill": {"tflops": prefill_tflops, "pct_mfma_peak": 100 * prefill_tflops / PEAK_BF16_TFLOPS,
                    "causal_ms": t_causal, "window_ms": t_window, "causal_tflops": causal_tflops,
                    "window_tflops": window_tflops, "window_gbs": window_gbs},
        "decode": {"gbs": decode_gbs, "pct_hbm_peak": 100 * decode_gbs / PEAK_HBM_GBS, "ms": t_decode,
                   "splits": DEC_SPLITS, "by_splits": per_split},
        "roofline": roof_causal, "rooflines": [roof_causal, roof_window, roof_decode],
        "device": {"name": props.name, "cus": props.multi_processor_count},
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="also run one plain device-to-device copy of this many MiB (a reference "
                         "for HBM byte counters)")
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
    g = gpu_bench(args.steps, args.warmup)
    out = {
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
        "cpu_baseline": cpu, "device": g["device"],
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
