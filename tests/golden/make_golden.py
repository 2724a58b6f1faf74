"""Writes the regression fixtures in this directory.

The stored values come only from ``oracle/`` (the float64 definition of sink
attention from the Perplexity page "GPT-OSS on day 0", section "GPT-OSS
kernels / Sink attention", with the window layers of the NVIDIA gpt-oss
announcement) applied to seeded inputs from
``attention_gqa_flash_amd.inputs``.  They pin the oracle against silent
changes; they are not values printed by the pages (the pages print none).

    python tests/golden/make_golden.py
"""

import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

from attention_gqa_flash_amd import inputs  # noqa: E402
from oracle import (decode_fp8_ref, decode_paged_ref, decode_ref, decode_split_partials_ref, oproj_ref,  # noqa: E402
                    prefill_append_ref, prefill_varlen_ref, rope_qkv_append_ref, yarn_inv_freq_ref)

PREFILL = dict(lengths=[33, 70], hq=4, hkv=2, d=64, seed=7)
PREFILL_ROWS = [0, 32, 102]
DECODE = dict(lengths=[1, 50, 129], hq=8, hkv=2, d=64, seed=8)


def _f(x):
    return [float(v) for v in np.asarray(x, dtype=np.float64).ravel()]


def build():
    out = {"source": "oracle/sink_attention.py on seeded inputs (see make_golden.py)",
           "prefill": {"inputs": PREFILL, "rows": PREFILL_ROWS, "cases": []},
           "decode": {"inputs": DECODE, "cases": []}}
    p = inputs.make_prefill(PREFILL["lengths"], PREFILL["hq"], PREFILL["hkv"], PREFILL["d"], seed=PREFILL["seed"])
    q, k, v = (inputs.bf16_bits_to_f32(x) for x in (p.q, p.k, p.v))
    for window in (0, 16):
        o, lse = prefill_varlen_ref(q, k, v, p.sinks, p.cu_seqlens, window, p.scale)
        out["prefill"]["cases"].append({"window": window, "lse": _f(lse), "o_rows_d8": _f(o[PREFILL_ROWS][..., :8])})
    dd = inputs.make_decode(DECODE["lengths"], DECODE["hq"], DECODE["hkv"], DECODE["d"], seed=DECODE["seed"])
    q, k, v = (inputs.bf16_bits_to_f32(x) for x in (dd.q, dd.k, dd.v))
    for window in (0, 32):
        o, lse = decode_ref(q, k, v, dd.cu_seqlens_k, dd.sinks, window, dd.scale)
        _, lp = decode_split_partials_ref(q, k, v, dd.cu_seqlens_k, dd.sinks, window, dd.scale, 4)
        out["decode"]["cases"].append({"window": window, "o_d8": _f(o[..., :8]), "lse": _f(lse), "split4_lse": _f(lp)})
    return out


APPEND = dict(q_lens=[3, 1, 20], k_lens=[40, 1, 20], hq=8, hkv=2, seed=9)
PAGED = dict(lengths=[5, 70], page_size=16, hq=8, hkv=2, seed=10)
FP8 = dict(lengths=[30, 90], hq=8, hkv=2, seed=11)
ROPE = dict(tokens=6, hq=4, hkv=2, cache_rows=10, seed=12)
YARN = dict(theta=150000.0, factor=32.0, original=4096, beta_fast=32.0, beta_slow=1.0)


def build_next():
    """The oracle functions of the appended-query, paged, FP8, rotary and
    projection workloads (oracle/append.py, paged.py, fp8.py, rope.py,
    oproj.py) on small seeded inputs."""
    out = {"source": "oracle/{append,paged,fp8,rope,oproj}.py on seeded inputs (see make_golden.py)"}
    a = inputs.make_append(APPEND["q_lens"], APPEND["k_lens"], APPEND["hq"], APPEND["hkv"], seed=APPEND["seed"])
    q, k, v = (inputs.bf16_bits_to_f32(x) for x in (a.q, a.k, a.v))
    out["append"] = {"inputs": APPEND, "cases": []}
    for window in (0, 8):
        o, lse = prefill_append_ref(q, k, v, a.sinks, a.cu_seqlens_q, a.cu_seqlens_k, window, a.scale)
        out["append"]["cases"].append({"window": window, "o_d8": _f(o[..., :8]), "lse": _f(lse)})
    p = inputs.make_paged_decode(PAGED["lengths"], PAGED["page_size"], PAGED["hq"], PAGED["hkv"], seed=PAGED["seed"])
    o, lse = decode_paged_ref(inputs.bf16_bits_to_f32(p.q), inputs.bf16_bits_to_f32(p.k_pages),
                              inputs.bf16_bits_to_f32(p.v_pages), p.block_table, p.seq_lens, p.page_size, p.sinks, 0,
                              p.scale)
    out["paged"] = {"inputs": PAGED, "o_d8": _f(o[..., :8]), "lse": _f(lse)}
    f8 = inputs.make_decode_fp8(FP8["lengths"], FP8["hq"], FP8["hkv"], seed=FP8["seed"])
    o, lse = decode_fp8_ref(inputs.bf16_bits_to_f32(f8.q), f8.k, f8.v, f8.k_scale, f8.v_scale, f8.cu_seqlens_k,
                            f8.sinks, 0, f8.scale)
    out["fp8"] = {"inputs": FP8, "o_d8": _f(o[..., :8]), "lse": _f(lse)}
    r = inputs.make_rope(ROPE["tokens"], ROPE["hq"], ROPE["hkv"], ROPE["cache_rows"], seed=ROPE["seed"])
    freq, m = yarn_inv_freq_ref(64, YARN["theta"], YARN["factor"], YARN["original"], YARN["beta_fast"],
                                YARN["beta_slow"])
    q_out, kc, _ = rope_qkv_append_ref(inputs.bf16_bits_to_f32(r.qkv), r.positions, ROPE["hq"], ROPE["hkv"], freq, m,
                                       r.slot_mapping, inputs.bf16_bits_to_f32(r.k_cache),
                                       inputs.bf16_bits_to_f32(r.v_cache))
    out["rope"] = {"inputs": ROPE, "yarn": YARN, "freq": _f(freq), "temperature": float(m),
                   "q_d8": _f(q_out[..., :8]), "k_cache_d8": _f(kc[..., :8])}
    rng = np.random.default_rng(13)
    o_in = rng.standard_normal((3, 128))
    w_in = rng.standard_normal((32, 128)) / np.sqrt(128)
    b_in = rng.standard_normal(32)
    out["oproj"] = {"seed": 13, "y": _f(oproj_ref(o_in, w_in, b_in))}
    return out


if __name__ == "__main__":
    data = build()
    with open(os.path.join(HERE, "oracle_regression.json"), "w") as f:
        json.dump(data, f)
    with open(os.path.join(HERE, "oracle_regression_next.json"), "w") as f:
        json.dump(build_next(), f)
    print("wrote oracle_regression.json, oracle_regression_next.json")
