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
from oracle import decode_ref, decode_split_partials_ref, prefill_varlen_ref  # noqa: E402

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


if __name__ == "__main__":
    data = build()
    with open(os.path.join(HERE, "oracle_regression.json"), "w") as f:
        json.dump(data, f)
    print("wrote oracle_regression.json")
