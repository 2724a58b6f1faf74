"""The oracle reproduces its stored regression fixture (tests/golden)."""

import json
import os

import numpy as np

from attention_gqa_flash_amd import inputs
from oracle import decode_ref, decode_split_partials_ref, prefill_varlen_ref

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load():
    with open(os.path.join(HERE, "oracle_regression.json")) as f:
        return json.load(f)


def test_prefill_fixture():
    g = _load()["prefill"]
    a = g["inputs"]
    p = inputs.make_prefill(a["lengths"], a["hq"], a["hkv"], a["d"], seed=a["seed"])
    q, k, v = (inputs.bf16_bits_to_f32(x) for x in (p.q, p.k, p.v))
    for case in g["cases"]:
        o, lse = prefill_varlen_ref(q, k, v, p.sinks, p.cu_seqlens, case["window"], p.scale)
        np.testing.assert_allclose(lse.ravel(), case["lse"], rtol=1e-12)
        np.testing.assert_allclose(o[g["rows"]][..., :8].ravel(), case["o_rows_d8"], rtol=1e-10, atol=1e-13)


def test_decode_fixture():
    g = _load()["decode"]
    a = g["inputs"]
    d = inputs.make_decode(a["lengths"], a["hq"], a["hkv"], a["d"], seed=a["seed"])
    q, k, v = (inputs.bf16_bits_to_f32(x) for x in (d.q, d.k, d.v))
    for case in g["cases"]:
        o, lse = decode_ref(q, k, v, d.cu_seqlens_k, d.sinks, case["window"], d.scale)
        _, lp = decode_split_partials_ref(q, k, v, d.cu_seqlens_k, d.sinks, case["window"], d.scale, 4)
        np.testing.assert_allclose(o[..., :8].ravel(), case["o_d8"], rtol=1e-10, atol=1e-13)
        np.testing.assert_allclose(lse.ravel(), case["lse"], rtol=1e-12)
        np.testing.assert_allclose(lp.ravel(), case["split4_lse"], rtol=1e-12)


def _load_next():
    with open(os.path.join(HERE, "oracle_regression_next.json")) as f:
        return json.load(f)


def test_next_fixture_against_the_current_oracle():
    """Appended queries, paged decode, FP8 decode, rotary step and projection
    reproduce their stored values (written by tests/golden/make_golden.py)."""
    import sys
    sys.path.insert(0, HERE)
    import make_golden
    stored = _load_next()
    fresh = make_golden.build_next()
    for key in ("append", "paged", "fp8", "rope", "oproj"):
        a, b = stored[key], fresh[key]
        for field, value in a.items():
            if field in ("inputs", "yarn", "seed"):
                assert value == b[field]
            elif field == "cases":
                for ca, cb in zip(value, b[field]):
                    for f2 in ca:
                        np.testing.assert_allclose(cb[f2], ca[f2], rtol=1e-10, atol=1e-13)
            else:
                np.testing.assert_allclose(b[field], value, rtol=1e-10, atol=1e-13)
