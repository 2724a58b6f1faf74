"""The five named workloads at full size, in the launch configuration the
benchmark times, against the float64 oracle.

Where the oracle cannot finish the whole output in seconds (long prefill),
it computes a sample of rows one by one: every row of the first tiles, rows
around tile and window boundaries, the last rows of every sequence and
seeded random rows, each for all 64 heads.  Decode outputs are compared in
full.  Bar: max |err| <= 2e-2, mean |err| <= 2e-3, lse within 4e-3.
"""

import numpy as np
import pytest
import torch

from attention_gqa_flash_amd import binding, inputs
from oracle import decode_ref, prefill_varlen_ref
from tests.helpers import (assert_close_lse, assert_close_out, bf16_to_device, f32_to_device, i32_to_device,
                           to_f64)

pytestmark = pytest.mark.gpu


def _sample_rows(cu, rng, per_seq_random=3):
    rows = set()
    for b in range(len(cu) - 1):
        a, e = int(cu[b]), int(cu[b + 1])
        n = e - a
        if n == 0:
            continue
        local = set(range(min(n, 3))) | {n - 1, n - 2}
        for edge in (31, 32, 63, 64, 127, 128, 129, 255, 256):
            if edge < n:
                local.add(edge)
        local |= set(int(x) for x in rng.integers(0, n, size=per_seq_random))
        rows |= {a + x for x in local if 0 <= x < n}
    return np.array(sorted(rows), dtype=np.int64)


def _prefill_full(p, window, rows):
    q, k, v = (bf16_to_device(x) for x in (p.q, p.k, p.v))
    o, lse = binding.prefill_varlen(q, k, v, f32_to_device(p.sinks), i32_to_device(p.cu_seqlens),
                                    max(p.lengths), window, p.scale, return_lse=True)
    torch.cuda.synchronize()
    o = to_f64(o)
    lse = lse.cpu().numpy()
    assert np.isfinite(o).all()
    qf, kf, vf = (inputs.bf16_bits_to_f32(x) for x in (p.q, p.k, p.v))
    ro, rl = prefill_varlen_ref(qf, kf, vf, p.sinks, p.cu_seqlens, window, p.scale, rows=rows)
    return o[rows], lse[rows], ro[rows], rl[rows]


@pytest.mark.parametrize("window", [0, 128])
def test_gptoss_prefill_8192(window):
    p = inputs.gptoss_prefill(seed=0)
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([np.arange(0, 96), np.arange(8192 - 40, 8192),
                                     rng.integers(0, 8192, size=120)]))
    o, lse, ro, rl = _prefill_full(p, window, rows)
    mx, mean = assert_close_out(o, ro, "prefill 8192 W=%d" % window)
    print("prefill 8192 W=%d rows=%d max|err| %.3g mean|err| %.3g" % (window, len(rows), mx, mean))
    assert_close_lse(lse, rl, "prefill 8192")


@pytest.mark.parametrize("window", [0, 128])
def test_ragged_varlen_prefill(window):
    p = inputs.ragged_prefill(seed=0)
    assert len(p.lengths) == 32 and min(p.lengths) >= 128 and max(p.lengths) <= 32768
    assert np.all(np.isneginf(p.sinks[list(inputs.NO_SINK_HEADS)]))
    rows = _sample_rows(p.cu_seqlens, np.random.default_rng(2))
    o, lse, ro, rl = _prefill_full(p, window, rows)
    mx, mean = assert_close_out(o, ro, "ragged W=%d" % window)
    print("ragged T=%d maxL=%d W=%d rows=%d max|err| %.3g mean|err| %.3g" % (
        sum(p.lengths), max(p.lengths), window, len(rows), mx, mean))
    assert_close_lse(lse, rl, "ragged")


def _decode_full(d, window, splits):
    q, k, v = (bf16_to_device(x) for x in (d.q, d.k, d.v))
    cu, sinks = i32_to_device(d.cu_seqlens_k), f32_to_device(d.sinks)
    outs = []
    for s in splits:
        o, lse = binding.decode_splitkv(q, k, v, cu, max(d.lengths), sinks, window, d.scale, s, return_lse=True)
        torch.cuda.synchronize()
        outs.append((s, to_f64(o), lse.cpu().numpy()))
    del q, k, v
    return outs


def test_gptoss_decode_splits_agree():
    d = inputs.gptoss_decode(seed=0)
    outs = _decode_full(d, 0, (1, 4, 16))
    qf, kf, vf = (inputs.bf16_bits_to_f32(x) for x in (d.q, d.k, d.v))
    ro, rl = decode_ref(qf, kf, vf, d.cu_seqlens_k, d.sinks, 0, d.scale)
    for s, o, lse in outs:
        mx, mean = assert_close_out(o, ro, "decode S=%d" % s)
        print("decode B=64 ctx=8192 S=%d max|err| %.3g mean|err| %.3g" % (s, mx, mean))
        assert_close_lse(lse, rl, "decode S=%d" % s)
    for s, o, _ in outs[1:]:
        assert_close_out(o, outs[0][1], "decode S=%d vs S=1" % s)


def test_long_decode_layer_pair():
    d = inputs.long_decode(seed=0)
    qf, kf, vf = (inputs.bf16_bits_to_f32(x) for x in (d.q, d.k, d.v))
    for window in (0, 128):
        (_, o, lse), = _decode_full(d, window, (32,))
        ro, rl = decode_ref(qf, kf, vf, d.cu_seqlens_k, d.sinks, window, d.scale)
        mx, mean = assert_close_out(o, ro, "long decode W=%d" % window)
        print("long decode B=16 ctx=32768 W=%d S=32 max|err| %.3g mean|err| %.3g" % (window, mx, mean))
        assert_close_lse(lse, rl, "long decode W=%d" % window)
