"""The 4-way tensor-parallel share of the GPT-OSS heads at full size: one
GPU's 16 query / 2 KV heads (the EP4 DP1 TP4 decode layout of "GPT-OSS on
day 0", Perplexity, section on cost and performance) with the same batch,
context and prompt length as the one-GPU workloads.  These shapes take their
own launch choices (one KV head per eight-wave workgroup at S = 1, four-wave
interleaved and two-wave workgroups at more splits, the E4M3 kernels for two
KV heads), so they are checked at the sizes the benchmark times.

Decode 64 x 8192 (bf16 and E4M3 caches): every head and query of 8 of the 64
sequences (seeded choice) against the float64 oracle.  Prefill 1 x 8192
(causal and 128-window): the first and last rows, the tile edges and random
rows.  Bars as in the rest of the suite: max |err| <= 2e-2, mean |err| <=
2e-3, lse within 4e-3.
"""

import functools

import numpy as np
import pytest
import torch

from attention_gqa_flash_amd import binding, inputs
from oracle import decode_fp8_ref, decode_ref, prefill_varlen_ref
from tests.helpers import (assert_close_lse, assert_close_out, bf16_to_device, f32_to_device, i32_to_device,
                           to_f64)

pytestmark = pytest.mark.gpu

B, CTX, HQ, HKV = 64, 8192, 16, 2
SAMPLE = np.sort(np.random.default_rng(321).choice(B, size=8, replace=False))


def _sub(q, k, v, cu, pick):
    ks = np.concatenate([k[cu[b]:cu[b + 1]] for b in pick])
    vs = np.concatenate([v[cu[b]:cu[b + 1]] for b in pick])
    lens = [int(cu[b + 1] - cu[b]) for b in pick]
    return q[pick], ks, vs, np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


@functools.lru_cache(maxsize=1)
def _bf16_inputs():
    return inputs.make_decode([CTX] * B, hq=HQ, hkv=HKV, seed=40)


@functools.lru_cache(maxsize=1)
def _fp8_inputs():
    return inputs.make_decode_fp8([CTX] * B, hq=HQ, hkv=HKV, seed=41)


@pytest.mark.parametrize("splits", [1, 2, 4, 16])
def test_tp_share_decode_64x8192(splits):
    d = _bf16_inputs()
    o, lse = binding.decode_splitkv(bf16_to_device(d.q), bf16_to_device(d.k), bf16_to_device(d.v),
                                    i32_to_device(d.cu_seqlens_k), CTX, f32_to_device(d.sinks), 0, d.scale, splits,
                                    return_lse=True)
    torch.cuda.synchronize()
    q, ks, vs, cu = _sub(inputs.bf16_bits_to_f32(d.q), inputs.bf16_bits_to_f32(d.k), inputs.bf16_bits_to_f32(d.v),
                         d.cu_seqlens_k, SAMPLE)
    ro, rl = decode_ref(q, ks, vs, cu, d.sinks, 0, d.scale)
    assert_close_out(to_f64(o)[SAMPLE], ro, "tp share decode S=%d" % splits)
    assert_close_lse(lse.cpu().numpy()[SAMPLE], rl, "tp share decode S=%d" % splits)


@pytest.mark.parametrize("splits", [1, 4, 16])
def test_tp_share_fp8_decode_64x8192(splits):
    d = _fp8_inputs()
    o, lse = binding.decode_splitkv_fp8(bf16_to_device(d.q), torch.from_numpy(d.k).cuda(), torch.from_numpy(d.v).cuda(),
                                        d.k_scale, d.v_scale, i32_to_device(d.cu_seqlens_k), CTX,
                                        f32_to_device(d.sinks), 0, d.scale, splits, return_lse=True)
    torch.cuda.synchronize()
    q, ks, vs, cu = _sub(inputs.bf16_bits_to_f32(d.q), d.k, d.v, d.cu_seqlens_k, SAMPLE)
    ro, rl = decode_fp8_ref(q, ks, vs, d.k_scale, d.v_scale, cu, d.sinks, 0, d.scale)
    assert_close_out(to_f64(o)[SAMPLE], ro, "tp share fp8 decode S=%d" % splits)
    assert_close_lse(lse.cpu().numpy()[SAMPLE], rl, "tp share fp8 decode S=%d" % splits)


@pytest.mark.parametrize("window", [0, 128])
def test_tp_share_prefill_8192(window):
    p = inputs.make_prefill([CTX], hq=HQ, hkv=HKV, seed=42)
    rng = np.random.default_rng(43)
    edges = [31, 32, 63, 64, 127, 128, 129, 4095, 4096]
    rows = np.unique(np.concatenate([np.arange(0, 40), np.arange(CTX - 40, CTX), edges,
                                     rng.integers(0, CTX, size=120)])).astype(np.int64)
    o, lse = binding.prefill_varlen(bf16_to_device(p.q), bf16_to_device(p.k), bf16_to_device(p.v),
                                    f32_to_device(p.sinks), i32_to_device(p.cu_seqlens), CTX, window, p.scale,
                                    return_lse=True)
    torch.cuda.synchronize()
    qf, kf, vf = (inputs.bf16_bits_to_f32(x) for x in (p.q, p.k, p.v))
    ro, rl = prefill_varlen_ref(qf, kf, vf, p.sinks, p.cu_seqlens, window, p.scale, rows=rows)
    assert_close_out(to_f64(o)[rows], ro[rows], "tp share prefill W=%d" % window)
    assert_close_lse(lse.cpu().numpy()[rows], rl[rows], "tp share prefill W=%d" % window)
