"""The workloads beyond the five named ones, at the sizes the benchmark times,
against the float64 oracle on host-generated inputs of the same shapes.

Outputs the oracle can produce in seconds are compared in full (the fused
rotary step and the 64-row projection); otherwise on samples: whole decode
sequences (every query head and draft token of 8 of the 64 sequences, chosen
by a seeded generator) and query rows of the long append chunk.  Bars as in the rest of
the suite: attention outputs max |err| <= 2e-2, mean |err| <= 2e-3, lse
within 4e-3; the rotary step and the projection within half a bf16 ulp (plus
1e-5, resp. 1e-3 for fp32 accumulation over K = 4096).
"""

import functools

import numpy as np
import pytest
import torch

from attention_gqa_flash_amd import binding, inputs
from oracle import (decode_fp8_ref, decode_paged_fp8_ref, decode_paged_multi_ref, decode_paged_ref, oproj_ref, prefill_append_ref, rope_qkv_append_ref,
                    yarn_inv_freq_ref)
from tests.helpers import (assert_close_lse, assert_close_out, bf16_to_device, f32_to_device, i32_to_device,
                           to_f64)

pytestmark = pytest.mark.gpu

B, CTX, HQ, HKV = 64, 8192, 64, 8
SAMPLE = np.sort(np.random.default_rng(123).choice(B, size=8, replace=False))


@functools.lru_cache(maxsize=1)
def _fp8_inputs():
    return inputs.make_decode_fp8([CTX] * B, hq=HQ, hkv=HKV, seed=0)


@functools.lru_cache(maxsize=1)
def _paged_inputs(page_size):
    return inputs.make_paged_decode([CTX] * B, page_size, hq=HQ, hkv=HKV, seed=0)


@functools.lru_cache(maxsize=1)
def _draft_inputs():
    return inputs.make_append([4] * B, [CTX] * B, hq=HQ, hkv=HKV, seed=0)


def _sub_decode(q, k, v, cu, pick):
    """The oracle's inputs restricted to sequences `pick` of a packed cache."""
    ks = np.concatenate([k[cu[b]:cu[b + 1]] for b in pick])
    vs = np.concatenate([v[cu[b]:cu[b + 1]] for b in pick])
    lens = [int(cu[b + 1] - cu[b]) for b in pick]
    return q[pick], ks, vs, np.concatenate([[0], np.cumsum(lens)])


@pytest.mark.parametrize("splits", [1, 4, 16])
def test_fp8_decode_64x8192(splits):
    d = _fp8_inputs()
    o, lse = binding.decode_splitkv_fp8(bf16_to_device(d.q), torch.from_numpy(d.k).cuda(), torch.from_numpy(d.v).cuda(),
                                        d.k_scale, d.v_scale, i32_to_device(d.cu_seqlens_k), CTX, f32_to_device(d.sinks),
                                        0, d.scale, splits, return_lse=True)
    torch.cuda.synchronize()
    q, ks, vs, cu = _sub_decode(inputs.bf16_bits_to_f32(d.q), d.k, d.v, d.cu_seqlens_k, SAMPLE)
    ro, rl = decode_fp8_ref(q, ks, vs, d.k_scale, d.v_scale, cu, d.sinks, 0, d.scale)
    assert_close_out(to_f64(o)[SAMPLE], ro, "fp8 64x8192 S=%d" % splits)
    assert_close_lse(lse.cpu().numpy()[SAMPLE], rl, "fp8 64x8192")


@pytest.mark.parametrize("splits", [1, 4, 16])
@pytest.mark.parametrize("page_size", [16, 64])
def test_paged_decode_64x8192(page_size, splits):
    p = _paged_inputs(page_size)
    o, lse = binding.decode_paged(bf16_to_device(p.q), bf16_to_device(p.k_pages), bf16_to_device(p.v_pages),
                                  i32_to_device(p.block_table), i32_to_device(p.seq_lens), CTX,
                                  f32_to_device(p.sinks), 0, p.scale, splits, return_lse=True)
    torch.cuda.synchronize()
    qf = inputs.bf16_bits_to_f32(p.q)
    ro, rl = decode_paged_ref(qf[SAMPLE], inputs.bf16_bits_to_f32(p.k_pages), inputs.bf16_bits_to_f32(p.v_pages),
                              p.block_table[SAMPLE], p.seq_lens[SAMPLE], page_size, p.sinks, 0, p.scale)
    assert_close_out(to_f64(o)[SAMPLE], ro, "paged ps=%d S=%d" % (page_size, splits))
    assert_close_lse(lse.cpu().numpy()[SAMPLE], rl, "paged")


@pytest.mark.parametrize("splits", [1, 4, 16])
def test_paged_fp8_decode_64x8192(splits):
    p = inputs.make_paged_decode_fp8([CTX] * B, 16, hq=HQ, hkv=HKV, seed=0)
    o, lse = binding.decode_paged_fp8(bf16_to_device(p.q), torch.from_numpy(p.k_pages).cuda(),
                                      torch.from_numpy(p.v_pages).cuda(), p.k_scale, p.v_scale,
                                      i32_to_device(p.block_table), i32_to_device(p.seq_lens), CTX,
                                      f32_to_device(p.sinks), 0, p.scale, splits, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = decode_paged_fp8_ref(inputs.bf16_bits_to_f32(p.q)[SAMPLE], p.k_pages, p.v_pages, p.k_scale, p.v_scale,
                                  p.block_table[SAMPLE], p.seq_lens[SAMPLE], 16, p.sinks, 0, p.scale)
    assert_close_out(to_f64(o)[SAMPLE], ro, "paged fp8 64x8192 S=%d" % splits)
    assert_close_lse(lse.cpu().numpy()[SAMPLE], rl, "paged fp8 64x8192")


@pytest.mark.parametrize("window", [0, 128])
def test_draft_verification_64x4_over_8192(window):
    """Both the append prefill and the multi-token decode (S = 1 and 4)."""
    a = _draft_inputs()
    q, k, v = (bf16_to_device(x) for x in (a.q, a.k, a.v))
    sinks = f32_to_device(a.sinks)
    cq, ck = i32_to_device(a.cu_seqlens_q), i32_to_device(a.cu_seqlens_k)
    rows = np.concatenate([np.arange(4 * b, 4 * b + 4) for b in SAMPLE])
    qf, kf, vf = (inputs.bf16_bits_to_f32(x) for x in (a.q, a.k, a.v))
    sub_k = np.concatenate([kf[a.cu_seqlens_k[b]:a.cu_seqlens_k[b + 1]] for b in SAMPLE])
    sub_v = np.concatenate([vf[a.cu_seqlens_k[b]:a.cu_seqlens_k[b + 1]] for b in SAMPLE])
    cu_q = np.arange(0, 4 * len(SAMPLE) + 1, 4)
    cu_k = np.arange(0, CTX * len(SAMPLE) + 1, CTX)
    ro, rl = prefill_append_ref(qf[rows], sub_k, sub_v, a.sinks, cu_q, cu_k, window, a.scale)
    got = binding.prefill_append(q, k, v, sinks, cq, ck, 4, CTX, window, a.scale, return_lse=True)
    for splits in (1, 4):
        got_m = binding.decode_splitkv_multi(q, k, v, cq, ck, 4, CTX, sinks, window, a.scale, splits, return_lse=True)
        torch.cuda.synchronize()
        assert_close_out(to_f64(got_m[0])[rows], ro, "multi decode S=%d W=%d" % (splits, window))
        assert_close_lse(got_m[1].cpu().numpy()[rows], rl, "multi decode")
    assert_close_out(to_f64(got[0])[rows], ro, "append prefill W=%d" % window)
    assert_close_lse(got[1].cpu().numpy()[rows], rl, "append prefill")


@pytest.mark.parametrize("window", [0, 128])
def test_draft_verification_64x4_over_8192_paged(window):
    """The multi-token decode against 16-token pages (S = 1 and 4)."""
    p = inputs.make_paged_append([4] * B, [CTX] * B, 16, hq=HQ, hkv=HKV, seed=0)
    args = [bf16_to_device(x) for x in (p.q, p.k_pages, p.v_pages)]
    table, lens, cq = (i32_to_device(x) for x in (p.block_table, p.seq_lens, p.cu_seqlens_q))
    rows = np.concatenate([np.arange(4 * b, 4 * b + 4) for b in SAMPLE])
    ro, rl = decode_paged_multi_ref(inputs.bf16_bits_to_f32(p.q)[rows], inputs.bf16_bits_to_f32(p.k_pages),
                                    inputs.bf16_bits_to_f32(p.v_pages), p.block_table[SAMPLE], p.seq_lens[SAMPLE],
                                    np.arange(0, 4 * len(SAMPLE) + 1, 4), 16, p.sinks, window, p.scale)
    for splits in (1, 4):
        o, lse = binding.decode_paged_multi(*args, table, lens, cq, 4, CTX, f32_to_device(p.sinks), window, p.scale,
                                            splits, return_lse=True)
        torch.cuda.synchronize()
        assert_close_out(to_f64(o)[rows], ro, "paged draft S=%d W=%d" % (splits, window))
        assert_close_lse(lse.cpu().numpy()[rows], rl, "paged draft")


@pytest.mark.parametrize("window", [0, 128])
def test_chunked_prefill_last_2048_of_8192_paged(window):
    p = inputs.make_paged_append([2048], [8192], 16, hq=HQ, hkv=HKV, seed=0)
    o, lse = binding.prefill_append_paged(bf16_to_device(p.q), bf16_to_device(p.k_pages), bf16_to_device(p.v_pages),
                                          i32_to_device(p.block_table), i32_to_device(p.seq_lens),
                                          i32_to_device(p.cu_seqlens_q), 2048, 8192, f32_to_device(p.sinks), window,
                                          p.scale, return_lse=True)
    torch.cuda.synchronize()
    rows = sorted(set(int(x) for x in np.random.default_rng(3).integers(0, 2048, 40)) | {0, 2047})
    ro, rl = decode_paged_multi_ref(inputs.bf16_bits_to_f32(p.q), inputs.bf16_bits_to_f32(p.k_pages),
                                    inputs.bf16_bits_to_f32(p.v_pages), p.block_table, p.seq_lens, p.cu_seqlens_q, 16,
                                    p.sinks, window, p.scale, rows=rows)
    assert_close_out(to_f64(o)[rows], ro[rows], "paged chunk W=%d" % window)
    assert_close_lse(lse.cpu().numpy()[rows], rl[rows], "paged chunk")


@pytest.mark.parametrize("window", [0, 128])
def test_chunked_prefill_last_2048_of_8192(window):
    a = inputs.make_append([2048], [8192], hq=HQ, hkv=HKV, seed=0)
    o, lse = binding.prefill_append(*(bf16_to_device(x) for x in (a.q, a.k, a.v)), f32_to_device(a.sinks),
                                    i32_to_device(a.cu_seqlens_q), i32_to_device(a.cu_seqlens_k), 2048, 8192, window,
                                    a.scale, return_lse=True)
    torch.cuda.synchronize()
    rows = sorted(set([0, 1, 2, 31, 32, 63, 64, 1023, 1024, 2046, 2047])
                  | set(int(x) for x in np.random.default_rng(1).integers(0, 2048, 40)))
    qf, kf, vf = (inputs.bf16_bits_to_f32(x) for x in (a.q, a.k, a.v))
    ro, rl = prefill_append_ref(qf, kf, vf, a.sinks, a.cu_seqlens_q, a.cu_seqlens_k, window, a.scale, rows=rows)
    assert_close_out(to_f64(o)[rows], ro[rows], "chunk W=%d" % window)
    assert_close_lse(lse.cpu().numpy()[rows], rl[rows], "chunk")


def test_rope_8192_tokens():
    r = inputs.make_rope(8192, HQ, HKV, cache_rows=16384, seed=0)
    params = dict(rope_theta=150000.0, yarn_factor=32.0, yarn_original_max_position=4096, yarn_beta_fast=32.0,
                  yarn_beta_slow=1.0)
    kc, vc = bf16_to_device(r.k_cache), bf16_to_device(r.v_cache)
    q_out = binding.rope_qkv_append(bf16_to_device(r.qkv), i32_to_device(r.positions), i32_to_device(r.slot_mapping),
                                    HQ, HKV, kc, vc, **params)
    torch.cuda.synchronize()
    f, m = yarn_inv_freq_ref(64, 150000.0, 32.0, 4096, 32.0, 1.0)
    rq, rk, _ = rope_qkv_append_ref(inputs.bf16_bits_to_f32(r.qkv), r.positions, HQ, HKV, f, m, r.slot_mapping,
                                    inputs.bf16_bits_to_f32(r.k_cache), inputs.bf16_bits_to_f32(r.v_cache))
    for got, ref in ((to_f64(q_out), rq), (to_f64(kc), rk)):
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-5)


@pytest.mark.parametrize("rows", [64, 8192])
def test_oproj_bench_shapes(rows):
    rng = np.random.default_rng(rows)
    o = inputs.round_to_bf16_bits(rng.standard_normal((rows, 4096), dtype=np.float32))
    w = inputs.round_to_bf16_bits((rng.standard_normal((2880, 4096)) / 64.0).astype(np.float32))
    b = rng.standard_normal(2880).astype(np.float32)
    y = binding.oproj_bias(bf16_to_device(o), bf16_to_device(w), f32_to_device(b))
    torch.cuda.synchronize()
    pick = np.arange(rows) if rows <= 64 else np.sort(rng.choice(rows, 256, replace=False))
    ref = oproj_ref(inputs.bf16_bits_to_f32(o[pick]), inputs.bf16_bits_to_f32(w), b)
    got = to_f64(y)[pick]
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-3)
