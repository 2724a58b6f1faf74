"""One long sequence, or a few, split many ways: the decode shapes of single-
user serving at long context (GPT-OSS layers see up to 131072 tokens; the
full-context layer of the NVIDIA gpt-oss announcement, model description).

These take launch choices of their own: with few (sequence, split) units
the decode runs a workgroup per (sequence, KV head, split) rather than per
(sequence, split), and a merge of more than 32 parts over fewer than 2048
rows gives each row a workgroup of several waves that share its parts.
Checked against the float64 oracle on every head and sequence, bf16 and
E4M3 caches, and the LSE merge entry point alone with many parts, empty
parts and empty rows.  Bars as in the rest of the suite: max |err| <= 2e-2,
mean |err| <= 2e-3, lse within 4e-3.
"""

import functools

import numpy as np
import pytest
import torch

from attention_gqa_flash_amd import binding, inputs
from oracle import decode_fp8_ref, decode_ref, merge_ref
from tests.helpers import (assert_close_lse, assert_close_out, bf16_to_device, f32_to_device, i32_to_device,
                           to_f64)

pytestmark = pytest.mark.gpu

SHAPES = {"1x131072": [131072], "4x32768": [32768] * 4}


@functools.lru_cache(maxsize=2)
def _bf16(shape):
    return inputs.make_decode(SHAPES[shape], hq=64, hkv=8, seed=50 + len(SHAPES[shape]))


@functools.lru_cache(maxsize=2)
def _fp8(shape):
    return inputs.make_decode_fp8(SHAPES[shape], hq=64, hkv=8, seed=60 + len(SHAPES[shape]))


@functools.lru_cache(maxsize=4)
def _bf16_ref(shape, window):
    d = _bf16(shape)
    qf, kf, vf = (inputs.bf16_bits_to_f32(x) for x in (d.q, d.k, d.v))
    return decode_ref(qf, kf, vf, d.cu_seqlens_k, d.sinks, window, d.scale)


@pytest.mark.parametrize("shape,splits", [("1x131072", 1), ("1x131072", 16), ("1x131072", 64), ("1x131072", 128),
                                          ("1x131072", 256), ("4x32768", 8), ("4x32768", 32), ("4x32768", 64)])
def test_long_context_decode(shape, splits):
    d = _bf16(shape)
    for window in (0, 128):
        o, lse = binding.decode_splitkv(bf16_to_device(d.q), bf16_to_device(d.k), bf16_to_device(d.v),
                                        i32_to_device(d.cu_seqlens_k), max(d.lengths), f32_to_device(d.sinks), window,
                                        d.scale, splits, return_lse=True)
        torch.cuda.synchronize()
        ro, rl = _bf16_ref(shape, window)
        what = "long decode %s S=%d W=%d" % (shape, splits, window)
        assert_close_out(to_f64(o), ro, what)
        assert_close_lse(lse.cpu().numpy(), rl, what)


@pytest.mark.parametrize("shape,splits", [("1x131072", 16), ("1x131072", 128), ("1x131072", 256), ("4x32768", 32)])
def test_long_context_fp8_decode(shape, splits):
    d = _fp8(shape)
    o, lse = binding.decode_splitkv_fp8(bf16_to_device(d.q), torch.from_numpy(d.k).cuda(), torch.from_numpy(d.v).cuda(),
                                        d.k_scale, d.v_scale, i32_to_device(d.cu_seqlens_k), max(d.lengths),
                                        f32_to_device(d.sinks), 0, d.scale, splits, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = decode_fp8_ref(inputs.bf16_bits_to_f32(d.q), d.k, d.v, d.k_scale, d.v_scale, d.cu_seqlens_k, d.sinks, 0,
                            d.scale)
    what = "long fp8 decode %s S=%d" % (shape, splits)
    assert_close_out(to_f64(o), ro, what)
    assert_close_lse(lse.cpu().numpy(), rl, what)


@pytest.mark.parametrize("parts,rows", [(33, 64), (300, 64), (257, 1), (40, 2047), (64, 2048)])
def test_merge_many_parts(parts, rows):
    """The merge entry point with more parts than one batch of loads: empty
    parts, a row with every part empty, parts ordered so the largest lse
    falls in different batches per row."""
    rng = np.random.default_rng(parts + rows)
    o_parts = rng.standard_normal((parts, rows, 1, 64)).astype(np.float32)
    lse_parts = (4.0 * rng.standard_normal((parts, rows, 1))).astype(np.float32)
    lse_parts[rng.random((parts, rows, 1)) < 0.1] = -np.inf
    lse_parts[:, 0, 0] = -np.inf  # row 0: every part empty
    o_parts[np.isinf(lse_parts)] = 0.0
    o, lse = binding.merge_lse(f32_to_device(o_parts), f32_to_device(lse_parts), return_lse=True)
    torch.cuda.synchronize()
    ro, rl = merge_ref(o_parts.astype(np.float64), lse_parts.astype(np.float64))
    what = "merge parts=%d rows=%d" % (parts, rows)
    assert_close_out(to_f64(o), ro, what)
    assert_close_lse(lse.cpu().numpy(), rl, what)
    assert np.all(to_f64(o)[0] == 0.0)


@pytest.mark.parametrize("page_size,splits", [(16, 16), (64, 64), (64, 256)])
def test_long_context_paged_decode(page_size, splits):
    """The same few-sequence launch choices over a paged cache (pages in a
    shuffled physical order, NaN in every slot no sequence owns)."""
    from oracle import decode_paged_ref
    p = inputs.make_paged_decode([131072], page_size, hq=64, hkv=8, seed=70 + page_size)
    o, lse = binding.decode_paged(bf16_to_device(p.q), bf16_to_device(p.k_pages), bf16_to_device(p.v_pages),
                                  i32_to_device(p.block_table), i32_to_device(p.seq_lens), 131072,
                                  f32_to_device(p.sinks), 0, p.scale, splits, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = decode_paged_ref(inputs.bf16_bits_to_f32(p.q), inputs.bf16_bits_to_f32(p.k_pages),
                              inputs.bf16_bits_to_f32(p.v_pages), p.block_table, p.seq_lens, page_size, p.sinks, 0,
                              p.scale)
    what = "long paged decode ps=%d S=%d" % (page_size, splits)
    assert_close_out(to_f64(o), ro, what)
    assert_close_lse(lse.cpu().numpy(), rl, what)
