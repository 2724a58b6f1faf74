"""GPU parity of the paged-KV decode against the float64 oracle (the decode
over the rows gathered through the block table).

Pages are scattered in a random physical order with spare pages, and every
slot no sequence owns holds a bf16 NaN, so a read outside a sequence's tokens
would show in its output.  Cases: page sizes 16 to 256 (a 32-key tile then
spans up to three pages), lengths on and off page and tile boundaries, every
decode kernel shape through the split counts, windows, GQA groups 4 to 32,
without sinks, agreement with the contiguous decode bit for bit, and the
debug check of the page table; the same over pages of FP8 (E4M3) codes,
with an E4M3 NaN in every unowned slot.  Bar: max |err| <= 2e-2, mean |err| <= 2e-3,
lse within 4e-3 with an identical -inf pattern.
"""

import numpy as np
import pytest
import torch

from attention_gqa_flash_amd import binding, inputs
from oracle import decode_paged_fp8_ref, decode_paged_ref
from tests.helpers import (assert_close_lse, assert_close_out, bf16_to_device, f32_to_device, i32_to_device,
                           to_f64)

pytestmark = pytest.mark.gpu

LENGTHS = [1, 15, 16, 17, 33, 300, 1500, 2100, 5000]


def _pages_to_device(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda")


def _run(p, window, splits, with_sinks=True):
    o, lse = binding.decode_paged(bf16_to_device(p.q), _pages_to_device(p.k_pages), _pages_to_device(p.v_pages),
                                  i32_to_device(p.block_table), i32_to_device(p.seq_lens), max(p.lengths),
                                  f32_to_device(p.sinks) if with_sinks else None, window, p.scale, splits,
                                  return_lse=True)
    torch.cuda.synchronize()
    return to_f64(o), lse.cpu().numpy()


def _ref(p, window, with_sinks=True):
    kf, vf = inputs.bf16_bits_to_f32(p.k_pages), inputs.bf16_bits_to_f32(p.v_pages)
    return decode_paged_ref(inputs.bf16_bits_to_f32(p.q), kf, vf, p.block_table, p.seq_lens, p.page_size,
                            p.sinks if with_sinks else None, window, p.scale)


@pytest.mark.parametrize("page_size", [16, 32, 64, 256])
@pytest.mark.parametrize("hq,hkv", [(64, 8), (32, 1), (16, 4)])
@pytest.mark.parametrize("splits", [1, 2, 4, 16])
def test_paged_decode(page_size, hq, hkv, splits):
    p = inputs.make_paged_decode(LENGTHS, page_size, hq=hq, hkv=hkv, seed=page_size + hq + hkv + splits)
    p.sinks[1] = -np.inf
    for window in (0, 128):
        o, lse = _run(p, window, splits)
        ro, rl = _ref(p, window)
        what = "paged ps=%d G=%d S=%d W=%d" % (page_size, hq // hkv, splits, window)
        assert_close_out(o, ro, what)
        assert_close_lse(lse, rl, what)


@pytest.mark.parametrize("splits", [1, 4, 32])
def test_paged_decode_gptoss_shape_without_sinks(splits):
    p = inputs.make_paged_decode([8192] * 6 + [32768, 129], 16, hq=64, hkv=8, seed=70 + splits)
    for window in (0, 128):
        o, lse = _run(p, window, splits, with_sinks=False)
        ro, rl = _ref(p, window, with_sinks=False)
        assert_close_out(o, ro, "paged gpt-oss S=%d W=%d" % (splits, window))
        assert_close_lse(lse, rl, "paged gpt-oss")


def test_paged_equals_contiguous_decode_bitwise():
    """The same draws, paged (16-token pages, shuffled) and contiguous: the
    kernels read the same values in the same order, so the outputs agree bit
    for bit."""
    lengths = [700, 1, 4096, 33]
    p = inputs.make_paged_decode(lengths, 16, hq=64, hkv=8, seed=71)
    d = inputs.make_decode(lengths, hq=64, hkv=8, seed=71)
    assert np.array_equal(p.q, d.q)
    q = bf16_to_device(d.q)
    sinks = f32_to_device(d.sinks)
    for splits in (1, 4, 16):
        o1 = binding.decode_paged(q, _pages_to_device(p.k_pages), _pages_to_device(p.v_pages),
                                  i32_to_device(p.block_table), i32_to_device(p.seq_lens), 4096, sinks, 0, d.scale,
                                  splits)
        o2 = binding.decode_splitkv(q, bf16_to_device(d.k), bf16_to_device(d.v), i32_to_device(d.cu_seqlens_k), 4096,
                                    sinks, 0, d.scale, splits)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), splits


def test_paged_debug_checks(monkeypatch):
    monkeypatch.setenv("SINKATTN_DEBUG_CHECKS", "1")
    p = inputs.make_paged_decode([40, 70], 16, hq=8, hkv=2, seed=72)  # NaN in every unowned slot: not inspected
    o, _ = _run(p, 0, 1)
    ro, _ = _ref(p, 0)
    assert_close_out(o, ro, "paged debug valid")
    bad = p.block_table.copy()
    bad[1, 2] = p.k_pages.shape[0]  # a page id one past the pool
    with pytest.raises(binding.SinkAttnError) as err:
        binding.decode_paged(bf16_to_device(p.q), _pages_to_device(p.k_pages), _pages_to_device(p.v_pages),
                             i32_to_device(bad), i32_to_device(p.seq_lens), 70, f32_to_device(p.sinks), 0, p.scale, 1)
    assert err.value.status == 1 and "page id" in str(err.value)
    short = i32_to_device(np.array([40, 0], dtype=np.int32))
    with pytest.raises(binding.SinkAttnError) as err:
        binding.decode_paged(bf16_to_device(p.q), _pages_to_device(p.k_pages), _pages_to_device(p.v_pages),
                             i32_to_device(p.block_table), short, 70, f32_to_device(p.sinks), 0, p.scale, 1)
    assert err.value.status == 1 and "empty" in str(err.value)
    nan_k = p.k_pages.copy()
    nan_k[p.block_table[0, 2], 7, 0, 3] = 0x7FC0  # a bf16 NaN in a slot sequence 0 uses
    with pytest.raises(binding.SinkAttnError) as err:
        binding.decode_paged(bf16_to_device(p.q), _pages_to_device(nan_k), _pages_to_device(p.v_pages),
                             i32_to_device(p.block_table), i32_to_device(p.seq_lens), 70, f32_to_device(p.sinks), 0,
                             p.scale, 1)
    assert err.value.status == 1 and "k holds" in str(err.value)


def _run_fp8(p, window, splits):
    o, lse = binding.decode_paged_fp8(bf16_to_device(p.q), torch.from_numpy(p.k_pages).cuda(),
                                      torch.from_numpy(p.v_pages).cuda(), p.k_scale, p.v_scale,
                                      i32_to_device(p.block_table), i32_to_device(p.seq_lens), max(p.lengths),
                                      f32_to_device(p.sinks), window, p.scale, splits, return_lse=True)
    torch.cuda.synchronize()
    return to_f64(o), lse.cpu().numpy()


@pytest.mark.parametrize("page_size", [16, 64, 256])
@pytest.mark.parametrize("hq,hkv", [(64, 8), (32, 1), (16, 4)])
@pytest.mark.parametrize("splits", [1, 4, 16])
def test_paged_fp8_decode(page_size, hq, hkv, splits):
    p = inputs.make_paged_decode_fp8(LENGTHS, page_size, hq=hq, hkv=hkv, seed=90 + page_size + hq + splits)
    p.sinks[2] = -np.inf
    for window in (0, 128):
        o, lse = _run_fp8(p, window, splits)
        ro, rl = decode_paged_fp8_ref(inputs.bf16_bits_to_f32(p.q), p.k_pages, p.v_pages, p.k_scale, p.v_scale,
                                      p.block_table, p.seq_lens, page_size, p.sinks, window, p.scale)
        what = "paged fp8 ps=%d G=%d S=%d W=%d" % (page_size, hq // hkv, splits, window)
        assert_close_out(o, ro, what)
        assert_close_lse(lse, rl, what)


def test_paged_fp8_equals_contiguous_fp8_bitwise():
    lengths = [700, 1, 4096, 33]
    p = inputs.make_paged_decode_fp8(lengths, 16, hq=64, hkv=8, seed=91)
    d = inputs.make_decode_fp8(lengths, hq=64, hkv=8, seed=91)
    assert np.array_equal(p.q, d.q)
    q = bf16_to_device(d.q)
    sinks = f32_to_device(d.sinks)
    for window in (0, 128):
        for splits in (1, 4, 16):
            o1 = binding.decode_paged_fp8(q, torch.from_numpy(p.k_pages).cuda(), torch.from_numpy(p.v_pages).cuda(),
                                          p.k_scale, p.v_scale, i32_to_device(p.block_table),
                                          i32_to_device(p.seq_lens), 4096, sinks, window, d.scale, splits)
            o2 = binding.decode_splitkv_fp8(q, torch.from_numpy(d.k).cuda(), torch.from_numpy(d.v).cuda(), d.k_scale,
                                            d.v_scale, i32_to_device(d.cu_seqlens_k), 4096, sinks, window, d.scale,
                                            splits)
            torch.cuda.synchronize()
            assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), (window, splits)


def test_paged_fp8_debug_checks(monkeypatch):
    monkeypatch.setenv("SINKATTN_DEBUG_CHECKS", "1")
    p = inputs.make_paged_decode_fp8([40, 70], 16, hq=8, hkv=2, seed=92)  # NaN codes in every unowned slot: not inspected
    o, _ = _run_fp8(p, 0, 1)
    ro, _ = decode_paged_fp8_ref(inputs.bf16_bits_to_f32(p.q), p.k_pages, p.v_pages, p.k_scale, p.v_scale,
                                 p.block_table, p.seq_lens, 16, p.sinks, 0, p.scale)
    assert_close_out(o, ro, "paged fp8 debug valid")
    bad = p.v_pages.copy()
    bad[p.block_table[1, 3], 5, 1, 7] = 0xFF  # an E4M3 NaN in a slot sequence 1 uses
    with pytest.raises(binding.SinkAttnError) as err:
        binding.decode_paged_fp8(bf16_to_device(p.q), torch.from_numpy(p.k_pages).cuda(), torch.from_numpy(bad).cuda(),
                                 p.k_scale, p.v_scale, i32_to_device(p.block_table), i32_to_device(p.seq_lens), 70,
                                 f32_to_device(p.sinks), 0, p.scale, 1)
    assert err.value.status == 1 and "v holds" in str(err.value)
