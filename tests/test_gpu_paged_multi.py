"""GPU parity of the multi-token-query decode against a paged cache (draft
tokens verified against a paged KV cache) with the float64 oracle: the
append prefill over the rows gathered through the block table.

Pages are scattered in a random physical order with spare pages and every
unowned slot holds a bf16 NaN.  Cases: page sizes 16 to 256, 1 to 8 query
tokens per sequence (none for some), cache lengths on and off page and tile
boundaries, the decode kernel shapes through the split counts, windows, GQA
groups 4 and 8, without sinks, agreement bit for bit with the multi-token
decode on the contiguous cache, and the debug check of the query counts.
Bar: max |err| <= 2e-2, mean |err| <= 2e-3, lse within 4e-3 with an identical
-inf pattern.
"""

import numpy as np
import pytest
import torch

from attention_gqa_flash_amd import binding, inputs
from oracle import decode_paged_multi_ref
from tests.helpers import (assert_close_lse, assert_close_out, bf16_to_device, f32_to_device, i32_to_device,
                           to_f64)

pytestmark = pytest.mark.gpu

K_LENS = [1, 4, 15, 16, 17, 33, 300, 1500, 2100, 5000]


def _q_lens(k_lens, max_q, seed):
    rng = np.random.default_rng(seed)
    lens = [int(min(k, rng.integers(0, max_q + 1))) for k in k_lens]
    lens[-1] = min(max_q, k_lens[-1])  # the longest count present at least once
    return lens


def _pages_to_device(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda")


def _run(p, window, splits, with_sinks=True):
    o, lse = binding.decode_paged_multi(bf16_to_device(p.q), _pages_to_device(p.k_pages), _pages_to_device(p.v_pages),
                                        i32_to_device(p.block_table), i32_to_device(p.seq_lens),
                                        i32_to_device(p.cu_seqlens_q), max(p.q_lens), max(p.k_lens),
                                        f32_to_device(p.sinks) if with_sinks else None, window, p.scale, splits,
                                        return_lse=True)
    torch.cuda.synchronize()
    return to_f64(o), lse.cpu().numpy()


def _ref(p, window, with_sinks=True):
    kf, vf = inputs.bf16_bits_to_f32(p.k_pages), inputs.bf16_bits_to_f32(p.v_pages)
    return decode_paged_multi_ref(inputs.bf16_bits_to_f32(p.q), kf, vf, p.block_table, p.seq_lens, p.cu_seqlens_q,
                                  p.page_size, p.sinks if with_sinks else None, window, p.scale)


@pytest.mark.parametrize("page_size", [16, 64, 256])
@pytest.mark.parametrize("hq,hkv,max_q", [(64, 8, 4), (16, 4, 8)])
@pytest.mark.parametrize("splits", [1, 2, 4, 16])
def test_paged_multi_decode(page_size, hq, hkv, max_q, splits):
    seed = page_size + hq + splits
    p = inputs.make_paged_append(_q_lens(K_LENS, max_q, seed), K_LENS, page_size, hq=hq, hkv=hkv, seed=seed)
    p.sinks[1] = -np.inf
    for window in (0, 128):
        o, lse = _run(p, window, splits)
        ro, rl = _ref(p, window)
        what = "paged multi ps=%d G=%d S=%d W=%d" % (page_size, hq // hkv, splits, window)
        assert_close_out(o, ro, what)
        assert_close_lse(lse, rl, what)


@pytest.mark.parametrize("splits", [1, 8])
def test_paged_multi_gptoss_shape_without_sinks(splits):
    p = inputs.make_paged_append([4, 3, 4, 1], [8192, 8192, 32768, 129], 16, hq=64, hkv=8, seed=80 + splits)
    for window in (0, 128):
        o, lse = _run(p, window, splits, with_sinks=False)
        ro, rl = _ref(p, window, with_sinks=False)
        assert_close_out(o, ro, "paged multi gpt-oss S=%d W=%d" % (splits, window))
        assert_close_lse(lse, rl, "paged multi gpt-oss")


def test_paged_multi_equals_contiguous_multi_bitwise():
    """The same draws, paged (16-token pages, shuffled) and contiguous: the
    kernels read the same values in the same order, so the outputs agree bit
    for bit."""
    q_lens, k_lens = [4, 1, 2, 3], [700, 1, 4096, 33]
    p = inputs.make_paged_append(q_lens, k_lens, 16, hq=64, hkv=8, seed=81)
    a = inputs.make_append(q_lens, k_lens, hq=64, hkv=8, seed=81)
    assert np.array_equal(p.q, a.q)
    q = bf16_to_device(a.q)
    sinks = f32_to_device(a.sinks)
    cq = i32_to_device(a.cu_seqlens_q)
    for window in (0, 128):
        for splits in (1, 4, 16):
            o1 = binding.decode_paged_multi(q, _pages_to_device(p.k_pages), _pages_to_device(p.v_pages),
                                            i32_to_device(p.block_table), i32_to_device(p.seq_lens), cq, 4, 4096,
                                            sinks, window, a.scale, splits)
            o2 = binding.decode_splitkv_multi(q, bf16_to_device(a.k), bf16_to_device(a.v), cq,
                                              i32_to_device(a.cu_seqlens_k), 4, 4096, sinks, window, a.scale, splits)
            torch.cuda.synchronize()
            assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), (window, splits)


def test_paged_multi_debug_checks(monkeypatch):
    monkeypatch.setenv("SINKATTN_DEBUG_CHECKS", "1")
    p = inputs.make_paged_append([3, 2], [40, 70], 16, hq=8, hkv=2, seed=82)  # NaN in every unowned slot: not inspected
    o, _ = _run(p, 0, 1)
    ro, _ = _ref(p, 0)
    assert_close_out(o, ro, "paged multi debug valid")
    short = i32_to_device(np.array([2, 70], dtype=np.int32))  # 3 queries against 2 keys
    with pytest.raises(binding.SinkAttnError) as err:
        binding.decode_paged_multi(bf16_to_device(p.q), _pages_to_device(p.k_pages), _pages_to_device(p.v_pages),
                                   i32_to_device(p.block_table), short, i32_to_device(p.cu_seqlens_q), 3, 70,
                                   f32_to_device(p.sinks), 0, p.scale, 1)
    assert err.value.status == 1 and "fewer keys than queries" in str(err.value)
    bad = p.block_table.copy()
    bad[1, 4] = p.k_pages.shape[0]  # a page id one past the pool
    with pytest.raises(binding.SinkAttnError) as err:
        binding.decode_paged_multi(bf16_to_device(p.q), _pages_to_device(p.k_pages), _pages_to_device(p.v_pages),
                                   i32_to_device(bad), i32_to_device(p.seq_lens), i32_to_device(p.cu_seqlens_q), 3,
                                   70, f32_to_device(p.sinks), 0, p.scale, 1)
    assert err.value.status == 1 and "page id" in str(err.value)
