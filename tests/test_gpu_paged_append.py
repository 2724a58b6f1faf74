"""GPU parity of the append (chunked) prefill against a paged cache with the
float64 oracle: the append prefill over the rows gathered through the block
table.

Pages are scattered in a random physical order with spare pages and every
unowned slot holds a bf16 NaN, so a copy from outside a sequence's tokens
would show in its output.  Cases: page sizes 16 to 256 (a 64-key tile then
spans up to four pages, or part of one), query counts 0 to 300 at key
offsets 0 to 1000, windows 0 to past the longest sequence, GQA groups 1 to 32,
without sinks, the last 2048-token chunk of an 8192-token prompt over 16-token
pages, agreement bit for bit with the append prefill on the contiguous cache,
and the debug checks.  Bar: max |err| <= 2e-2, mean |err| <= 2e-3, lse within
4e-3 with an identical -inf pattern.
"""

import numpy as np
import pytest
import torch

from attention_gqa_flash_amd import binding, inputs
from oracle import decode_paged_multi_ref
from tests.helpers import (assert_close_lse, assert_close_out, bf16_to_device, f32_to_device, i32_to_device,
                           to_f64)

pytestmark = pytest.mark.gpu

Q_LENS = [5, 1, 40, 33, 64, 300, 7, 0, 129]
K_LENS = [5, 2, 71, 65, 97, 364, 107, 3, 1129]


def _run(p, window, with_sinks=True):
    o, lse = binding.prefill_append_paged(bf16_to_device(p.q), bf16_to_device(p.k_pages), bf16_to_device(p.v_pages),
                                          i32_to_device(p.block_table), i32_to_device(p.seq_lens),
                                          i32_to_device(p.cu_seqlens_q), max(p.q_lens), max(p.k_lens),
                                          f32_to_device(p.sinks) if with_sinks else None, window, p.scale,
                                          return_lse=True)
    torch.cuda.synchronize()
    return to_f64(o), lse.cpu().numpy()


def _ref(p, window, with_sinks=True, rows=None):
    return decode_paged_multi_ref(inputs.bf16_bits_to_f32(p.q), inputs.bf16_bits_to_f32(p.k_pages),
                                  inputs.bf16_bits_to_f32(p.v_pages), p.block_table, p.seq_lens, p.cu_seqlens_q,
                                  p.page_size, p.sinks if with_sinks else None, window, p.scale, rows=rows)


@pytest.mark.parametrize("page_size", [16, 32, 64, 256])
@pytest.mark.parametrize("window", [0, 1, 100, 128, 5000])
@pytest.mark.parametrize("hq,hkv", [(64, 8), (32, 1), (16, 16)])
def test_paged_append(page_size, window, hq, hkv):
    p = inputs.make_paged_append(Q_LENS, K_LENS, page_size, hq=hq, hkv=hkv, seed=page_size + window + hq + hkv)
    o, lse = _run(p, window)
    ro, rl = _ref(p, window)
    what = "paged append ps=%d W=%d G=%d" % (page_size, window, hq // hkv)
    assert_close_out(o, ro, what)
    assert_close_lse(lse, rl, what)


def test_paged_append_without_sinks():
    p = inputs.make_paged_append(Q_LENS, K_LENS, 16, hq=64, hkv=8, seed=3)
    for window in (0, 128):
        o, lse = _run(p, window, with_sinks=False)
        ro, rl = _ref(p, window, with_sinks=False)
        assert_close_out(o, ro, "paged append no sinks W=%d" % window)
        assert_close_lse(lse, rl, "paged append no sinks")


@pytest.mark.parametrize("window", [0, 128])
def test_paged_chunk_last_2048_of_8192(window):
    p = inputs.make_paged_append([2048], [8192], 16, hq=64, hkv=8, seed=0)
    o, lse = _run(p, window)
    rows = sorted(set([0, 1, 31, 32, 63, 64, 1023, 1024, 2046, 2047])
                  | set(int(x) for x in np.random.default_rng(2).integers(0, 2048, 30)))
    ro, rl = _ref(p, window, rows=rows)
    assert_close_out(o[rows], ro[rows], "paged chunk W=%d" % window)
    assert_close_lse(lse[rows], rl[rows], "paged chunk")


def test_paged_append_equals_contiguous_append_bitwise():
    """The same draws, paged (16-token pages, shuffled) and contiguous: the
    kernel copies the same rows into the same LDS slots, so the outputs agree
    bit for bit."""
    p = inputs.make_paged_append(Q_LENS, K_LENS, 16, hq=64, hkv=8, seed=9)
    a = inputs.make_append(Q_LENS, K_LENS, hq=64, hkv=8, seed=9)
    assert np.array_equal(p.q, a.q)
    q, sinks, cq = bf16_to_device(a.q), f32_to_device(a.sinks), i32_to_device(a.cu_seqlens_q)
    for window in (0, 128):
        o1 = binding.prefill_append_paged(q, bf16_to_device(p.k_pages), bf16_to_device(p.v_pages),
                                          i32_to_device(p.block_table), i32_to_device(p.seq_lens), cq, max(Q_LENS),
                                          max(K_LENS), sinks, window, a.scale)
        o2 = binding.prefill_append(q, bf16_to_device(a.k), bf16_to_device(a.v), sinks, cq,
                                    i32_to_device(a.cu_seqlens_k), max(Q_LENS), max(K_LENS), window, a.scale)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), window


def test_paged_append_debug_checks(monkeypatch):
    monkeypatch.setenv("SINKATTN_DEBUG_CHECKS", "1")
    p = inputs.make_paged_append([30, 2], [40, 70], 16, hq=8, hkv=2, seed=10)  # NaN in every unowned slot: not inspected
    o, _ = _run(p, 0)
    ro, _ = _ref(p, 0)
    assert_close_out(o, ro, "paged append debug valid")
    args = [bf16_to_device(p.q), bf16_to_device(p.k_pages), bf16_to_device(p.v_pages)]
    short = i32_to_device(np.array([20, 70], dtype=np.int32))  # 30 queries against 20 keys
    with pytest.raises(binding.SinkAttnError) as err:
        binding.prefill_append_paged(*args, i32_to_device(p.block_table), short, i32_to_device(p.cu_seqlens_q), 30,
                                     70, f32_to_device(p.sinks), 0, p.scale)
    assert err.value.status == 1 and "fewer keys than queries" in str(err.value)
    bad = p.block_table.copy()
    bad[1, 4] = p.k_pages.shape[0]  # a page id one past the pool
    with pytest.raises(binding.SinkAttnError) as err:
        binding.prefill_append_paged(*args, i32_to_device(bad), i32_to_device(p.seq_lens),
                                     i32_to_device(p.cu_seqlens_q), 30, 70, f32_to_device(p.sinks), 0, p.scale)
    assert err.value.status == 1 and "page id" in str(err.value)
