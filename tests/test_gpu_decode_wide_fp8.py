"""GPU parity of the decode kernels' wider and narrower column layouts and of
draft tokens against an E4M3 cache.

* 33 to 64 (token, query head) columns per KV head (5 to 8 draft tokens at
  8 query heads per KV head: Baseten, "How to run GPT OSS 120B at 500+
  tokens per second on NVIDIA GPUs", next performance optimizations) through
  the multi-token decode, contiguous and paged, against the append oracle;
* several query tokens against an E4M3 cache (vLLM, "GPT-OSS performance
  optimizations on NVIDIA Blackwell", FlashInfer integration: FP8 KV cache),
  contiguous and paged, against the oracle's E4M3 composition, with 1 to 8
  tokens (16-, 32- and 64-column layouts), every decode kernel shape, windows,
  sequences without queries, without sinks; at one token equal to the
  single-token E4M3 decode (bitwise where both run the same kernel), and
  paged equal to contiguous.

Bar: max |err| <= 2e-2, mean |err| <= 2e-3 against the float64 oracle; lse
within tests.helpers.LSE_ABS with an identical -inf pattern.
"""

import numpy as np
import pytest
import torch

from attention_gqa_flash_amd import binding, inputs
from oracle import decode_fp8_multi_ref, decode_paged_fp8_multi_ref, prefill_append_ref
from tests.helpers import (assert_close_lse, assert_close_out, bf16_to_device, f32_to_device, i32_to_device,
                           to_f64)

pytestmark = pytest.mark.gpu

K_LENS = [1, 31, 300, 1500, 2100, 64, 5000]


def _u8(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _q_lens(n_tok):
    q_lens = [min(n_tok, n) for n in K_LENS]
    q_lens[5] = 0  # a sequence with no query this step
    return q_lens


@pytest.mark.parametrize("hq,hkv,n_tok", [(64, 8, 5), (64, 8, 8), (16, 1, 4), (64, 2, 2), (48, 8, 7)])
@pytest.mark.parametrize("splits", [1, 2, 4, 16])
def test_multi_decode_up_to_64_columns(hq, hkv, n_tok, splits):
    a = inputs.make_append(_q_lens(n_tok), K_LENS, hq=hq, hkv=hkv, seed=7 * hq + hkv + 13 * n_tok + splits)
    a.sinks[0] = -np.inf
    q, k, v = (bf16_to_device(x) for x in (a.q, a.k, a.v))
    qf, kf, vf = (inputs.bf16_bits_to_f32(x) for x in (a.q, a.k, a.v))
    for window in (0, 128, 1800):
        o, lse = binding.decode_splitkv_multi(q, k, v, i32_to_device(a.cu_seqlens_q), i32_to_device(a.cu_seqlens_k),
                                              max(a.q_lens), max(a.k_lens), f32_to_device(a.sinks), window, a.scale,
                                              splits, return_lse=True)
        torch.cuda.synchronize()
        ro, rl = prefill_append_ref(qf, kf, vf, a.sinks, a.cu_seqlens_q, a.cu_seqlens_k, window, a.scale)
        what = "wide multi G=%d n=%d S=%d W=%d" % (hq // hkv, n_tok, splits, window)
        assert_close_out(to_f64(o), ro, what)
        assert_close_lse(lse.cpu().numpy(), rl, what)


@pytest.mark.parametrize("splits", [1, 4])
def test_paged_multi_decode_64_columns_equals_contiguous(splits):
    q_lens, k_lens = [8, 8, 3, 0, 8], [8192, 300, 40, 17, 1029]
    p = inputs.make_paged_append(q_lens, k_lens, 16, hq=64, hkv=8, seed=70 + splits)
    a = inputs.make_append(q_lens, k_lens, hq=64, hkv=8, seed=70 + splits)
    assert np.array_equal(p.q, a.q)
    q, sinks = bf16_to_device(a.q), f32_to_device(a.sinks)
    cq = i32_to_device(a.cu_seqlens_q)
    qf, kf, vf = (inputs.bf16_bits_to_f32(x) for x in (a.q, a.k, a.v))
    for window in (0, 128):
        o1 = binding.decode_paged_multi(q, bf16_to_device(p.k_pages), bf16_to_device(p.v_pages),
                                        i32_to_device(p.block_table), i32_to_device(p.seq_lens), cq, 8, 8192, sinks,
                                        window, a.scale, splits)
        o2 = binding.decode_splitkv_multi(q, bf16_to_device(a.k), bf16_to_device(a.v), cq,
                                          i32_to_device(a.cu_seqlens_k), 8, 8192, sinks, window, a.scale, splits)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), (window, splits)
        ro, _ = prefill_append_ref(qf, kf, vf, a.sinks, a.cu_seqlens_q, a.cu_seqlens_k, window, a.scale)
        assert_close_out(to_f64(o1), ro, "paged wide multi W=%d S=%d" % (window, splits))


def _run_fp8_multi(a, window, splits, with_sinks=True):
    o, lse = binding.decode_splitkv_multi_fp8(bf16_to_device(a.q), _u8(a.k), _u8(a.v), a.k_scale, a.v_scale,
                                              i32_to_device(a.cu_seqlens_q), i32_to_device(a.cu_seqlens_k),
                                              max(a.q_lens), max(a.k_lens),
                                              f32_to_device(a.sinks) if with_sinks else None, window, a.scale, splits,
                                              return_lse=True)
    torch.cuda.synchronize()
    return to_f64(o), lse.cpu().numpy()


@pytest.mark.parametrize("hq,hkv,n_tok", [(64, 8, 1), (64, 8, 2), (64, 8, 4), (64, 8, 8), (16, 2, 3), (32, 8, 8),
                                          (64, 2, 1)])
@pytest.mark.parametrize("splits", [1, 4, 16])
def test_fp8_multi_decode(hq, hkv, n_tok, splits):
    a = inputs.make_append_fp8(_q_lens(n_tok), K_LENS, hq=hq, hkv=hkv, seed=3 * hq + hkv + 17 * n_tok + splits)
    a.sinks[1] = -np.inf
    qf = inputs.bf16_bits_to_f32(a.q)
    for window in (0, 128, 1800):
        o, lse = _run_fp8_multi(a, window, splits)
        ro, rl = decode_fp8_multi_ref(qf, a.k, a.v, a.k_scale, a.v_scale, a.cu_seqlens_q, a.cu_seqlens_k, a.sinks,
                                      window, a.scale)
        what = "fp8 multi G=%d n=%d S=%d W=%d" % (hq // hkv, n_tok, splits, window)
        assert_close_out(o, ro, what)
        assert_close_lse(lse, rl, what)


def test_fp8_multi_scales_and_no_sinks():
    a = inputs.make_append_fp8([4, 2, 4], [4096, 77, 9000], hq=64, hkv=8, seed=90, k_scale=1 / 32, v_scale=1 / 8)
    qf = inputs.bf16_bits_to_f32(a.q)
    for with_sinks in (True, False):
        o, lse = _run_fp8_multi(a, 0, 4, with_sinks)
        ro, rl = decode_fp8_multi_ref(qf, a.k, a.v, a.k_scale, a.v_scale, a.cu_seqlens_q, a.cu_seqlens_k,
                                      a.sinks if with_sinks else None, 0, a.scale)
        assert_close_out(o, ro, "fp8 multi sinks=%s" % with_sinks)
        assert_close_lse(lse, rl, "fp8 multi sinks=%s" % with_sinks)


@pytest.mark.parametrize("hq,hkv", [(20, 5), (64, 8)])
def test_fp8_multi_one_token_equals_single_token_fp8_decode(hq, hkv):
    """One query per sequence: the numbers of sinkattn_decode_splitkv_fp8.  Bit
    for bit where both calls run the same kernel (an odd number of KV heads);
    with G <= 8 over an even number of KV heads the single-token call runs
    the KV-head-pair kernel, which sums in another order, so there both are
    held to the bar against the oracle."""
    a = inputs.make_append_fp8([1] * 4, [700, 1, 4096, 33], hq=hq, hkv=hkv, seed=91)
    q, k, v = bf16_to_device(a.q), _u8(a.k), _u8(a.v)
    sinks = f32_to_device(a.sinks)
    cq, ck = i32_to_device(a.cu_seqlens_q), i32_to_device(a.cu_seqlens_k)
    qf = inputs.bf16_bits_to_f32(a.q)
    ro, _ = decode_fp8_multi_ref(qf, a.k, a.v, a.k_scale, a.v_scale, a.cu_seqlens_q, a.cu_seqlens_k, a.sinks, 0,
                                 a.scale)
    for splits in (1, 4, 16):
        o1 = binding.decode_splitkv_multi_fp8(q, k, v, a.k_scale, a.v_scale, cq, ck, 1, 4096, sinks, 0, a.scale,
                                              splits)
        o2 = binding.decode_splitkv_fp8(q, k, v, a.k_scale, a.v_scale, ck, 4096, sinks, 0, a.scale, splits)
        torch.cuda.synchronize()
        if hkv % 2:
            assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), splits
        else:
            assert_close_out(to_f64(o1), ro, "fp8 multi, one token, S=%d" % splits)
            assert_close_out(to_f64(o2), ro, "fp8 single token (pair kernel), S=%d" % splits)


@pytest.mark.parametrize("n_tok,splits", [(1, 1), (2, 4), (4, 1), (8, 4), (8, 16)])
def test_paged_fp8_multi_decode(n_tok, splits):
    """Over shuffled 16-token pages whose unowned slots hold NaN codes:
    against the paged E4M3 oracle, and bitwise equal to the contiguous E4M3
    multi-token decode."""
    q_lens = _q_lens(n_tok)
    p = inputs.make_paged_append_fp8(q_lens, K_LENS, 16, hq=64, hkv=8, seed=95 + n_tok + splits)
    a = inputs.make_append_fp8(q_lens, K_LENS, hq=64, hkv=8, seed=95 + n_tok + splits)
    assert np.array_equal(p.q, a.q) and np.array_equal(p.sinks, a.sinks)
    q, sinks, cq = bf16_to_device(p.q), f32_to_device(p.sinks), i32_to_device(p.cu_seqlens_q)
    qf = inputs.bf16_bits_to_f32(p.q)
    for window in (0, 128):
        o, lse = binding.decode_paged_multi_fp8(q, _u8(p.k_pages), _u8(p.v_pages), p.k_scale, p.v_scale,
                                                i32_to_device(p.block_table), i32_to_device(p.seq_lens), cq,
                                                max(q_lens), max(K_LENS), sinks, window, p.scale, splits,
                                                return_lse=True)
        o2 = binding.decode_splitkv_multi_fp8(q, _u8(a.k), _u8(a.v), a.k_scale, a.v_scale, cq,
                                              i32_to_device(a.cu_seqlens_k), max(q_lens), max(K_LENS), sinks, window,
                                              a.scale, splits)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o2.view(torch.int16)), (window, splits)
        ro, rl = decode_paged_fp8_multi_ref(qf, p.k_pages, p.v_pages, p.k_scale, p.v_scale, p.block_table, p.seq_lens,
                                            p.cu_seqlens_q, 16, p.sinks, window, p.scale)
        what = "paged fp8 multi n=%d S=%d W=%d" % (n_tok, splits, window)
        assert_close_out(to_f64(o), ro, what)
        assert_close_lse(lse.cpu().numpy(), rl, what)


def test_fp8_multi_debug_check_reports_nan_code(monkeypatch):
    monkeypatch.setenv("SINKATTN_DEBUG_CHECKS", "1")
    a = inputs.make_append_fp8([3, 2], [40, 70], hq=16, hkv=4, seed=97)
    o, _ = _run_fp8_multi(a, 0, 1)
    ro, _ = decode_fp8_multi_ref(inputs.bf16_bits_to_f32(a.q), a.k, a.v, a.k_scale, a.v_scale, a.cu_seqlens_q,
                                 a.cu_seqlens_k, a.sinks, 0, a.scale)
    assert_close_out(o, ro, "fp8 multi debug valid")
    bad = a.k.copy()
    bad[50, 1, 3] = 0x7F  # an E4M3 NaN in a key row of sequence 1
    with pytest.raises(binding.SinkAttnError) as err:
        binding.decode_splitkv_multi_fp8(bf16_to_device(a.q), _u8(bad), _u8(a.v), a.k_scale, a.v_scale,
                                         i32_to_device(a.cu_seqlens_q), i32_to_device(a.cu_seqlens_k), 3, 70,
                                         f32_to_device(a.sinks), 0, a.scale, 1)
    assert err.value.status == 1 and "k holds" in str(err.value)
