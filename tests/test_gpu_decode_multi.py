"""GPU parity of the multi-token-query decode (draft-token verification)
against the float64 append oracle: each sequence's newest Lq_b tokens are
queries against its cache, the causal / window mask aligned at the bottom
right, computed by the decode kernels with one MFMA column per (token, query
head) pair.

Every decode kernel shape is reached (two- and four-wave workgroups, head
pairs, a split per wave, a wave per KV head, window layers evaluated as one
range), with 1 to 8 tokens per sequence, sequences with no query, caches
shorter than a tile, several split counts (the results must agree with the
oracle at every S), with and without sinks.  Bar: max |err| <= 2e-2, mean
|err| <= 2e-3, lse within 4e-3 with an identical -inf pattern.
"""

import numpy as np
import pytest
import torch

from attention_gqa_flash_amd import binding, inputs
from oracle import prefill_append_ref
from tests.helpers import (assert_close_lse, assert_close_out, bf16_to_device, f32_to_device, i32_to_device,
                           to_f64)

pytestmark = pytest.mark.gpu


def _run(a, window, splits, with_sinks=True):
    q, k, v = (bf16_to_device(x) for x in (a.q, a.k, a.v))
    o, lse = binding.decode_splitkv_multi(q, k, v, i32_to_device(a.cu_seqlens_q), i32_to_device(a.cu_seqlens_k),
                                          max(a.q_lens), max(a.k_lens), f32_to_device(a.sinks) if with_sinks else None,
                                          window, a.scale, splits, return_lse=True)
    torch.cuda.synchronize()
    return to_f64(o), lse.cpu().numpy()


def _ref(a, window, with_sinks=True):
    qf, kf, vf = (inputs.bf16_bits_to_f32(x) for x in (a.q, a.k, a.v))
    return prefill_append_ref(qf, kf, vf, a.sinks if with_sinks else None, a.cu_seqlens_q, a.cu_seqlens_k, window,
                              a.scale)


K_LENS = [1, 31, 300, 1500, 2100, 64, 5000]


@pytest.mark.parametrize("hq,hkv,n_tok", [(64, 8, 4), (64, 8, 2), (16, 2, 3), (8, 2, 8), (32, 1, 1), (20, 5, 6),
                                          (32, 8, 8)])
@pytest.mark.parametrize("splits", [1, 2, 4, 16])
def test_multi_decode_kernel_shapes(hq, hkv, n_tok, splits):
    q_lens = [min(n_tok, n) for n in K_LENS]
    q_lens[5] = 0  # a sequence with no query this step
    a = inputs.make_append(q_lens, K_LENS, hq=hq, hkv=hkv, seed=hq + 3 * hkv + 11 * n_tok + splits)
    a.sinks[0] = -np.inf
    for window in (0, 128, 1800):
        o, lse = _run(a, window, splits)
        ro, rl = _ref(a, window)
        what = "multi G=%d n=%d S=%d W=%d" % (hq // hkv, n_tok, splits, window)
        assert_close_out(o, ro, what)
        assert_close_lse(lse, rl, what)


@pytest.mark.parametrize("splits", [1, 4, 32])
def test_multi_decode_gptoss_shape_and_no_sinks(splits):
    """64/8 heads, 4 draft tokens, 32 sequences of 8192 and one of 32768
    cached tokens; full and 128-window layers; without sinks too."""
    k_lens = [8192] * 8 + [32768, 4097, 129, 4]
    q_lens = [4] * 11 + [3]
    a = inputs.make_append(q_lens, k_lens, hq=64, hkv=8, seed=50 + splits, sink_std=2 ** 0.5)
    for window in (0, 128):
        for with_sinks in (True, False):
            o, lse = _run(a, window, splits, with_sinks)
            ro, rl = _ref(a, window, with_sinks)
            assert_close_out(o, ro, "gpt-oss multi S=%d W=%d sinks=%s" % (splits, window, with_sinks))
            assert_close_lse(lse, rl, "gpt-oss multi")


def test_multi_decode_one_token_equals_single_token_decode():
    """Lq_b = 1 everywhere: the same numbers as sinkattn_decode_splitkv."""
    k_lens = [700, 1, 4096, 33]
    a = inputs.make_append([1] * 4, k_lens, hq=64, hkv=8, seed=60)
    q, k, v = (bf16_to_device(x) for x in (a.q, a.k, a.v))
    sinks = f32_to_device(a.sinks)
    cq, ck = i32_to_device(a.cu_seqlens_q), i32_to_device(a.cu_seqlens_k)
    for splits in (1, 4):
        o1 = binding.decode_splitkv_multi(q, k, v, cq, ck, 1, 4096, sinks, 0, a.scale, splits)
        o2 = binding.decode_splitkv(q, k, v, ck, 4096, sinks, 0, a.scale, splits)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_multi_decode_debug_check(monkeypatch):
    monkeypatch.setenv("SINKATTN_DEBUG_CHECKS", "1")
    a = inputs.make_append([2, 3], [10, 3], hq=16, hkv=4, seed=61)
    o, _ = _run(a, 0, 1)
    ro, _ = _ref(a, 0)
    assert_close_out(o, ro, "debug valid")
    q, k, v = (bf16_to_device(x) for x in (a.q, a.k, a.v))
    bad_k = i32_to_device(np.array([0, 10, 12]))  # sequence 1: 2 keys for 3 queries
    with pytest.raises(binding.SinkAttnError) as err:
        binding.decode_splitkv_multi(q, k[:12], v[:12], i32_to_device(a.cu_seqlens_q), bad_k, 3, 10,
                                     f32_to_device(a.sinks), 0, a.scale, 1)
    assert err.value.status == 1 and "fewer keys" in str(err.value)
