"""GPU parity of the append prefill (chunked prefill, multi-token-query
decode) against the float64 oracle: each sequence's queries are its last
tokens, the causal / window mask aligned at the bottom right.

Cases: offsets that are and are not multiples of the 32-token query tile and
the 64-key tile, one to eight queries per sequence against long caches
(draft-token verification), prompts cut into chunks (every chunk must give
the rows of the whole prefill), empty query sets, windows that do and do not
reach the cache's start, GQA groups from 1 to 32, with and without sinks,
and the debug check for a sequence with fewer keys than queries.

Bar as the rest of the library: max |err| <= 2e-2, mean |err| <= 2e-3 on the
bf16 outputs, lse within 4e-3 with an identical -inf pattern, and masks bit
for bit (one-hot V probes).
"""

import numpy as np
import pytest
import torch

from attention_gqa_flash_amd import binding, inputs
from oracle import append_mask_ref, prefill_append_ref, prefill_varlen_ref
from tests.helpers import (assert_close_lse, assert_close_out, bf16_to_device, f32_to_device, i32_to_device,
                           to_f64)

pytestmark = pytest.mark.gpu


def _run(a, window, with_sinks=True):
    q, k, v = (bf16_to_device(x) for x in (a.q, a.k, a.v))
    sinks = f32_to_device(a.sinks) if with_sinks else None
    o, lse = binding.prefill_append(q, k, v, sinks, i32_to_device(a.cu_seqlens_q), i32_to_device(a.cu_seqlens_k),
                                    max(a.q_lens), max(a.k_lens), window, a.scale, return_lse=True)
    torch.cuda.synchronize()
    return to_f64(o), lse.cpu().numpy()


def _ref(a, window, with_sinks=True, rows=None):
    qf, kf, vf = (inputs.bf16_bits_to_f32(x) for x in (a.q, a.k, a.v))
    return prefill_append_ref(qf, kf, vf, a.sinks if with_sinks else None, a.cu_seqlens_q, a.cu_seqlens_k,
                              window, a.scale, rows=rows)


@pytest.mark.parametrize("window", [0, 1, 32, 100, 128, 129, 5000])
@pytest.mark.parametrize("hq,hkv", [(64, 8), (8, 2), (32, 1), (16, 16)])
def test_append_ragged(window, hq, hkv):
    # offsets 0, 1, 31, 32, 33, 64, 100, 1000 and queries of 1 .. 300
    q_lens = [5, 1, 40, 33, 64, 300, 7, 0, 129]
    k_lens = [5, 2, 71, 65, 97, 364, 107, 3, 1129]
    a = inputs.make_append(q_lens, k_lens, hq=hq, hkv=hkv, seed=window + 7 * hq + hkv)
    o, lse = _run(a, window)
    ro, rl = _ref(a, window)
    assert_close_out(o, ro, "append W=%d G=%d" % (window, hq // hkv))
    assert_close_lse(lse, rl, "append")


@pytest.mark.parametrize("n_draft", [1, 2, 4, 8])
@pytest.mark.parametrize("window", [0, 128])
def test_multi_token_query_decode(n_draft, window):
    """Draft tokens verified against long caches: 64/8 heads, 16 sequences."""
    k_lens = [8192, 1, 37, 129, 4100, 2048, 8191, 300, 64, 65, 8192, 1000, 513, 257, 9000, 33]
    q_lens = [min(n_draft, n) for n in k_lens]
    a = inputs.make_append(q_lens, k_lens, hq=64, hkv=8, seed=n_draft + window)
    o, lse = _run(a, window)
    ro, rl = _ref(a, window)
    assert_close_out(o, ro, "draft %d W=%d" % (n_draft, window))
    assert_close_lse(lse, rl, "draft")


@pytest.mark.parametrize("window", [0, 128])
def test_chunked_prefill_gives_the_whole_prefill(window):
    """A 3000-token prompt in chunks (ragged cut points, one chunk per call
    and all chunks in one batch) reproduces the self-attention prefill."""
    length = 3000
    p = inputs.make_prefill([length], hq=64, hkv=8, seed=40 + window)
    q, k, v = (bf16_to_device(x) for x in (p.q, p.k, p.v))
    sinks = f32_to_device(p.sinks)
    whole = binding.prefill_varlen(q, k, v, sinks, i32_to_device(p.cu_seqlens), length, window, p.scale)
    qf, kf, vf = (inputs.bf16_bits_to_f32(x) for x in (p.q, p.k, p.v))
    ref, _ = prefill_varlen_ref(qf, kf, vf, p.sinks, p.cu_seqlens, window, p.scale)
    assert_close_out(to_f64(whole), ref, "whole")
    cuts = [0, 1, 500, 531, 1024, 2047, 3000]
    got = torch.empty_like(q)
    for a_, b_ in zip(cuts[:-1], cuts[1:]):
        cq = i32_to_device(np.array([0, b_ - a_]))
        ck = i32_to_device(np.array([0, b_]))
        binding.prefill_append(q[a_:b_], k[:b_], v[:b_], sinks, cq, ck, b_ - a_, b_, window, p.scale,
                               out=got[a_:b_])
    torch.cuda.synchronize()
    assert_close_out(to_f64(got), ref, "chunks, one call each")
    # all chunks in one batch: chunk c's keys are the prompt's first cuts[c+1] rows
    spans = list(zip(cuts[:-1], cuts[1:]))
    kk = torch.cat([k[:b_] for _, b_ in spans])
    vv = torch.cat([v[:b_] for _, b_ in spans])
    cq = i32_to_device(np.array(cuts))
    ck = i32_to_device(np.concatenate([[0], np.cumsum([b_ for _, b_ in spans])]))
    got2 = binding.prefill_append(q, kk, vv, sinks, cq, ck, max(b_ - a_ for a_, b_ in spans), length, window,
                                  p.scale)
    torch.cuda.synchronize()
    assert_close_out(to_f64(got2), ref, "chunks in one batch")


def test_equal_offsets_match_self_attention_prefill_bitwise():
    """Lq = Lk through the append entry point runs the same kernel work as
    sinkattn_prefill_varlen: the outputs agree bit for bit."""
    lens = [1, 77, 300, 64]
    a = inputs.make_append(lens, lens, hq=16, hkv=2, seed=5)
    q, k, v = (bf16_to_device(x) for x in (a.q, a.k, a.v))
    sinks = f32_to_device(a.sinks)
    cq = i32_to_device(a.cu_seqlens_q)
    ck = i32_to_device(a.cu_seqlens_k)  # a separate array with the same offsets
    for window in (0, 128):
        o1 = binding.prefill_append(q, k, v, sinks, cq, ck, 300, 300, window, a.scale)
        o2 = binding.prefill_varlen(q, k, v, sinks, cq, 300, window, a.scale)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_append_without_sinks():
    a = inputs.make_append([3, 50, 0], [10, 300, 2], hq=16, hkv=4, seed=6)
    for window in (0, 20):
        o, lse = _run(a, window, with_sinks=False)
        ro, rl = _ref(a, window, with_sinks=False)
        assert_close_out(o, ro, "no sinks")
        assert_close_lse(lse, rl, "no sinks")


@pytest.mark.parametrize("window", [0, 1, 63, 64, 65, 128])
def test_append_mask_bit_identical(window):
    """q = 0, sinks = 0 (uniform weights) and one-hot V: output column c of
    probe round r is exactly 0 iff key 64 r + c is outside the row's mask."""
    q_lens, k_lens = [40, 1, 97], [300, 129, 97]
    hq, hkv = 8, 1
    tq, tk = sum(q_lens), sum(k_lens)
    cq = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(k_lens)]).astype(np.int32)
    q = torch.zeros((tq, hq, 64), dtype=torch.bfloat16, device="cuda")
    k = bf16_to_device(inputs.round_to_bf16_bits(np.random.default_rng(1).standard_normal((tk, hkv, 64),
                                                                                          dtype=np.float32)))
    sinks = torch.zeros(hq, dtype=torch.float32, device="cuda")
    for r in range((max(k_lens) + 63) // 64):
        vh = np.zeros((tk, hkv, 64), dtype=np.float32)
        for b in range(len(k_lens)):
            for c in range(64):
                j = 64 * r + c
                if j < k_lens[b]:
                    vh[ck[b] + j, :, c] = 1.0
        v = bf16_to_device(inputs.round_to_bf16_bits(vh))
        o = binding.prefill_append(q, k, v, sinks, i32_to_device(cq), i32_to_device(ck), max(q_lens), max(k_lens),
                                   window, 0.125)
        torch.cuda.synchronize()
        nz = (o.float().cpu().numpy() != 0.0)
        for b in range(len(q_lens)):
            m = append_mask_ref(q_lens[b], k_lens[b], window)
            for c in range(64):
                j = 64 * r + c
                want = m[:, j] if j < k_lens[b] else np.zeros(q_lens[b], dtype=bool)
                got = nz[cq[b]:cq[b + 1], :, c]
                assert np.array_equal(got, np.repeat(want[:, None], hq, axis=1)), (b, r, c)


def test_debug_check_reports_fewer_keys_than_queries(monkeypatch):
    monkeypatch.setenv("SINKATTN_DEBUG_CHECKS", "1")
    a = inputs.make_append([4, 6], [10, 6], hq=8, hkv=2, seed=8)
    q, k, v = (bf16_to_device(x) for x in (a.q, a.k, a.v))
    sinks = f32_to_device(a.sinks)
    o = binding.prefill_append(q, k, v, sinks, i32_to_device(a.cu_seqlens_q), i32_to_device(a.cu_seqlens_k), 6, 10,
                               0, a.scale)
    torch.cuda.synchronize()
    ro, _ = _ref(a, 0)
    assert_close_out(to_f64(o), ro, "debug valid")
    bad_k = i32_to_device(np.array([0, 10, 13]))  # sequence 1: 3 keys for 6 queries
    with pytest.raises(binding.SinkAttnError) as err:
        binding.prefill_append(q, k[:13], v[:13], sinks, i32_to_device(a.cu_seqlens_q), bad_k, 6, 10, 0, a.scale)
    assert err.value.status == 1 and "fewer keys" in str(err.value)
