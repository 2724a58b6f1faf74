"""GPU parity of the split-KV append prefill (sinkattn_prefill_append_splitkv):
each 32-query tile's keys are cut into S shares whose normalised partials
are merged with the log-sum-exp merge, the sink counted in the first share
only (Perplexity, "GPT-OSS on day 0", Sink attention).  Against the float64
append oracle: ragged chunks (one query to 300) over caches of 1 to 5000
keys, sequences with no query, windows, no sinks, every group shape, S
from 2 to more shares than a tile has key tiles (empty shares), and a
256-token chunk over a 32768-token cache on sampled rows.  The result
equals the unsplit path's up to fp32 rounding.  Bars as in the rest of the
suite: max |err| <= 2e-2, mean |err| <= 2e-3, lse within 4e-3.
"""

import numpy as np
import pytest
import torch

from attention_gqa_flash_amd import binding, inputs
from oracle import prefill_append_ref
from tests.helpers import (assert_close_lse, assert_close_out, bf16_to_device, f32_to_device, i32_to_device,
                           to_f64)

pytestmark = pytest.mark.gpu

Q_LENS = [1, 33, 300, 0, 64, 5, 129]
K_LENS = [1, 1000, 5000, 40, 64, 2047, 4100]


def _run(a, window, splits, with_sinks=True):
    q, k, v = (bf16_to_device(x) for x in (a.q, a.k, a.v))
    o, lse = binding.prefill_append(q, k, v, f32_to_device(a.sinks) if with_sinks else None,
                                    i32_to_device(a.cu_seqlens_q), i32_to_device(a.cu_seqlens_k), max(a.q_lens),
                                    max(a.k_lens), window, a.scale, return_lse=True, num_splits=splits)
    torch.cuda.synchronize()
    return to_f64(o), lse.cpu().numpy()


def _ref(a, window, with_sinks=True, rows=None):
    qf, kf, vf = (inputs.bf16_bits_to_f32(x) for x in (a.q, a.k, a.v))
    return prefill_append_ref(qf, kf, vf, a.sinks if with_sinks else None, a.cu_seqlens_q, a.cu_seqlens_k, window,
                              a.scale, rows=rows)


def _owned(a):
    """Rows of o that belong to a sequence."""
    cu = a.cu_seqlens_q
    return np.concatenate([np.arange(cu[b], cu[b + 1]) for b in range(len(cu) - 1)]).astype(np.int64)


@pytest.mark.parametrize("hq,hkv", [(64, 8), (16, 2), (8, 1), (32, 16)])
@pytest.mark.parametrize("splits", [2, 3, 8, 64])
def test_split_append_prefill(hq, hkv, splits):
    a = inputs.make_append(Q_LENS, K_LENS, hq=hq, hkv=hkv, seed=900 + hq + hkv + splits)
    a.sinks[0] = -np.inf
    rows = _owned(a)
    for window in (0, 128, 1000):
        o, lse = _run(a, window, splits)
        ro, rl = _ref(a, window)
        what = "split append G=%d S=%d W=%d" % (hq // hkv, splits, window)
        assert_close_out(o[rows], ro[rows], what)
        assert_close_lse(lse[rows], rl[rows], what)


def test_split_append_prefill_without_sinks_and_against_unsplit():
    a = inputs.make_append(Q_LENS, K_LENS, hq=64, hkv=8, seed=950)
    rows = _owned(a)
    ro, rl = _ref(a, 0, with_sinks=False)
    base = None
    for splits in (1, 4, 16):
        o, lse = _run(a, 0, splits, with_sinks=False)
        assert_close_out(o[rows], ro[rows], "no sinks S=%d" % splits)
        assert_close_lse(lse[rows], rl[rows], "no sinks S=%d" % splits)
        if base is None:
            base = o
        else:
            assert_close_out(o[rows], base[rows], "S=%d against S=1" % splits)


def test_split_append_prefill_self_attention_offsets():
    """One offsets array for queries and keys (the whole prompt) also splits."""
    p = inputs.make_prefill([700, 33, 1], hq=16, hkv=2, seed=960)
    cu = i32_to_device(p.cu_seqlens)
    q, k, v = (bf16_to_device(x) for x in (p.q, p.k, p.v))
    qf, kf, vf = (inputs.bf16_bits_to_f32(x) for x in (p.q, p.k, p.v))
    ro, rl = prefill_append_ref(qf, kf, vf, p.sinks, p.cu_seqlens, p.cu_seqlens, 0, p.scale)
    o, lse = binding.prefill_append(q, k, v, f32_to_device(p.sinks), cu, cu, max(p.lengths), max(p.lengths), 0,
                                    p.scale, return_lse=True, num_splits=5)
    torch.cuda.synchronize()
    assert_close_out(to_f64(o), ro, "self-attention offsets S=5")
    assert_close_lse(lse.cpu().numpy(), rl, "self-attention offsets S=5")


@pytest.mark.parametrize("window", [0, 128])
def test_split_chunk_256_over_32768(window):
    a = inputs.make_append([256], [32768], hq=64, hkv=8, seed=970 + window)
    rows = np.unique(np.concatenate([np.arange(0, 40), np.arange(216, 256),
                                     np.random.default_rng(971).integers(0, 256, size=40)])).astype(np.int64)
    o, lse = _run(a, window, 16)
    ro, rl = _ref(a, window, rows=rows)
    what = "chunk 256 of 32768 S=16 W=%d" % window
    assert_close_out(o[rows], ro[rows], what)
    assert_close_lse(lse[rows], rl[rows], what)


# ---------------------------------------------------------------------------
# Over a paged cache (sinkattn_prefill_append_paged_splitkv)
# ---------------------------------------------------------------------------

P_Q_LENS = [5, 1, 40, 33, 64, 300, 7, 0, 129]
P_K_LENS = [5, 2, 71, 65, 97, 3364, 107, 3, 4129]


def _paged_run(p, window, splits, with_sinks=True):
    o, lse = binding.prefill_append_paged(bf16_to_device(p.q), bf16_to_device(p.k_pages), bf16_to_device(p.v_pages),
                                          i32_to_device(p.block_table), i32_to_device(p.seq_lens),
                                          i32_to_device(p.cu_seqlens_q), max(p.q_lens), max(p.k_lens),
                                          f32_to_device(p.sinks) if with_sinks else None, window, p.scale,
                                          return_lse=True, num_splits=splits)
    torch.cuda.synchronize()
    return to_f64(o), lse.cpu().numpy()


def _paged_ref(p, window, with_sinks=True):
    from oracle import decode_paged_multi_ref
    return decode_paged_multi_ref(inputs.bf16_bits_to_f32(p.q), inputs.bf16_bits_to_f32(p.k_pages),
                                  inputs.bf16_bits_to_f32(p.v_pages), p.block_table, p.seq_lens, p.cu_seqlens_q,
                                  p.page_size, p.sinks if with_sinks else None, window, p.scale)


@pytest.mark.parametrize("page_size", [16, 64, 256])
@pytest.mark.parametrize("splits", [2, 7, 32])
def test_split_paged_append_prefill(page_size, splits):
    p = inputs.make_paged_append(P_Q_LENS, P_K_LENS, page_size, hq=64, hkv=8, seed=980 + page_size + splits)
    cu = p.cu_seqlens_q
    rows = np.concatenate([np.arange(cu[b], cu[b + 1]) for b in range(len(cu) - 1)]).astype(np.int64)
    for window in (0, 128):
        o, lse = _paged_run(p, window, splits)
        ro, rl = _paged_ref(p, window)
        what = "split paged append ps=%d S=%d W=%d" % (page_size, splits, window)
        assert_close_out(o[rows], ro[rows], what)
        assert_close_lse(lse[rows], rl[rows], what)
    o, lse = _paged_run(p, 0, splits, with_sinks=False)
    ro, rl = _paged_ref(p, 0, with_sinks=False)
    assert_close_out(o[rows], ro[rows], "split paged append, no sinks")
    assert_close_lse(lse[rows], rl[rows], "split paged append, no sinks")


def test_split_debug_checks(monkeypatch):
    """SINKATTN_DEBUG_CHECKS=1 applies to the split entry point as to the
    unsplit one: valid inputs pass with the same result, a sequence with
    fewer keys than queries is reported before anything is launched."""
    a = inputs.make_append([4, 6], [10, 600], hq=8, hkv=2, seed=990)
    q, k, v = (bf16_to_device(x) for x in (a.q, a.k, a.v))
    sinks, cq, ck = f32_to_device(a.sinks), i32_to_device(a.cu_seqlens_q), i32_to_device(a.cu_seqlens_k)
    plain = binding.prefill_append(q, k, v, sinks, cq, ck, 6, 600, 0, a.scale, num_splits=3)
    torch.cuda.synchronize()
    monkeypatch.setenv("SINKATTN_DEBUG_CHECKS", "1")
    checked = binding.prefill_append(q, k, v, sinks, cq, ck, 6, 600, 0, a.scale, num_splits=3)
    torch.cuda.synchronize()
    assert torch.equal(checked, plain)
    bad_k = i32_to_device(np.array([0, 10, 13], np.int32))  # sequence 1: 3 keys for 6 queries
    with pytest.raises(binding.SinkAttnError) as err:
        binding.prefill_append(q, k[:13], v[:13], sinks, cq, bad_k, 6, 10, 0, a.scale, num_splits=3)
    assert err.value.status == 1 and "fewer keys" in str(err.value)


def test_split_append_prefill_is_deterministic():
    """Repeated calls give bit-identical outputs (no atomics: every partial
    has one writer and the merge a fixed order)."""
    a = inputs.make_append([256, 40], [32768, 900], hq=64, hkv=8, seed=995)
    q, k, v = (bf16_to_device(x) for x in (a.q, a.k, a.v))
    args = (q, k, v, f32_to_device(a.sinks), i32_to_device(a.cu_seqlens_q), i32_to_device(a.cu_seqlens_k), 256, 32768,
            0, a.scale)
    first = binding.prefill_append(*args, num_splits=8)
    for _ in range(3):
        again = binding.prefill_append(*args, num_splits=8)
        torch.cuda.synchronize()
        assert torch.equal(first, again)
