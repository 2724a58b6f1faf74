"""Bit-identical masking at the production shapes, on sampled probe rounds.

The probe of tests/test_gpu_masks.py (q = 0, so every visible key gets a
weight 1 / (|J(i)| + e^z) > 0; one-hot V with V[j, :, c] = 1 iff the key's
local position j is 64 r + c in round r): output element (i, h, c) is exactly
0.0 iff key 64 r + c is not visible to row i.  Here at the shapes the
benchmark and the named workloads run:

* the 1 x 8192 prefill with 64 / 8 heads, causal and 128-window (the
  window layer of NVIDIA's gpt-oss announcement, model description), on the
  rounds at the first tiles, the middle and the end of the sequence;
* the ragged pack of 32 sequences (log-uniform lengths 128..32768, seed 0,
  heads 0, 9, 18, 27 without sink), causal and 128-window, on the first
  rounds and the last round of several sequences;
* draft tokens against a cache (1 to 8 queries per sequence, 8 to 64
  (token, head) columns; Perplexity, "GPT-OSS on day 0", in-house inference
  engine) through the multi-token decode, bf16 and E4M3 caches, contiguous
  and paged, windows 0 / 1 / 127 / 128 / 129, 1 / 4 / 16 splits, on the
  rounds at the diagonal and around the window edge.

The zero pattern is compared with the oracle's integer mask
(append_mask_cols_ref; q_len = k_len is the prefill mask) bit for bit.  Every
head must show the same pattern.
"""

import numpy as np
import pytest
import torch

from attention_gqa_flash_amd import binding, inputs
from oracle import append_mask_cols_ref
from tests.helpers import i32_to_device

pytestmark = pytest.mark.gpu

HQ, HKV = 64, 8


def _sinks(hq, no_sink=()):
    s = torch.zeros(hq, dtype=torch.float32, device="cuda")
    if no_sink:
        s[list(no_sink)] = float("-inf")
    return s


def _one_hot_rows(cu_k, k_lens, r):
    """Rows of the packed keys and the V column that are 1 in round r."""
    rows, cols = [], []
    for b, n in enumerate(k_lens):
        c = np.arange(64)
        j = 64 * r + c
        ok = j < n
        rows.append(int(cu_k[b]) + j[ok])
        cols.append(c[ok])
    return np.concatenate(rows), np.concatenate(cols)


def _one_hot_v_device(cu_k, k_lens, hkv, r):
    v = torch.zeros((int(cu_k[-1]), hkv, 64), dtype=torch.bfloat16, device="cuda")
    rows, cols = _one_hot_rows(cu_k, k_lens, r)
    if rows.size:
        v[torch.from_numpy(rows).cuda(), :, torch.from_numpy(cols).cuda()] = 1.0
    return v


def _pattern(o):
    """[rows, 64] visibility pattern; every head must agree."""
    nz = o != 0
    every, some = nz.all(dim=1), nz.any(dim=1)
    assert torch.equal(every, some), "heads disagree on the mask"
    return every.cpu().numpy()


def _check_rows(got, q_lens, k_lens, cu_q, window, r, what):
    keys = 64 * r + np.arange(64)
    for b, (nq, nk) in enumerate(zip(q_lens, k_lens)):
        expect = append_mask_cols_ref(nq, nk, window, keys)
        assert np.array_equal(got[cu_q[b]:cu_q[b] + nq], expect), (what, window, r, b, nq, nk)


@pytest.mark.parametrize("window", [0, 128])
def test_prefill_mask_8192(window):
    n = 8192
    cu = np.array([0, n], dtype=np.int32)
    cu_d = i32_to_device(cu)
    q = torch.zeros((n, HQ, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((n, HKV, 64), dtype=torch.bfloat16, device="cuda")
    sinks = _sinks(HQ)
    o = torch.empty_like(q)
    for r in (0, 1, 2, 3, 4, 63, 64, 65, 125, 126, 127):
        v = _one_hot_v_device(cu, [n], HKV, r)
        binding.prefill_varlen(q, k, v, sinks, cu_d, n, window, 0.125, out=o)
        _check_rows(_pattern(o), [n], [n], cu, window, r, "prefill 8192")


@pytest.mark.parametrize("window", [0, 128])
def test_prefill_mask_ragged_pack(window):
    lengths = [int(x) for x in inputs.ragged_lengths(np.random.default_rng(0), 32)]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    t, lmax = int(cu[-1]), max(lengths)
    cu_d = i32_to_device(cu)
    q = torch.zeros((t, HQ, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((t, HKV, 64), dtype=torch.bfloat16, device="cuda")
    sinks = _sinks(HQ, inputs.NO_SINK_HEADS)
    o = torch.empty_like(q)
    ends = sorted(set((n - 1) // 64 for n in sorted(lengths)[::4]))
    for r in sorted(set([0, 1, 2, 3] + ends + [(lmax - 1) // 64])):
        v = _one_hot_v_device(cu, lengths, HKV, r)
        binding.prefill_varlen(q, k, v, sinks, cu_d, lmax, window, 0.125, out=o)
        _check_rows(_pattern(o), lengths, lengths, cu, window, r, "ragged")
    del q, k, o
    torch.cuda.empty_cache()


def _pages(v_bits, cu_k, k_lens, page_size, seed, fill):
    """Scatter packed rows into a shuffled page pool (spare pages and unowned
    slots hold the NaN pattern `fill`)."""
    rng = np.random.default_rng(seed)
    zeros = np.zeros_like(v_bits)
    kp, vp, bt = inputs._scatter_pages(zeros, v_bits, cu_k, k_lens, page_size, rng, 3, fill)
    return kp, vp, bt


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "e4m3"])
@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged16"])
@pytest.mark.parametrize("hq,lq", [(64, 1), (64, 2), (64, 4), (32, 8), (64, 8)])
def test_draft_token_decode_mask(paged, hq, lq, fp8):
    hkv = 8
    k_lens = [lq, 127 + lq, 128 + lq, 129 + lq, 1000, 8192]
    q_lens = [lq, lq, lq, max(1, lq - 1), lq, lq]
    cu_k = np.concatenate([[0], np.cumsum(k_lens)]).astype(np.int32)
    cu_q = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    tq, tk = int(cu_q[-1]), int(cu_k[-1])
    q = torch.zeros((tq, hq, 64), dtype=torch.bfloat16, device="cuda")
    sinks = _sinks(hq, (0,))
    cq_d, ck_d = i32_to_device(cu_q), i32_to_device(cu_k)
    lens_d = i32_to_device(np.array(k_lens, dtype=np.int32))
    for window in (0, 1, 127, 128, 129):
        rounds = {0, 1, 2, 127}
        for nk, nq in zip(k_lens, q_lens):
            first = nk - nq - window + 1 if window > 0 else 0   # the first query's window start
            for key in (first, nk - nq, nk - 1):                # window edge, diagonal, last key
                for d in (-1, 0, 1):
                    rounds.add(max(0, key // 64 + d))
        rounds = sorted(x for x in rounds if 64 * x < max(k_lens))
        for r in rounds:
            rows, cols = _one_hot_rows(cu_k, k_lens, r)
            # one-hot V: bf16 1.0 (0x3F80) or the E4M3 code of 1.0 (0x38)
            v_bits = np.zeros((tk, hkv, 64), dtype=np.uint8 if fp8 else np.uint16)
            v_bits[rows, :, cols] = 0x38 if fp8 else 0x3F80
            if fp8:
                def dev(x):
                    return torch.from_numpy(np.ascontiguousarray(x)).cuda()
            else:
                def dev(x):
                    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
            if paged:
                kp, vp, bt = _pages(v_bits, cu_k, k_lens, 16, seed=r, fill=0x7F if fp8 else 0x7FC0)
                kp_d, vp_d, bt_d = dev(kp), dev(vp), i32_to_device(bt)
            else:
                k_d, v_d = dev(np.zeros_like(v_bits)), dev(v_bits)
            for splits in (1, 4, 16):
                if paged and fp8:
                    o = binding.decode_paged_multi_fp8(q, kp_d, vp_d, 1.0, 1.0, bt_d, lens_d, cq_d, max(q_lens),
                                                       max(k_lens), sinks, window, 0.125, splits)
                elif paged:
                    o = binding.decode_paged_multi(q, kp_d, vp_d, bt_d, lens_d, cq_d, max(q_lens), max(k_lens), sinks,
                                                   window, 0.125, splits)
                elif fp8:
                    o = binding.decode_splitkv_multi_fp8(q, k_d, v_d, 1.0, 1.0, cq_d, ck_d, max(q_lens), max(k_lens),
                                                         sinks, window, 0.125, splits)
                else:
                    o = binding.decode_splitkv_multi(q, k_d, v_d, cq_d, ck_d, max(q_lens), max(k_lens), sinks, window,
                                                     0.125, splits)
                _check_rows(_pattern(o), q_lens, k_lens, cu_q, window, r,
                            "draft %s hq=%d lq=%d S=%d" % ("paged" if paged else "contiguous", hq, lq, splits))
