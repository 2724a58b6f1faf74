"""Pins for the paged-KV decode oracle (CPU).

K/V pages [P, page_size, Hkv, D]; token j of sequence b is page
block_table[b, j // page_size], slot j % page_size.  Pinned against the
contiguous decode (identity tables), invariance under any permutation of the
physical pages, page sizes that do and do not divide the lengths, and brute
force with Python loops.  The multi-token form (each sequence's newest tokens
are its queries) against the contiguous append prefill, the single-token paged
decode, and brute force with the bottom-right mask written out.  The FP8 form
(E4M3 codes in the pages) against the contiguous FP8 decode under any page
order, and the paged decode of the scaled decoded values.
"""

import math

import numpy as np
import pytest

from oracle import (decode_fp8_ref, decode_paged_fp8_ref, decode_paged_multi_ref, decode_paged_ref, decode_ref,
                    e4m3_to_float64, gather_pages, prefill_append_ref)


def _paged_from_contiguous(k, v, lens, page_size, rng=None, spare=3):
    """Scatter a packed cache into pages (optionally in a shuffled order, with
    spare unused pages); returns pages and the block table."""
    n_pages = [-(-n // page_size) for n in lens]
    total = sum(n_pages) + spare
    order = np.arange(total) if rng is None else rng.permutation(total)
    hkv, d = k.shape[1], k.shape[2]
    kp = np.full((total, page_size, hkv, d), np.nan)
    vp = np.full((total, page_size, hkv, d), np.nan)
    bt = np.full((len(lens), max(n_pages) + 2), -1, dtype=np.int64)
    nxt = 0
    base = 0
    for b, n in enumerate(lens):
        for p in range(n_pages[b]):
            phys = order[nxt]
            nxt += 1
            bt[b, p] = phys
            lo, hi = p * page_size, min(n, (p + 1) * page_size)
            kp[phys, :hi - lo] = k[base + lo:base + hi]
            vp[phys, :hi - lo] = v[base + lo:base + hi]
        base += n
    return kp, vp, bt


@pytest.mark.parametrize("page_size", [1, 16, 32, 48, 1000])
@pytest.mark.parametrize("window", [0, 5, 128])
def test_equals_contiguous_decode_under_any_page_order(page_size, window):
    rng = np.random.default_rng(page_size + window)
    lens = [1, 17, 300, 64, 129]
    hq, hkv, d = 16, 4, 8
    q = rng.standard_normal((len(lens), hq, d))
    k = rng.standard_normal((sum(lens), hkv, d))
    v = rng.standard_normal((sum(lens), hkv, d))
    sinks = rng.standard_normal(hq)
    cu = np.concatenate([[0], np.cumsum(lens)])
    ro, rl = decode_ref(q, k, v, cu, sinks, window, 0.3)
    for shuffle in (None, rng):
        kp, vp, bt = _paged_from_contiguous(k, v, lens, page_size, shuffle)
        o, lse = decode_paged_ref(q, kp, vp, bt, lens, page_size, sinks, window, 0.3)
        assert np.max(np.abs(o - ro)) < 1e-13 and np.max(np.abs(lse - rl)) < 1e-13


def test_gather_reads_exactly_the_table():
    pages = np.arange(6 * 4 * 1 * 1, dtype=np.float64).reshape(6, 4, 1, 1)
    bt = np.array([[5, 2, 0], [1, 4, 3]])
    rows, cu = gather_pages(pages, bt, [6, 9], 4)
    assert cu.tolist() == [0, 6, 15]
    assert rows[:, 0, 0].tolist() == [20, 21, 22, 23, 8, 9, 4, 5, 6, 7, 16, 17, 18, 19, 12]


def test_brute_force():
    rng = np.random.default_rng(9)
    page_size, lens = 3, [7, 2]
    hq, hkv, d = 4, 2, 3
    kp = rng.standard_normal((6, page_size, hkv, d))
    vp = rng.standard_normal((6, page_size, hkv, d))
    bt = np.array([[4, 0, 5], [2, 1, 3]])
    q = rng.standard_normal((2, hq, d))
    sinks = rng.standard_normal(hq)
    o, lse = decode_paged_ref(q, kp, vp, bt, lens, page_size, sinks, 0, 0.7)
    for b, n in enumerate(lens):
        for h in range(hq):
            g = h // (hq // hkv)
            rows = [(bt[b, j // page_size], j % page_size) for j in range(n)]
            logits = [0.7 * math.fsum(q[b, h, c] * kp[p, s, g, c] for c in range(d)) for p, s in rows]
            mx = max(logits + [sinks[h]])
            w = [math.exp(x - mx) for x in logits]
            den = math.fsum(w + [math.exp(sinks[h] - mx)])
            for c in range(d):
                want = math.fsum(wj * vp[p, s, g, c] for wj, (p, s) in zip(w, rows)) / den
                assert abs(o[b, h, c] - want) < 1e-12
            assert abs(lse[b, h] - (mx + math.log(den))) < 1e-12


@pytest.mark.parametrize("page_size", [1, 16, 48])
@pytest.mark.parametrize("window", [0, 5, 128])
def test_multi_equals_contiguous_append_under_any_page_order(page_size, window):
    rng = np.random.default_rng(100 + page_size + window)
    k_lens, q_lens = [1, 17, 300, 64, 129], [1, 3, 4, 0, 2]
    hq, hkv, d = 8, 2, 8
    q = rng.standard_normal((sum(q_lens), hq, d))
    k = rng.standard_normal((sum(k_lens), hkv, d))
    v = rng.standard_normal((sum(k_lens), hkv, d))
    sinks = rng.standard_normal(hq)
    cu_q = np.concatenate([[0], np.cumsum(q_lens)])
    cu_k = np.concatenate([[0], np.cumsum(k_lens)])
    ro, rl = prefill_append_ref(q, k, v, sinks, cu_q, cu_k, window, 0.3)
    for shuffle in (None, rng):
        kp, vp, bt = _paged_from_contiguous(k, v, k_lens, page_size, shuffle)
        o, lse = decode_paged_multi_ref(q, kp, vp, bt, k_lens, cu_q, page_size, sinks, window, 0.3)
        assert np.max(np.abs(o - ro)) < 1e-13 and np.max(np.abs(lse - rl)) < 1e-13


def test_multi_with_one_query_is_the_paged_decode():
    rng = np.random.default_rng(11)
    lens, page_size = [9, 33, 2], 4
    hq, hkv, d = 4, 2, 5
    k = rng.standard_normal((sum(lens), hkv, d))
    v = rng.standard_normal((sum(lens), hkv, d))
    q = rng.standard_normal((len(lens), hq, d))
    sinks = rng.standard_normal(hq)
    kp, vp, bt = _paged_from_contiguous(k, v, lens, page_size, rng)
    for window in (0, 3):
        ro, rl = decode_paged_ref(q, kp, vp, bt, lens, page_size, sinks, window, 0.4)
        o, lse = decode_paged_multi_ref(q, kp, vp, bt, lens, np.arange(len(lens) + 1), page_size, sinks, window,
                                        0.4)
        assert np.max(np.abs(o - ro)) < 1e-13 and np.max(np.abs(lse - rl)) < 1e-13


def test_multi_brute_force():
    rng = np.random.default_rng(12)
    page_size, k_lens, q_lens, window = 3, [7, 4], [3, 2], 4
    hq, hkv, d = 4, 2, 3
    kp = rng.standard_normal((6, page_size, hkv, d))
    vp = rng.standard_normal((6, page_size, hkv, d))
    bt = np.array([[4, 0, 5], [2, 1, 3]])
    cu_q = [0, 3, 5]
    q = rng.standard_normal((5, hq, d))
    sinks = rng.standard_normal(hq)
    o, lse = decode_paged_multi_ref(q, kp, vp, bt, k_lens, cu_q, page_size, sinks, window, 0.7)
    for b in range(2):
        for i in range(q_lens[b]):
            r = cu_q[b] + i
            pos = k_lens[b] - q_lens[b] + i          # the query is the sequence's token `pos`
            seen = [j for j in range(k_lens[b]) if pos - window < j <= pos]
            for h in range(hq):
                g = h // (hq // hkv)
                slots = [(bt[b, j // page_size], j % page_size) for j in seen]
                logits = [0.7 * math.fsum(q[r, h, c] * kp[p, s, g, c] for c in range(d)) for p, s in slots]
                mx = max(logits + [sinks[h]])
                w = [math.exp(x - mx) for x in logits]
                den = math.fsum(w + [math.exp(sinks[h] - mx)])
                for c in range(d):
                    want = math.fsum(wj * vp[p, s, g, c] for wj, (p, s) in zip(w, slots)) / den
                    assert abs(o[r, h, c] - want) < 1e-12
                assert abs(lse[r, h] - (mx + math.log(den))) < 1e-12


@pytest.mark.parametrize("page_size", [1, 16, 48])
@pytest.mark.parametrize("window", [0, 5])
def test_fp8_equals_contiguous_fp8_decode_and_the_decoded_paged_decode(page_size, window):
    rng = np.random.default_rng(200 + page_size + window)
    lens = [1, 17, 300, 64]
    hq, hkv, d = 8, 2, 8
    q = rng.standard_normal((len(lens), hq, d))
    codes = rng.integers(0, 256, size=(2, sum(lens), hkv, d)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38  # no NaN codes (0x38 is 1.0)
    kc, vc = codes
    sinks = rng.standard_normal(hq)
    cu = np.concatenate([[0], np.cumsum(lens)])
    ks, vs = 0.03, 0.5
    ro, rl = decode_fp8_ref(q, kc, vc, ks, vs, cu, sinks, window, 0.3)
    for shuffle in (None, rng):
        kp, vp, bt = _paged_from_contiguous(kc.astype(np.float64), vc.astype(np.float64), lens, page_size, shuffle)
        kp = np.nan_to_num(kp, nan=0.0).astype(np.uint8)
        vp = np.nan_to_num(vp, nan=0.0).astype(np.uint8)
        o, lse = decode_paged_fp8_ref(q, kp, vp, ks, vs, bt, lens, page_size, sinks, window, 0.3)
        assert np.max(np.abs(o - ro)) < 1e-13 and np.max(np.abs(lse - rl)) < 1e-13
        o2, lse2 = decode_paged_ref(q, ks * e4m3_to_float64(kp), vs * e4m3_to_float64(vp), bt, lens, page_size,
                                    sinks, window, 0.3)
        assert np.max(np.abs(o - o2)) < 1e-12 and np.max(np.abs(lse - lse2)) < 1e-12


@pytest.mark.parametrize("page_size", [1, 16, 48])
@pytest.mark.parametrize("window", [0, 5])
def test_fp8_multi_equals_contiguous_fp8_multi_under_any_page_order(page_size, window):
    from attention_gqa_flash_amd import inputs
    from oracle import decode_fp8_multi_ref, decode_paged_fp8_multi_ref
    q_lens, k_lens = [2, 1, 4, 0], [9, 64, 130, 5]
    a = inputs.make_append_fp8(q_lens, k_lens, hq=8, hkv=2, d=8, seed=300 + page_size + window)
    qf = inputs.bf16_bits_to_f32(a.q)
    ro, rl = decode_fp8_multi_ref(qf, a.k, a.v, a.k_scale, a.v_scale, a.cu_seqlens_q, a.cu_seqlens_k, a.sinks,
                                  window, a.scale)
    rng = np.random.default_rng(page_size)
    for shuffle in (None, rng):
        kp, vp, bt = _paged_from_contiguous(a.k.astype(np.float64), a.v.astype(np.float64), k_lens, page_size, shuffle)
        kp = np.nan_to_num(kp, nan=127.0).astype(np.uint8)   # unowned slots: E4M3 NaN codes
        vp = np.nan_to_num(vp, nan=127.0).astype(np.uint8)
        o, lse = decode_paged_fp8_multi_ref(qf, kp, vp, a.k_scale, a.v_scale, bt, k_lens, a.cu_seqlens_q, page_size,
                                            a.sinks, window, a.scale)
        assert np.max(np.abs(o - ro)) < 1e-13 and np.array_equal(np.isneginf(lse), np.isneginf(rl))
        fin = np.isfinite(rl)
        assert np.max(np.abs(lse[fin] - rl[fin])) < 1e-13


def test_fp8_multi_with_one_query_is_the_paged_fp8_decode():
    from attention_gqa_flash_amd import inputs
    from oracle import decode_paged_fp8_multi_ref
    p = inputs.make_paged_append_fp8([1, 1, 1], [3, 40, 77], 16, hq=8, hkv=2, seed=301)
    qf = inputs.bf16_bits_to_f32(p.q)
    for window in (0, 9):
        o1, l1 = decode_paged_fp8_multi_ref(qf, p.k_pages, p.v_pages, p.k_scale, p.v_scale, p.block_table, p.seq_lens,
                                            p.cu_seqlens_q, 16, p.sinks, window, p.scale)
        o2, l2 = decode_paged_fp8_ref(qf, p.k_pages, p.v_pages, p.k_scale, p.v_scale, p.block_table, p.seq_lens, 16,
                                      p.sinks, window, p.scale)
        assert np.allclose(o1, o2, rtol=0, atol=1e-14) and np.allclose(l1, l2, rtol=0, atol=1e-13)
