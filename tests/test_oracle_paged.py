"""Pins for the paged-KV decode oracle (CPU).

K/V pages [P, page_size, Hkv, D]; token j of sequence b is page
block_table[b, j // page_size], slot j % page_size.  Pinned against the
contiguous decode (identity tables), invariance under any permutation of the
physical pages, page sizes that do and do not divide the lengths, and brute
force with Python loops.
"""

import math

import numpy as np
import pytest

from oracle import decode_paged_ref, decode_ref, gather_pages


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
