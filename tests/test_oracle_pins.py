"""Pins for the CPU oracle, against things other than the oracle itself.

Each check targets a mistake a sink-attention implementation could plausibly
make (sink dropped or scaled, wrong sign, off-by-one window, transposed
operand, wrong GQA grouping, sink in the wrong split, broken merge):

* library routine: torch's scaled_dot_product_attention in float64 on the
  CPU, with the sink realised as one extra zero key / zero value whose
  additive mask entry is the sink logit (exact sink attention through a
  library routine), and plain causal SDPA when there is no sink;
* closed forms: zero queries (uniform weights), the first token and the
  window-1 layer (logistic of the logit minus the sink), a huge sink;
* brute-force enumeration with Python loops and math.fsum on tiny shapes;
* invariants: window >= length equals full causal, split-KV invariance,
  sink-only partial merge, GQA equals MHA with repeated K/V, varlen
  repacking, o/lse consistency through a column of ones.

The definition pinned is the one on the Perplexity page "GPT-OSS on day 0"
(section "GPT-OSS kernels / Sink attention") with the window layers of the
NVIDIA gpt-oss announcement (model description).
"""

import math

import numpy as np
import pytest
import torch

from oracle import (decode_key_range, decode_ref, decode_split_partials_ref,
                    merge_ref, prefill_mask_ref, prefill_varlen_ref,
                    split_chunks_ref)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _sdpa_sequence(q, k, v, sinks, window, scale):
    """Library evaluation of one sequence: q [L, Hq, D], k/v [L, Hkv, D]."""
    length, hq, d = q.shape
    g = hq // k.shape[1]
    qt = torch.from_numpy(q).permute(1, 0, 2).contiguous()                      # [Hq, L, D]
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(g, dim=0)       # [Hq, L, D]
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(g, dim=0)
    allowed = torch.zeros(length, length, dtype=torch.bool)
    for i in range(length):
        first = 0 if window <= 0 else max(0, i - window + 1)
        allowed[i, first:i + 1] = True
    bias = torch.full((hq, length, length + 1), float("-inf"), dtype=torch.float64)
    bias[:, :, :length] = torch.where(allowed, 0.0, float("-inf")).to(torch.float64)
    if sinks is None:
        bias = bias[:, :, :length]
    else:
        kt = torch.cat([kt, torch.zeros(hq, 1, d, dtype=torch.float64)], dim=1)
        vt = torch.cat([vt, torch.zeros(hq, 1, d, dtype=torch.float64)], dim=1)
        bias[:, :, length] = torch.from_numpy(np.asarray(sinks, dtype=np.float64))[:, None]
    out = torch.nn.functional.scaled_dot_product_attention(
        qt, kt.contiguous(), vt.contiguous(), attn_mask=bias, scale=scale)
    return out.permute(1, 0, 2).numpy()


# ---------------------------------------------------------------------------
# Library routine
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("window", [0, 1, 3, 16, 40])
@pytest.mark.parametrize("hq,hkv", [(4, 1), (4, 2), (6, 3), (8, 8)])
def test_matches_sdpa_with_sink_column(window, hq, hkv):
    rng = np.random.default_rng(100 + window + 7 * hq + hkv)
    lengths = [1, 17, 40, 5]
    t = sum(lengths)
    d = 16
    q, k, v = _rand(rng, t, hq, d), _rand(rng, t, hkv, d), _rand(rng, t, hkv, d)
    sinks = 2.0 * _rand(rng, hq)
    sinks[0] = -np.inf if hq > 1 else sinks[0]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    scale = 0.37
    o, _ = prefill_varlen_ref(q, k, v, sinks, cu, window, scale)
    for b in range(len(lengths)):
        a, e = cu[b], cu[b + 1]
        ref = _sdpa_sequence(q[a:e], k[a:e], v[a:e], sinks, window, scale)
        np.testing.assert_allclose(o[a:e], ref, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("sinks_kind", ["none", "neg_inf"])
def test_no_sink_is_plain_causal_softmax(sinks_kind):
    rng = np.random.default_rng(5)
    length, hq, hkv, d = 29, 4, 2, 8
    q, k, v = _rand(rng, length, hq, d), _rand(rng, length, hkv, d), _rand(rng, length, hkv, d)
    sinks = None if sinks_kind == "none" else np.full(hq, -np.inf)
    o, lse = prefill_varlen_ref(q, k, v, sinks, [0, length], 0, 0.5)
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(2, dim=0)
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(2, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt.contiguous(), kt.contiguous(), vt.contiguous(), is_causal=True, scale=0.5)
    np.testing.assert_allclose(o, ref.permute(1, 0, 2).numpy(), rtol=1e-11, atol=1e-12)
    # lse without sink: log of the causal partition function
    logits = 0.5 * torch.einsum("hid,hjd->hij", qt, kt)
    logits = logits.masked_fill(~torch.ones(length, length, dtype=torch.bool).tril(), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(logits, dim=-1).T.numpy(), rtol=1e-12)


# ---------------------------------------------------------------------------
# Closed forms
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("window", [0, 1, 4, 9])
def test_zero_query_closed_form(window):
    """q = 0: every logit is 0, so o_i = sum_{j in J(i)} v_j / (|J(i)| + e^z)
    and lse = ln(|J(i)| + e^z)."""
    rng = np.random.default_rng(11)
    length, hq, d = 23, 3, 5
    v = _rand(rng, length, 1, d)
    k = _rand(rng, length, 1, d)
    q = np.zeros((length, hq, d))
    sinks = np.array([0.0, 1.7, -2.2])
    o, lse = prefill_varlen_ref(q, k, v, sinks, [0, length], window, 0.125)
    for i in range(length):
        first = 0 if window <= 0 else max(0, i - window + 1)
        n = i - first + 1
        vs = v[first:i + 1, 0].sum(axis=0)
        for h in range(hq):
            den = n + math.exp(sinks[h])
            np.testing.assert_allclose(o[i, h], vs / den, rtol=1e-13, atol=1e-15)
            assert lse[i, h] == pytest.approx(math.log(den), rel=1e-14)


def _logistic(x):
    return 1.0 / (1.0 + math.exp(-x))


def test_first_token_logistic():
    """J(0) = {0}: o_0 = v_0 * sigma(scale * q_0.k_0 - z)."""
    rng = np.random.default_rng(12)
    hq, d, scale = 4, 7, 0.3
    q, k, v = _rand(rng, 6, hq, d), _rand(rng, 6, 2, d), _rand(rng, 6, 2, d)
    sinks = np.array([0.4, -1.0, 2.5, 0.0])
    o, lse = prefill_varlen_ref(q, k, v, sinks, [0, 6], 0, scale)
    for h in range(hq):
        g = h // 2
        s = scale * float(q[0, h] @ k[0, g])
        np.testing.assert_allclose(o[0, h], v[0, g] * _logistic(s - sinks[h]), rtol=1e-13)
        assert lse[0, h] == pytest.approx(math.log(math.exp(s) + math.exp(sinks[h])), rel=1e-13)


def test_window_one_logistic():
    """W = 1: every query sees only itself, o_i = v_i * sigma(s_ii - z)."""
    rng = np.random.default_rng(13)
    length, hq, d, scale = 19, 2, 6, 0.8
    q, k, v = _rand(rng, length, hq, d), _rand(rng, length, 1, d), _rand(rng, length, 1, d)
    sinks = np.array([-0.3, 1.1])
    o, _ = prefill_varlen_ref(q, k, v, sinks, [0, length], 1, scale)
    for i in range(length):
        for h in range(hq):
            s = scale * float(q[i, h] @ k[i, 0])
            np.testing.assert_allclose(o[i, h], v[i, 0] * _logistic(s - sinks[h]), rtol=1e-13)


def test_huge_sink_zeroes_output():
    rng = np.random.default_rng(14)
    length, hq, d = 12, 2, 8
    q, k, v = _rand(rng, length, hq, d), _rand(rng, length, 1, d), _rand(rng, length, 1, d)
    o, lse = prefill_varlen_ref(q, k, v, np.array([1000.0, 1000.0]), [0, length], 0, 0.125)
    assert np.all(o == 0.0)
    assert np.all(lse == 1000.0)


# ---------------------------------------------------------------------------
# Brute force (tiny shapes, Python loops, math.fsum)
# ---------------------------------------------------------------------------

def _brute(q, k, v, sinks, lengths, window, scale):
    t, hq, d = q.shape
    g = hq // k.shape[1]
    o = [[[0.0] * d for _ in range(hq)] for _ in range(t)]
    lse = [[0.0] * hq for _ in range(t)]
    base = 0
    for length in lengths:
        for i in range(length):
            for h in range(hq):
                keys = [j for j in range(length) if j <= i and (window <= 0 or i - j < window)]
                logits = [scale * math.fsum(q[base + i, h, c] * k[base + j, h // g, c] for c in range(d))
                          for j in keys]
                z = float(sinks[h])
                mx = max(logits + [z])
                w = [math.exp(x - mx) for x in logits]
                den = math.fsum(w + [math.exp(z - mx)])
                for c in range(d):
                    o[base + i][h][c] = math.fsum(wj * v[base + j, h // g, c] for wj, j in zip(w, keys)) / den
                lse[base + i][h] = mx + math.log(den)
        base += length
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("window_kind", ["0", "1", "2", "3", "5", "Lm1", "L", "Lp1"])
def test_brute_force_tiny(window_kind):
    rng = np.random.default_rng(21)
    lengths = [9, 1, 14]
    lmax = max(lengths)
    window = {"Lm1": lmax - 1, "L": lmax, "Lp1": lmax + 1}.get(window_kind)
    window = int(window_kind) if window is None else window
    hq, hkv, d = 4, 2, 3
    t = sum(lengths)
    q, k, v = _rand(rng, t, hq, d), _rand(rng, t, hkv, d), _rand(rng, t, hkv, d)
    sinks = np.array([0.5, -1.5, 3.0, -np.inf])
    cu = np.concatenate([[0], np.cumsum(lengths)])
    o, lse = prefill_varlen_ref(q, k, v, sinks, cu, window, 0.7)
    bo, blse = _brute(q, k, v, sinks, lengths, window, 0.7)
    np.testing.assert_allclose(o, bo, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, blse, rtol=1e-12, atol=1e-14)


def test_decode_brute_force():
    rng = np.random.default_rng(22)
    lengths = [1, 6, 13]
    hq, hkv, d = 4, 1, 3
    q = _rand(rng, 3, hq, d)
    k, v = _rand(rng, sum(lengths), hkv, d), _rand(rng, sum(lengths), hkv, d)
    sinks = np.array([0.2, -0.7, 1.9, -np.inf])
    cu = np.concatenate([[0], np.cumsum(lengths)])
    for window in (0, 1, 4, 13):
        o, lse = decode_ref(q, k, v, cu, sinks, window, 0.9)
        for b, length in enumerate(lengths):
            kk = k[cu[b]:cu[b + 1]]
            vv = v[cu[b]:cu[b + 1]]
            # decode query = last position of a prefill whose other queries are irrelevant
            qq = np.zeros((length, hq, d))
            qq[-1] = q[b]
            bo, blse = _brute(qq, kk, vv, sinks, [length], window, 0.9)
            np.testing.assert_allclose(o[b], bo[-1], rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(lse[b], blse[-1], rtol=1e-12)


# ---------------------------------------------------------------------------
# Invariants
# ---------------------------------------------------------------------------

def test_window_at_least_length_is_full_causal():
    rng = np.random.default_rng(31)
    length, hq, d = 33, 4, 8
    q, k, v = _rand(rng, length, hq, d), _rand(rng, length, 2, d), _rand(rng, length, 2, d)
    sinks = _rand(rng, hq)
    full, full_lse = prefill_varlen_ref(q, k, v, sinks, [0, length], 0, 0.125)
    for w in (length, length + 1, 10 * length):
        o, lse = prefill_varlen_ref(q, k, v, sinks, [0, length], w, 0.125)
        np.testing.assert_array_equal(o, full)
        np.testing.assert_array_equal(lse, full_lse)
    o, _ = prefill_varlen_ref(q, k, v, sinks, [0, length], length - 1, 0.125)
    assert not np.allclose(o[-1], full[-1])


def test_gqa_equals_mha_with_repeated_kv():
    rng = np.random.default_rng(32)
    length, hq, hkv, d = 21, 8, 2, 8
    q, k, v = _rand(rng, length, hq, d), _rand(rng, length, hkv, d), _rand(rng, length, hkv, d)
    sinks = _rand(rng, hq)
    o, lse = prefill_varlen_ref(q, k, v, sinks, [0, length], 5, 0.25)
    o2, lse2 = prefill_varlen_ref(q, np.repeat(k, hq // hkv, axis=1), np.repeat(v, hq // hkv, axis=1),
                                  sinks, [0, length], 5, 0.25)
    np.testing.assert_allclose(o, o2, rtol=1e-14, atol=0)
    np.testing.assert_allclose(lse, lse2, rtol=1e-14, atol=0)


def test_varlen_repacking():
    rng = np.random.default_rng(33)
    lengths = [7, 1, 30, 12]
    hq, d = 4, 8
    t = sum(lengths)
    q, k, v = _rand(rng, t, hq, d), _rand(rng, t, 2, d), _rand(rng, t, 2, d)
    sinks = _rand(rng, hq)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    o, lse = prefill_varlen_ref(q, k, v, sinks, cu, 6, 0.125)
    order = [2, 0, 3, 1]
    pieces = [slice(cu[b], cu[b + 1]) for b in order]
    q2 = np.concatenate([q[p] for p in pieces])
    k2 = np.concatenate([k[p] for p in pieces])
    v2 = np.concatenate([v[p] for p in pieces])
    cu2 = np.concatenate([[0], np.cumsum([lengths[b] for b in order])])
    o2, lse2 = prefill_varlen_ref(q2, k2, v2, sinks, cu2, 6, 0.125)
    for new, b in enumerate(order):
        np.testing.assert_array_equal(o2[cu2[new]:cu2[new + 1]], o[cu[b]:cu[b + 1]])
        np.testing.assert_array_equal(lse2[cu2[new]:cu2[new + 1]], lse[cu[b]:cu[b + 1]])
        single, _ = prefill_varlen_ref(q[cu[b]:cu[b + 1]], k[cu[b]:cu[b + 1]], v[cu[b]:cu[b + 1]],
                                       sinks, [0, lengths[b]], 6, 0.125)
        np.testing.assert_array_equal(single, o[cu[b]:cu[b + 1]])


def test_lse_consistency_with_ones_column():
    """With V[..., c] = 1 the output column is the total non-sink weight:
    o[..., c] = 1 - exp(z - lse)."""
    rng = np.random.default_rng(34)
    length, hq, d = 25, 4, 6
    q, k, v = _rand(rng, length, hq, d), _rand(rng, length, 1, d), _rand(rng, length, 1, d)
    v[:, :, 2] = 1.0
    sinks = np.array([-1.0, 0.0, 2.0, 4.0])
    for w in (0, 3):
        o, lse = prefill_varlen_ref(q, k, v, sinks, [0, length], w, 0.5)
        np.testing.assert_allclose(o[:, :, 2], 1.0 - np.exp(sinks[None, :] - lse), rtol=1e-12, atol=1e-13)


def test_decode_equals_last_prefill_row():
    rng = np.random.default_rng(35)
    lengths = [5, 64, 130]
    hq, hkv, d = 8, 2, 16
    t = sum(lengths)
    q, k, v = _rand(rng, t, hq, d), _rand(rng, t, hkv, d), _rand(rng, t, hkv, d)
    sinks = _rand(rng, hq)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    last = cu[1:] - 1
    for w in (0, 1, 32, 128):
        po, plse = prefill_varlen_ref(q, k, v, sinks, cu, w, 0.125)
        do, dlse = decode_ref(q[last], k, v, cu, sinks, w, 0.125)
        np.testing.assert_allclose(do, po[last], rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(dlse, plse[last], rtol=1e-13)


@pytest.mark.parametrize("window", [0, 4, 100])
def test_split_invariance_and_sink_in_first_split(window):
    rng = np.random.default_rng(36)
    lengths = [1, 5, 37, 64, 200]
    hq, hkv, d = 4, 2, 8
    q = _rand(rng, len(lengths), hq, d)
    k, v = _rand(rng, sum(lengths), hkv, d), _rand(rng, sum(lengths), hkv, d)
    sinks = np.array([0.3, -np.inf, 1.5, -0.5])
    cu = np.concatenate([[0], np.cumsum(lengths)])
    o, lse = decode_ref(q, k, v, cu, sinks, window, 0.125)
    for s in (1, 2, 3, 4, 7, 16, 32):
        op, lp = decode_split_partials_ref(q, k, v, cu, sinks, window, 0.125, s)
        mo, ml = merge_ref(op, lp)
        np.testing.assert_allclose(mo, o, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(ml, lse, rtol=1e-12)
        # a sink-only partial merged into unseeded partials equals the seeded result
        up, ul = decode_split_partials_ref(q, k, v, cu, None, window, 0.125, s)
        sink_o = np.zeros((1,) + up.shape[1:])
        sink_l = np.broadcast_to(sinks[None, None, :], (1,) + ul.shape[1:])
        mo2, ml2 = merge_ref(np.concatenate([up, sink_o]), np.concatenate([ul, sink_l]))
        np.testing.assert_allclose(mo2, o, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(ml2, lse, rtol=1e-12)
    # the sink sits in chunk 0 only: with S = 32 the single-key sequence's
    # chunk 0 holds the key and the sink, later chunks are empty (-inf)
    op, lp = decode_split_partials_ref(q, k, v, cu, sinks, window, 0.125, 32)
    assert np.all(np.isneginf(lp[1:, 0]))
    assert np.all(op[1:, 0] == 0.0)


def test_merge_closed_forms():
    rng = np.random.default_rng(37)
    o1 = _rand(rng, 3, 5)
    l1 = _rand(rng, 3)
    # merging a partial with an identical copy keeps o and adds ln 2
    mo, ml = merge_ref(np.stack([o1, o1]), np.stack([l1, l1]))
    np.testing.assert_allclose(mo, o1, rtol=1e-15)
    np.testing.assert_allclose(ml, l1 + math.log(2.0), rtol=1e-15)
    # two partials: o = sigma(l1 - l2) o1 + sigma(l2 - l1) o2
    o2, l2 = _rand(rng, 3, 5), _rand(rng, 3)
    mo, ml = merge_ref(np.stack([o1, o2]), np.stack([l1, l2]))
    w1 = np.array([_logistic(a - b) for a, b in zip(l1, l2)])
    np.testing.assert_allclose(mo, w1[:, None] * o1 + (1 - w1)[:, None] * o2, rtol=1e-13)
    np.testing.assert_allclose(ml, np.logaddexp(l1, l2), rtol=1e-14)
    # all partials empty
    mo, ml = merge_ref(np.zeros((4, 2, 3)), np.full((4, 2), -np.inf))
    assert np.all(mo == 0.0) and np.all(np.isneginf(ml))


def test_mask_and_key_ranges():
    for length in (1, 2, 5, 130):
        for w in (0, 1, 2, 64, 128, 129, 1000):
            m = prefill_mask_ref(length, w)
            counts = m.sum(axis=1)
            expect = np.arange(1, length + 1) if w <= 0 else np.minimum(np.arange(1, length + 1), w)
            np.testing.assert_array_equal(counts, expect)
            assert np.all(m[np.arange(length), np.arange(length)])      # the query sees itself
            assert not np.any(np.triu(m, 1))                             # never the future
            lo, hi = decode_key_range(length, w)
            assert hi == length and hi - lo == (length if w <= 0 else min(length, w))


def test_split_chunks():
    assert split_chunks_ref(0, 10, 4) == [(0, 3), (3, 6), (6, 9), (9, 10)]
    assert split_chunks_ref(5, 7, 4) == [(5, 6), (6, 7), (7, 7), (7, 7)]
    assert split_chunks_ref(3, 3, 3) == [(3, 3)] * 3
    for n in range(0, 40):
        for s in (1, 2, 3, 7, 32):
            ch = split_chunks_ref(100, 100 + n, s)
            assert ch[0][0] == 100 and ch[-1][1] == 100 + n
            assert all(a <= b for a, b in ch)
            assert all(ch[i][1] == ch[i + 1][0] for i in range(s - 1))
            assert sum(b - a for a, b in ch) == n


def test_row_subset_matches_full():
    rng = np.random.default_rng(38)
    lengths = [300, 40]
    t = sum(lengths)
    q, k, v = _rand(rng, t, 4, 8), _rand(rng, t, 1, 8), _rand(rng, t, 1, 8)
    sinks = _rand(rng, 4)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    full, full_lse = prefill_varlen_ref(q, k, v, sinks, cu, 7, 0.125)
    rows = [0, 1, 255, 256, 257, 299, 300, 339]
    o, lse = prefill_varlen_ref(q, k, v, sinks, cu, 7, 0.125, rows=rows)
    # the key band of a row block depends on the block, so BLAS may round differently
    np.testing.assert_allclose(o[rows], full[rows], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse[rows], full_lse[rows], rtol=1e-14)
    other = np.setdiff1d(np.arange(t), rows)
    assert np.all(np.isnan(o[other]))


def test_pool_matches_serial():
    rng = np.random.default_rng(39)
    lengths = [600, 90]
    t = sum(lengths)
    q, k, v = _rand(rng, t, 4, 8), _rand(rng, t, 2, 8), _rand(rng, t, 2, 8)
    sinks = _rand(rng, 4)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    a, al = prefill_varlen_ref(q, k, v, sinks, cu, 0, 0.125)
    b, bl = prefill_varlen_ref(q, k, v, sinks, cu, 0, 0.125, workers=2)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(al, bl)
