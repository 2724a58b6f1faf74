"""Pins for the append-prefill oracle (CPU).

Query tokens appended to a sequence sit at its last positions (bottom-right
causal alignment): query i of Lq sees keys j <= Lk - Lq + i, and j > that
position - W for a window of W keys.  Pinned against things other than the
function itself:

* brute-force enumeration with Python loops, math.exp and math.fsum;
* torch's scaled_dot_product_attention in float64 with an explicit boolean
  mask and the sink as one zero key / zero value whose additive mask entry is
  the sink logit;
* special cases: Lq = Lk is self-attention prefill, Lq = 1 is decode;
* chunked-prefill invariance: a prompt's queries cut into chunks, each chunk
  attending to every key up to its end, give the rows of the whole prefill.

Sources: Perplexity, "GPT-OSS on day 0" (in-house inference engine:
speculative and MTP decoders; sink attention); Baseten, "How to run GPT OSS
120B at 500+ tokens per second on NVIDIA GPUs" (draft tokens verified by the
target model).
"""

import math

import numpy as np
import pytest
import torch

from oracle import append_mask_cols_ref, append_mask_ref, decode_ref, prefill_append_ref, prefill_varlen_ref


def _cu(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)


def _case(rng, q_lens, k_lens, hq, hkv, d, sink_scale=1.0):
    q = rng.standard_normal((sum(q_lens), hq, d))
    k = rng.standard_normal((sum(k_lens), hkv, d))
    v = rng.standard_normal((sum(k_lens), hkv, d))
    sinks = sink_scale * rng.standard_normal(hq)
    return q, k, v, sinks


def _brute(q, k, v, sinks, q_lens, k_lens, window, scale):
    hq, d = q.shape[1], q.shape[2]
    g = hq // k.shape[1]
    o = np.zeros(q.shape)
    lse = np.zeros(q.shape[:2])
    qa = ka = 0
    for lq, lk in zip(q_lens, k_lens):
        for i in range(lq):
            p = lk - lq + i
            keys = [j for j in range(lk) if j <= p and (window <= 0 or j > p - window)]
            for h in range(hq):
                z = sinks[h]
                logits = [scale * math.fsum(q[qa + i, h, c] * k[ka + j, h // g, c] for c in range(d)) for j in keys]
                mx = max(logits + [z])
                w = [math.exp(s - mx) for s in logits]
                den = math.fsum(w + [math.exp(z - mx)])
                for c in range(d):
                    o[qa + i, h, c] = math.fsum(wj * v[ka + j, h // g, c] for wj, j in zip(w, keys)) / den
                lse[qa + i, h] = mx + math.log(den)
        qa += lq
        ka += lk
    return o, lse


@pytest.mark.parametrize("window", [0, 1, 2, 3, 5, 9])
def test_brute_force(window):
    rng = np.random.default_rng(100 + window)
    q_lens, k_lens = [1, 3, 5, 0, 2], [1, 7, 5, 4, 9]
    q, k, v, sinks = _case(rng, q_lens, k_lens, 4, 2, 3)
    o, lse = prefill_append_ref(q, k, v, sinks, _cu(q_lens), _cu(k_lens), window, 0.6)
    bo, bl = _brute(q, k, v, sinks, q_lens, k_lens, window, 0.6)
    assert np.max(np.abs(o - bo)) < 1e-12
    assert np.max(np.abs(lse - bl)) < 1e-12


@pytest.mark.parametrize("window", [0, 1, 4, 33])
def test_matches_sdpa_with_bottom_right_mask(window):
    rng = np.random.default_rng(7 + window)
    lq, lk, hq, hkv, d = 17, 50, 8, 2, 16
    q, k, v, sinks = _case(rng, [lq], [lk], hq, hkv, d)
    scale = 0.25
    allowed = torch.zeros(lq, lk, dtype=torch.bool)
    for i in range(lq):
        p = lk - lq + i
        first = 0 if window <= 0 else max(0, p - window + 1)
        allowed[i, first:p + 1] = True
    g = hq // hkv
    qt = torch.from_numpy(q).permute(1, 0, 2).contiguous()
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(g, dim=0)
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(g, dim=0)
    kt = torch.cat([kt, torch.zeros(hq, 1, d, dtype=torch.float64)], dim=1).contiguous()
    vt = torch.cat([vt, torch.zeros(hq, 1, d, dtype=torch.float64)], dim=1).contiguous()
    bias = torch.full((hq, lq, lk + 1), float("-inf"), dtype=torch.float64)
    bias[:, :, :lk] = torch.where(allowed, 0.0, float("-inf")).to(torch.float64)
    bias[:, :, lk] = torch.from_numpy(sinks)[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=bias, scale=scale)
    o, _ = prefill_append_ref(q, k, v, sinks, [0, lq], [0, lk], window, scale)
    assert np.max(np.abs(o - ref.permute(1, 0, 2).numpy())) < 1e-12


@pytest.mark.parametrize("window", [0, 3, 64])
def test_equal_lengths_is_self_attention_prefill(window):
    rng = np.random.default_rng(3)
    lens = [9, 1, 40, 23]
    q, k, v, sinks = _case(rng, lens, lens, 8, 2, 8)
    sinks[1] = -np.inf
    o, lse = prefill_append_ref(q, k, v, sinks, _cu(lens), _cu(lens), window, 0.3)
    ro, rl = prefill_varlen_ref(q, k, v, sinks, _cu(lens), window, 0.3)
    assert np.max(np.abs(o - ro)) < 1e-13
    assert np.array_equal(np.isinf(lse), np.isinf(rl))
    assert np.max(np.abs(lse - rl)) < 1e-13


@pytest.mark.parametrize("window", [0, 1, 5, 200])
def test_one_query_is_decode(window):
    rng = np.random.default_rng(4)
    k_lens = [1, 30, 77, 128]
    q, k, v, sinks = _case(rng, [1] * 4, k_lens, 16, 4, 8)
    o, lse = prefill_append_ref(q, k, v, sinks, _cu([1] * 4), _cu(k_lens), window, 0.2)
    ro, rl = decode_ref(q, k, v, _cu(k_lens), sinks, window, 0.2)
    assert np.max(np.abs(o - ro)) < 1e-13
    assert np.max(np.abs(lse - rl)) < 1e-13


@pytest.mark.parametrize("window", [0, 7])
def test_chunked_prefill_reproduces_whole_prefill(window):
    rng = np.random.default_rng(5)
    length = 61
    q, k, v, sinks = _case(rng, [length], [length], 8, 1, 8)
    whole, whole_lse = prefill_varlen_ref(q, k, v, sinks, [0, length], window, 0.4)
    cuts = [0, 13, 14, 40, 61]
    for a, b in zip(cuts[:-1], cuts[1:]):
        o, lse = prefill_append_ref(q[a:b], k[:b], v[:b], sinks, [0, b - a], [0, b], window, 0.4)
        assert np.max(np.abs(o - whole[a:b])) < 1e-13
        assert np.max(np.abs(lse - whole_lse[a:b])) < 1e-13


def test_rows_subset_and_mask():
    rng = np.random.default_rng(6)
    q_lens, k_lens = [5, 12], [20, 12]
    q, k, v, sinks = _case(rng, q_lens, k_lens, 4, 4, 4)
    full, _ = prefill_append_ref(q, k, v, sinks, _cu(q_lens), _cu(k_lens), 4, 0.5)
    part, _ = prefill_append_ref(q, k, v, sinks, _cu(q_lens), _cu(k_lens), 4, 0.5, rows=[0, 4, 9, 16])
    for r in [0, 4, 9, 16]:
        assert np.max(np.abs(part[r] - full[r])) < 1e-14  # (BLAS may round other shapes differently)
    assert np.isnan(part[1]).all()
    m = append_mask_ref(3, 6, 2)
    assert m.tolist() == [[False, False, True, True, False, False],
                          [False, False, False, True, True, False],
                          [False, False, False, False, True, True]]
    assert append_mask_ref(4, 4, 0).tolist() == np.tril(np.ones((4, 4), dtype=bool)).tolist()


@pytest.mark.parametrize("q_len,k_len", [(1, 1), (5, 9), (70, 70), (3, 200), (130, 130)])
@pytest.mark.parametrize("window", [0, 1, 64, 128, 129, 500])
def test_mask_columns_equal_columns_of_the_whole_mask(q_len, k_len, window):
    """The column form used by the long-sequence mask probes equals the
    columns of the whole mask (brute force below); keys outside the sequence
    are never visible."""
    cols = np.array([-3, -1, 0, 1, 31, 32, 63, 64, 65, 127, 128, 129, k_len - 1, k_len, k_len + 40])
    got = append_mask_cols_ref(q_len, k_len, window, cols)
    whole = append_mask_ref(q_len, k_len, window)
    for c_i, c in enumerate(cols):
        if 0 <= c < k_len:
            assert np.array_equal(got[:, c_i], whole[:, c]), (c, window)
        else:
            assert not got[:, c_i].any()
    off = k_len - q_len
    brute = np.array([[0 <= c < k_len and c <= off + i and (window <= 0 or c > off + i - window) for c in cols]
                      for i in range(q_len)])
    assert np.array_equal(got, brute)
