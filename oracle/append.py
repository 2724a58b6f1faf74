"""Append (chunked) prefill and multi-token-query decode for the float64 oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed: new query tokens attend to a sequence whose key/value rows
already hold every token up to and including themselves.  Sequence b has
``Lk_b`` key rows and its last ``Lq_b <= Lk_b`` tokens are the queries, so
query ``i`` (0-based among the queries) sits at position ``p = Lk_b - Lq_b + i``
of the sequence and sees the keys ``j <= p`` (and ``j > p - W`` for a window
of ``W`` keys): the causal mask aligned at the bottom right.  With
``Lq_b = Lk_b`` this is self-attention prefill; with ``Lq_b = 1`` it is the
single-token decode; in between it is a chunk of a longer prompt (chunked
prefill) or the draft tokens a speculative or multi-token-prediction decoder
hands to the target model for verification.

Sources: Perplexity, "GPT-OSS on day 0", section "In-house inference engine"
(the engine's decoders include speculative and MTP decoding) and
"GPT-OSS kernels / Sink attention" (the sink, the online softmax);
Baseten, "How to run GPT OSS 120B at 500+ tokens per second on NVIDIA GPUs",
sections "Key to optimizing inference performance" and "Next performance
optimizations" (draft tokens predicted by a smaller model and verified by the
target model); NVIDIA's gpt-oss announcement, model description (128-token
window layers).  The pages do not state the alignment of the causal mask for
queries appended to a cache; bottom-right (the queries are the newest tokens)
is the only reading under which decode and prefill are special cases.

Parity status: pinned by CPU tests (tests/test_oracle_append.py) against
brute-force enumeration, the self-attention prefill and decode special cases,
chunked-prefill invariance, and torch's scaled_dot_product_attention with an
explicit bottom-right mask.
"""

from __future__ import annotations

from typing import Iterable, Optional

import numpy as np

from .sink_attention import _attend, _as_f64

_ROW_BLOCK = 256


def append_mask_ref(q_len: int, k_len: int, window: int) -> np.ndarray:
    """Boolean [q_len, k_len]; (i, j) is True iff key j is visible to query i,
    which sits at position k_len - q_len + i: j <= that position and, for a
    window W > 0, j > position - W."""
    assert 0 <= q_len <= k_len
    pos = (k_len - q_len) + np.arange(q_len)[:, None]
    j = np.arange(k_len)[None, :]
    valid = j <= pos
    if window > 0:
        valid &= j > pos - window
    return valid


def append_mask_cols_ref(q_len: int, k_len: int, window: int, cols) -> np.ndarray:
    """Columns `cols` (key positions; positions outside [0, k_len) are never
    visible) of append_mask_ref(q_len, k_len, window), Boolean
    [q_len, len(cols)], without forming the whole [q_len, k_len] matrix: for
    the mask probes of long sequences.  q_len = k_len is the prefill mask."""
    assert 0 <= q_len <= k_len
    pos = (k_len - q_len) + np.arange(q_len)[:, None]
    j = np.asarray(cols, dtype=np.int64)[None, :]
    valid = (j >= 0) & (j < k_len) & (j <= pos)
    if window > 0:
        valid &= j > pos - window
    return valid


def prefill_append_ref(q, k, v, sinks, cu_seqlens_q, cu_seqlens_k, window: int, scale: float,
                       rows: Optional[Iterable[int]] = None):
    """Append prefill with sinks, float64.

    q [Tq, Hq, D] packed by cu_seqlens_q [B+1]; k/v [Tk, Hkv, D] packed by
    cu_seqlens_k [B+1]; per sequence Lq_b <= Lk_b.  sinks [Hq] (None = no
    sink).  Returns o [Tq, Hq, D] and lse [Tq, Hq]; with ``rows`` (global
    query-token indices) only those rows are computed, the rest are NaN."""
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    tq, hq, d = q.shape
    hkv = k.shape[1]
    assert hq % hkv == 0
    group = hq // hkv
    z = np.full(hq, -np.inf) if sinks is None else _as_f64(sinks)
    cq = [int(x) for x in cu_seqlens_q]
    ck = [int(x) for x in cu_seqlens_k]
    assert len(cq) == len(ck)
    o = np.full((tq, hq, d), np.nan)
    lse = np.full((tq, hq), np.nan)
    wanted = None if rows is None else np.unique(np.asarray(list(rows), dtype=np.int64))
    for b in range(len(cq) - 1):
        qa, lq = cq[b], cq[b + 1] - cq[b]
        ka, lk = ck[b], ck[b + 1] - ck[b]
        assert 0 <= lq <= lk, "each sequence needs at least as many keys as queries"
        if lq == 0:
            continue
        if wanted is None:
            local = np.arange(lq)
        else:
            local = wanted[(wanted >= qa) & (wanted < qa + lq)] - qa
        off = lk - lq
        for start in range(0, local.size, _ROW_BLOCK):
            blk = local[start:start + _ROW_BLOCK]
            pos = off + blk                                   # positions in the sequence
            hi = int(pos.max()) + 1
            lo = max(0, int(pos.min()) - window + 1) if window > 0 else 0
            jj = np.arange(lo, hi)[None, :]
            valid = jj <= pos[:, None]
            if window > 0:
                valid &= jj > pos[:, None] - window
            for h in range(hq):
                g = h // group
                ob, lb = _attend(_as_f64(q[qa + blk, h, :]), _as_f64(k[ka + lo:ka + hi, g, :]),
                                 _as_f64(v[ka + lo:ka + hi, g, :]), valid, z[h], scale)
                o[qa + blk, h, :] = ob
                lse[qa + blk, h] = lb
    return o, lse
