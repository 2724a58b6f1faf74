"""Plain float64 CPU oracle for grouped-query attention with a learned sink.

TEST INFRASTRUCTURE ONLY -- never imported by the product path.

What is computed (sources: Perplexity, "GPT-OSS on day 0", sections
"Hopper: attention with sinks (GQA)" and "GPT-OSS kernels / Sink attention";
NVIDIA's gpt-oss Blackwell announcement, model description paragraph, for the
alternating full-context / 128-token sliding-window layers):

* Every attention head owns one pretrained scalar, its sink ``z``.  It takes
  part in the softmax as one extra logit that has no value vector: for query
  row ``i`` of head ``h`` with valid key set ``J(i)``

      s_j  = scale * <q_i, k_j>                  (j in J(i))
      M    = max(z, max_j s_j)
      den  = exp(z - M) + sum_j exp(s_j - M)
      o_i  = sum_j exp(s_j - M) v_j / den
      lse  = M + ln(den)

  The sink is in logit units and is *not* multiplied by ``scale``.
* The Perplexity page describes the online form: a running max ``m``
  initialised to the head's sink value and a denominator ``d`` initialised
  to 1 (that is exp(z - z)); when the keys are split along the sequence, only
  the first split starts from the sink.  The online form reaches the
  definition above exactly (up to rounding), so this oracle is the definition
  itself; the split form is provided separately (``decode_split_partials_ref``
  plus ``merge_ref``) so that split invariance can be tested.
* GQA: query head ``h`` reads KV head ``h // G`` with ``G = Hq / Hkv``.
* Masks: causal, optionally restricted to a sliding window of ``W`` keys that
  includes the query itself, ``i - W < j <= i``.  Positions are local to each
  sequence of a varlen pack.

Readings taken where the pages are silent (each one is listed with its
reason in the design notes): natural-log lse that includes the sink; z = -inf
means "no sink"; an empty key set with no sink gives o = 0 and lse = -inf;
decode puts the single query at position L-1 of its sequence; split chunk 0
holds the lowest key positions and carries the sink even when it is empty.

Parity status: every function here is pinned by CPU tests against closed
forms, a library routine (torch's scaled_dot_product_attention in float64)
and brute-force enumeration; see ``tests/test_oracle_pins.py``.

Rows are independent, so the functions may evaluate the rows of a sequence in
blocks (for memory) or only a requested subset of rows (for sampled checks);
no reduction is reordered or blocked.
"""

from __future__ import annotations

import math
import os
from typing import Iterable, Optional, Sequence

import numpy as np

LOG2E = 1.0 / math.log(2.0)

_ROW_BLOCK = 256


# ---------------------------------------------------------------------------
# Masks and key ranges (integer work)
# ---------------------------------------------------------------------------

def prefill_mask_ref(length: int, window: int) -> np.ndarray:
    """Boolean [length, length] matrix; entry (i, j) is True iff key j is
    visible to query i: j <= i (causal) and, for window > 0, j > i - window.

    Source: NVIDIA gpt-oss announcement, model description (layers alternate
    between full context and a 128-token sliding window)."""
    i = np.arange(length)[:, None]
    j = np.arange(length)[None, :]
    valid = j <= i
    if window > 0:
        valid &= j > i - window
    return valid


def decode_key_range(length: int, window: int) -> tuple[int, int]:
    """Keys [lo, length) seen by the decode query at position length-1."""
    lo = max(0, length - window) if window > 0 else 0
    return lo, length


def split_chunks_ref(lo: int, hi: int, num_splits: int) -> list[tuple[int, int]]:
    """Cut [lo, hi) into num_splits contiguous chunks of ceil(n / S) keys
    (trailing chunks may be empty).  Chunk 0 holds the lowest positions.

    Source: Perplexity, "GPT-OSS on day 0", Sink attention: attention split
    along the sequence into blocks, with the sink-initialised max only in the
    first block."""
    n = hi - lo
    size = -(-n // num_splits) if n > 0 else 0
    out = []
    for s in range(num_splits):
        a = min(hi, lo + s * size)
        b = min(hi, lo + (s + 1) * size)
        out.append((a, b))
    return out


# ---------------------------------------------------------------------------
# The definition for a block of query rows against one key set
# ---------------------------------------------------------------------------

def _attend(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray,
            valid: np.ndarray, z: float, scale: float):
    """Sink attention of R query rows of one head.

    q_rows [R, D], k/v [N, D], valid bool [R, N], z the head's sink (may be
    -inf, meaning no sink).  Returns o [R, D] and lse [R] in float64.

    Source: Perplexity, "GPT-OSS on day 0", Sink attention (the sink is an
    extra softmax term that has no value vector)."""
    s = scale * (q_rows @ k.T)                      # [R, N]
    s = np.where(valid, s, -np.inf)
    row_max = s.max(axis=1) if s.shape[1] > 0 else np.full(s.shape[0], -np.inf)
    big_m = np.maximum(row_max, z)                  # M = max(z, max_j s_j)
    finite = np.isfinite(big_m)
    m_safe = np.where(finite, big_m, 0.0)
    e = np.exp(s - m_safe[:, None])                 # masked entries -> 0
    den = np.exp(z - m_safe) + e.sum(axis=1)
    num = e @ v                                     # [R, D]
    has = den > 0
    o = np.where(has[:, None], num / np.where(has, den, 1.0)[:, None], 0.0)
    lse = np.where(has, m_safe + np.log(np.where(has, den, 1.0)), -np.inf)
    return o, lse


def _as_f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# Prefill (varlen, self-attention, causal with optional window)
# ---------------------------------------------------------------------------

def _prefill_task(args):
    """One block of query rows of one GQA group: q_rows [R, G, D] at local
    positions ``pos`` [R], against keys/values [N, D] at positions lo..lo+N-1,
    with sinks z [G]."""
    (q_rows, k_g, v_g, pos, lo, z, window, scale) = args
    jj = lo + np.arange(k_g.shape[0])[None, :]
    ii = pos[:, None]
    valid = jj <= ii
    if window > 0:
        valid &= jj > ii - window
    o = np.zeros(q_rows.shape)
    lse = np.zeros(q_rows.shape[:2])
    for c in range(q_rows.shape[1]):
        o[:, c, :], lse[:, c] = _attend(q_rows[:, c, :], k_g, v_g, valid, z[c], scale)
    return o, lse


def prefill_varlen_ref(q, k, v, sinks, cu_seqlens, window: int, scale: float,
                       rows: Optional[Iterable[int]] = None,
                       workers: int = 1):
    """Varlen self-attention prefill with sinks.

    q [T, Hq, D], k/v [T, Hkv, D] (any float dtype; upcast exactly to
    float64), sinks [Hq] (None = no sink), cu_seqlens [B+1] with
    cu_seqlens[0] = 0.  Query and key lengths agree per sequence.

    Returns o [T, Hq, D] and lse [T, Hq] in float64.  When ``rows`` (global
    token indices) is given, only those rows are computed and every other
    row is NaN.  ``workers`` > 1 evaluates independent row blocks in a pool
    of spawned processes (one BLAS thread each).

    Source: Perplexity, "GPT-OSS on day 0", Sink attention; NVIDIA gpt-oss
    announcement, model description (window layers)."""
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    t_total, hq, d = q.shape
    hkv = k.shape[1]
    assert hq % hkv == 0
    group = hq // hkv
    z = np.full(hq, -np.inf) if sinks is None else _as_f64(sinks)
    cu = [int(x) for x in cu_seqlens]
    o = np.full((t_total, hq, d), np.nan)
    lse = np.full((t_total, hq), np.nan)
    wanted = None if rows is None else np.unique(np.asarray(list(rows), dtype=np.int64))

    tasks, places = [], []
    for b in range(len(cu) - 1):
        a, e = cu[b], cu[b + 1]
        if e <= a:
            continue
        if wanted is None:
            local = np.arange(e - a)
        else:
            sel = wanted[(wanted >= a) & (wanted < e)]
            if sel.size == 0:
                continue
            local = sel - a
        for start in range(0, local.size, _ROW_BLOCK):
            blk = local[start:start + _ROW_BLOCK]
            hi = int(blk.max()) + 1
            lo = max(0, int(blk.min()) - window + 1) if window > 0 else 0
            for g in range(hkv):
                heads = list(range(g * group, (g + 1) * group))
                tasks.append((_as_f64(q[a + blk][:, heads, :]), _as_f64(k[a + lo:a + hi, g, :]),
                              _as_f64(v[a + lo:a + hi, g, :]), blk, lo, z[heads], window, scale))
                places.append((a, blk, heads))

    results = _run(tasks, workers)
    for (a, blk, heads), (ob, lb) in zip(places, results):
        o[np.ix_(a + blk, heads)] = ob
        lse[np.ix_(a + blk, heads)] = lb
    return o, lse


# ---------------------------------------------------------------------------
# Decode (one query per sequence at position L-1), split-KV partials, merge
# ---------------------------------------------------------------------------

def decode_ref(q, k_cache, v_cache, cu_seqlens_k, sinks, window: int, scale: float):
    """Single-token decode against a packed KV cache.

    q [B, Hq, D]; k_cache/v_cache [Tk, Hkv, D] packed by cu_seqlens_k [B+1];
    the query of sequence b sits at position L_b - 1 and sees keys
    decode_key_range(L_b, window).  Returns o [B, Hq, D], lse [B, Hq].

    Source: Perplexity, "GPT-OSS on day 0", Sink attention (decode template
    with sinks); NVIDIA gpt-oss announcement (window layers)."""
    q = _as_f64(q)
    k_cache = _as_f64(k_cache)
    v_cache = _as_f64(v_cache)
    bsz, hq, d = q.shape
    hkv = k_cache.shape[1]
    group = hq // hkv
    z = np.full(hq, -np.inf) if sinks is None else _as_f64(sinks)
    o = np.zeros((bsz, hq, d))
    lse = np.zeros((bsz, hq))
    for b in range(bsz):
        base = int(cu_seqlens_k[b])
        length = int(cu_seqlens_k[b + 1]) - base
        lo, hi = decode_key_range(length, window)
        valid = np.ones((1, hi - lo), dtype=bool)
        for h in range(hq):
            g = h // group
            ob, lb = _attend(q[b, h][None, :], k_cache[base + lo:base + hi, g],
                             v_cache[base + lo:base + hi, g], valid, z[h], scale)
            o[b, h], lse[b, h] = ob[0], lb[0]
    return o, lse


def decode_split_partials_ref(q, k_cache, v_cache, cu_seqlens_k, sinks,
                              window: int, scale: float, num_splits: int):
    """Per-split partial results of decode: o_parts [S, B, Hq, D] (each
    normalised by its own denominator) and lse_parts [S, B, Hq].  The sink
    belongs to chunk 0 only; an empty chunk without the sink has o = 0 and
    lse = -inf.

    Source: Perplexity, "GPT-OSS on day 0", Sink attention (split along the
    sequence, max initialised to the sink in the first block only)."""
    q = _as_f64(q)
    k_cache = _as_f64(k_cache)
    v_cache = _as_f64(v_cache)
    bsz, hq, d = q.shape
    hkv = k_cache.shape[1]
    group = hq // hkv
    z = np.full(hq, -np.inf) if sinks is None else _as_f64(sinks)
    o = np.zeros((num_splits, bsz, hq, d))
    lse = np.zeros((num_splits, bsz, hq))
    for b in range(bsz):
        base = int(cu_seqlens_k[b])
        length = int(cu_seqlens_k[b + 1]) - base
        lo, hi = decode_key_range(length, window)
        for s, (a, e) in enumerate(split_chunks_ref(lo, hi, num_splits)):
            valid = np.ones((1, e - a), dtype=bool)
            for h in range(hq):
                g = h // group
                zs = z[h] if s == 0 else -np.inf
                ob, lb = _attend(q[b, h][None, :], k_cache[base + a:base + e, g],
                                 v_cache[base + a:base + e, g], valid, zs, scale)
                o[s, b, h], lse[s, b, h] = ob[0], lb[0]
    return o, lse


def merge_ref(o_parts, lse_parts):
    """Log-sum-exp merge of S partials: M = max_s lse_s, w_s = exp(lse_s - M),
    o = sum_s w_s o_s / sum_s w_s, lse = M + ln sum_s w_s; when every
    partial is empty (lse = -inf) the result is o = 0, lse = -inf.

    o_parts [S, ..., D], lse_parts [S, ...].  Source: Perplexity, "GPT-OSS on
    day 0", Sink attention (attention parallelised over the KV length, then
    combined; the combination formula is not printed, this is the standard
    log-sum-exp merge that the running max/denominator pair implies)."""
    o_parts = _as_f64(o_parts)
    lse_parts = _as_f64(lse_parts)
    big_m = lse_parts.max(axis=0)
    finite = np.isfinite(big_m)
    m_safe = np.where(finite, big_m, 0.0)
    w = np.exp(lse_parts - m_safe[None])            # empty partials -> 0
    wsum = w.sum(axis=0)
    has = wsum > 0
    num = (w[..., None] * o_parts).sum(axis=0)
    o = np.where(has[..., None], num / np.where(has, wsum, 1.0)[..., None], 0.0)
    lse = np.where(has, m_safe + np.log(np.where(has, wsum, 1.0)), -np.inf)
    return o, lse


# ---------------------------------------------------------------------------
# Process pool plumbing (independent row blocks only)
# ---------------------------------------------------------------------------

def _pool_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover - threadpoolctl is optional
        pass


def _run(tasks: Sequence, workers: int):
    if workers <= 1 or len(tasks) <= 1:
        return [_prefill_task(t) for t in tasks]
    import multiprocessing as mp
    ctx = mp.get_context("spawn")
    pool = ctx.Pool(processes=workers, initializer=_pool_init)
    try:
        return pool.map(_prefill_task, tasks, chunksize=1)
    finally:
        pool.close()
        pool.join()


def default_workers() -> int:
    """Host cores available to this process (affinity mask), at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))
