"""Paged KV-cache decode for the float64 oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

A paged cache stores each sequence's keys and values in fixed-size pages of
a shared pool: K/V pages [num_pages, page_size, Hkv, D]; sequence b's token j
lives in page block_table[b, j // page_size] at slot j % page_size.  The
attention itself is the single-token decode over the sequence's tokens in
order, so the oracle gathers the rows and evaluates ``decode_ref``.

Source: the serving layout around the same decode (Perplexity, "GPT-OSS on
day 0", in-house inference engine and the FlashInfer decode template it
extends; Baseten, "How to run GPT OSS 120B at 500+ tokens per second on
NVIDIA GPUs", KV-cache-aware routing).  The pages name the KV cache but not
its layout; fixed-size pages addressed through a per-sequence table is the
layout of the inference engines they name (vLLM, SGLang, TensorRT-LLM).

An FP8 paged cache holds E4M3 codes in the same layout; the gathered codes go
through the FP8 decode (``decode_fp8_ref``, per-tensor scales).  Several
query tokens per sequence (draft-token verification against a paged cache)
follow the same rule: the gathered rows go through the append prefill
(``prefill_append_ref``: the newest tokens are the queries, bottom-right
causal).

Parity status: pinned by CPU tests (tests/test_oracle_paged.py) against the
contiguous decode (identity table), page permutations, and brute force; the
multi-token form against the contiguous append prefill under shuffled pages,
the single-token paged decode, and brute force; the FP8 form against the
contiguous FP8 decode under shuffled pages and the paged decode of the
decoded values.
"""

from __future__ import annotations

import numpy as np

from .append import prefill_append_ref
from .fp8 import decode_fp8_multi_ref, decode_fp8_ref
from .sink_attention import decode_ref


def gather_pages(pages, block_table, seq_lens, page_size: int) -> tuple[np.ndarray, np.ndarray]:
    """Rows of every sequence in order, packed: returns (rows [sum L, Hkv, D],
    cu_seqlens [B+1])."""
    pages = np.asarray(pages)
    bt = np.asarray(block_table)
    lens = [int(x) for x in seq_lens]
    out = []
    for b, length in enumerate(lens):
        j = np.arange(length)
        out.append(pages[bt[b, j // page_size], j % page_size])
    rows = np.concatenate(out, axis=0) if out else pages[:0, 0]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return rows, cu


def decode_paged_ref(q, k_pages, v_pages, block_table, seq_lens, page_size: int, sinks, window: int,
                     scale: float):
    """Single-token decode against a paged cache (float64): q [B, Hq, D];
    k_pages / v_pages [P, page_size, Hkv, D]; block_table [B, max_pages]
    int; seq_lens [B] (>= 1).  Returns o [B, Hq, D], lse [B, Hq]."""
    k, cu = gather_pages(k_pages, block_table, seq_lens, page_size)
    v, _ = gather_pages(v_pages, block_table, seq_lens, page_size)
    return decode_ref(q, k, v, cu, sinks, window, scale)


def decode_paged_multi_ref(q, k_pages, v_pages, block_table, seq_lens, cu_seqlens_q, page_size: int, sinks,
                           window: int, scale: float, rows=None):
    """Several query tokens per sequence against a paged cache (float64),
    whether a few draft tokens or a prompt chunk (the append prefill over
    pages computes the same thing):
    q [Tq, Hq, D], sequence b's queries are rows cu_seqlens_q[b] ..
    cu_seqlens_q[b+1] - 1, its newest Lq_b <= seq_lens[b] tokens; pages and
    table as ``decode_paged_ref``.  Returns o [Tq, Hq, D], lse [Tq, Hq]."""
    k, cu = gather_pages(k_pages, block_table, seq_lens, page_size)
    v, _ = gather_pages(v_pages, block_table, seq_lens, page_size)
    return prefill_append_ref(q, k, v, sinks, cu_seqlens_q, cu, window, scale, rows=rows)


def decode_paged_fp8_ref(q, k_pages, v_pages, k_scale: float, v_scale: float, block_table, seq_lens,
                         page_size: int, sinks, window: int, scale: float):
    """Single-token decode against a paged cache of E4M3 codes (float64):
    k_pages / v_pages uint8 [P, page_size, Hkv, D]; K = k_scale * e4m3(code),
    V = v_scale * e4m3(code); everything else as ``decode_paged_ref``."""
    k, cu = gather_pages(k_pages, block_table, seq_lens, page_size)
    v, _ = gather_pages(v_pages, block_table, seq_lens, page_size)
    return decode_fp8_ref(q, k, v, k_scale, v_scale, cu, sinks, window, scale)


def decode_paged_fp8_multi_ref(q, k_pages, v_pages, k_scale: float, v_scale: float, block_table, seq_lens,
                               cu_seqlens_q, page_size: int, sinks, window: int, scale: float, rows=None):
    """Several query tokens per sequence against a paged cache of E4M3
    codes (float64): queries as ``decode_paged_multi_ref``, pages, table and
    scales as ``decode_paged_fp8_ref``."""
    k, cu = gather_pages(k_pages, block_table, seq_lens, page_size)
    v, _ = gather_pages(v_pages, block_table, seq_lens, page_size)
    return decode_fp8_multi_ref(q, k, v, k_scale, v_scale, cu_seqlens_q, cu, sinks, window, scale, rows=rows)
