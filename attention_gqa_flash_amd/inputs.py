"""Seeded synthetic inputs for sink attention.

This module is shared by the tests, the benchmark and the oracle checks.  It
only draws random numbers and rounds them to bfloat16 (round to nearest
even); it holds none of the attention arithmetic.

Draw order for every workload: sequence lengths (varlen only) -> q -> k ->
v -> sinks, from ``numpy.random.default_rng(seed)``; q/k/v are standard
normals drawn in float32 and rounded to bf16, sinks stay float32.

Workloads take the GPT-OSS attention shape (64 query heads, 8 KV heads,
head_dim 64, scale 1/8) with the sequence lengths the pages measure decode
at (8192 and 32768; Perplexity, "GPT-OSS on day 0", cost and performance
section) and the 128-token window layers (NVIDIA gpt-oss announcement, model
description).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# Heads whose sink is forced to -inf in the ragged varlen workload: four
# different KV groups at four different positions inside their group.
NO_SINK_HEADS = (0, 9, 18, 27)


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even.
    Inputs are finite normals, so no NaN/Inf handling is needed."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + rounding) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal_bf16(rng: np.random.Generator, shape, std: float = 1.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return round_to_bf16_bits(x)


@dataclass
class PrefillInputs:
    q: np.ndarray            # uint16 bf16 bits [T, Hq, D]
    k: np.ndarray            # uint16 bf16 bits [T, Hkv, D]
    v: np.ndarray            # uint16 bf16 bits [T, Hkv, D]
    sinks: np.ndarray        # float32 [Hq]
    cu_seqlens: np.ndarray   # int32 [B+1]
    scale: float
    lengths: list = field(default_factory=list)

    @property
    def max_seqlen(self) -> int:
        return int(max(self.lengths)) if self.lengths else 0


@dataclass
class DecodeInputs:
    q: np.ndarray            # uint16 bf16 bits [B, Hq, D]
    k: np.ndarray            # uint16 bf16 bits [Tk, Hkv, D]
    v: np.ndarray            # uint16 bf16 bits [Tk, Hkv, D]
    sinks: np.ndarray        # float32 [Hq]
    cu_seqlens_k: np.ndarray  # int32 [B+1]
    scale: float
    lengths: list = field(default_factory=list)

    @property
    def max_seqlen(self) -> int:
        return int(max(self.lengths)) if self.lengths else 0


def _cu(lengths) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


def make_prefill(lengths, hq: int, hkv: int, d: int = 64, seed: int = 0,
                 scale: float = 0.125, sink_std: float = 1.0,
                 no_sink_heads=(), rng: Optional[np.random.Generator] = None):
    rng = rng if rng is not None else np.random.default_rng(seed)
    lengths = [int(x) for x in lengths]
    t = int(sum(lengths))
    q = _normal_bf16(rng, (t, hq, d))
    k = _normal_bf16(rng, (t, hkv, d))
    v = _normal_bf16(rng, (t, hkv, d))
    sinks = rng.standard_normal(size=hq, dtype=np.float32)
    if sink_std != 1.0:
        sinks = sinks * np.float32(sink_std)
    for h in no_sink_heads:
        sinks[h] = -np.inf
    return PrefillInputs(q, k, v, sinks.astype(np.float32), _cu(lengths), scale, lengths)


def make_decode(lengths, hq: int, hkv: int, d: int = 64, seed: int = 0,
                scale: float = 0.125, sink_std: float = 1.0,
                rng: Optional[np.random.Generator] = None):
    rng = rng if rng is not None else np.random.default_rng(seed)
    lengths = [int(x) for x in lengths]
    tk = int(sum(lengths))
    q = _normal_bf16(rng, (len(lengths), hq, d))
    k = _normal_bf16(rng, (tk, hkv, d))
    v = _normal_bf16(rng, (tk, hkv, d))
    sinks = rng.standard_normal(size=hq, dtype=np.float32)
    if sink_std != 1.0:
        sinks = sinks * np.float32(sink_std)
    return DecodeInputs(q, k, v, sinks.astype(np.float32), _cu(lengths), scale, lengths)


@dataclass
class AppendInputs:
    q: np.ndarray             # uint16 bf16 bits [Tq, Hq, D]
    k: np.ndarray             # uint16 bf16 bits [Tk, Hkv, D]
    v: np.ndarray             # uint16 bf16 bits [Tk, Hkv, D]
    sinks: np.ndarray         # float32 [Hq]
    cu_seqlens_q: np.ndarray  # int32 [B+1]
    cu_seqlens_k: np.ndarray  # int32 [B+1]
    scale: float
    q_lens: list = field(default_factory=list)
    k_lens: list = field(default_factory=list)


def make_append(q_lens, k_lens, hq: int, hkv: int, d: int = 64, seed: int = 0, scale: float = 0.125,
                sink_std: float = 1.0, rng: Optional[np.random.Generator] = None):
    """Queries appended to cached sequences: sequence b has k_lens[b] key rows
    and its last q_lens[b] <= k_lens[b] tokens are queries.  Draw order
    q -> k -> v -> sinks, N(0,1) rounded to bf16; sinks N(0, sink_std^2)."""
    rng = rng if rng is not None else np.random.default_rng(seed)
    q_lens = [int(x) for x in q_lens]
    k_lens = [int(x) for x in k_lens]
    assert len(q_lens) == len(k_lens) and all(0 <= a <= b for a, b in zip(q_lens, k_lens))
    q = _normal_bf16(rng, (sum(q_lens), hq, d))
    k = _normal_bf16(rng, (sum(k_lens), hkv, d))
    v = _normal_bf16(rng, (sum(k_lens), hkv, d))
    sinks = rng.standard_normal(size=hq, dtype=np.float32)
    if sink_std != 1.0:
        sinks = sinks * np.float32(sink_std)
    return AppendInputs(q, k, v, sinks.astype(np.float32), _cu(q_lens), _cu(k_lens), scale, q_lens, k_lens)


@dataclass
class PagedDecodeInputs:
    q: np.ndarray            # uint16 bf16 bits [B, Hq, D]
    k_pages: np.ndarray      # uint16 bf16 bits [P, page_size, Hkv, D]
    v_pages: np.ndarray
    block_table: np.ndarray  # int32 [B, max_pages] (-1 past a sequence's pages)
    seq_lens: np.ndarray     # int32 [B]
    sinks: np.ndarray        # float32 [Hq]
    page_size: int
    scale: float
    lengths: list = field(default_factory=list)


def make_paged_decode(lengths, page_size: int, hq: int, hkv: int, d: int = 64, seed: int = 0,
                      scale: float = 0.125, spare_pages: int = 3, fill_bits: int = 0x7FC0,
                      sink_std: float = 1.0, rng: Optional[np.random.Generator] = None):
    """A paged cache holding the same draws as make_decode (q -> k -> v ->
    sinks, N(0,1) rounded to bf16), scattered into pages in a random physical
    order (drawn after the sinks) with spare pages; slots no sequence owns hold
    ``fill_bits`` (a bf16 NaN by default, so that a read outside a sequence's
    tokens shows in its output)."""
    rng = rng if rng is not None else np.random.default_rng(seed)
    dec = make_decode(lengths, hq, hkv, d, rng=rng, scale=scale, sink_std=sink_std)
    kp, vp, bt = _scatter_pages(dec.k, dec.v, dec.cu_seqlens_k, dec.lengths, page_size, rng, spare_pages, fill_bits)
    return PagedDecodeInputs(dec.q, kp, vp, bt, np.asarray(dec.lengths, dtype=np.int32), dec.sinks, page_size,
                             scale, list(dec.lengths))


def _scatter_pages(k, v, cu, lengths, page_size, rng, spare_pages, fill_bits):
    """Packed rows (bf16 bits or E4M3 codes) -> pages in a random physical
    order (one permutation drawn from rng) with spare pages; unowned slots
    hold fill_bits.  Returns
    (k_pages, v_pages, block_table with -1 past each sequence's pages)."""
    hkv, d = k.shape[1], k.shape[2]
    n_pages = [-(-int(n) // page_size) for n in lengths]
    total = sum(n_pages) + spare_pages
    order = rng.permutation(total)
    kp = np.full((total, page_size, hkv, d), fill_bits, dtype=k.dtype)
    vp = np.full((total, page_size, hkv, d), fill_bits, dtype=k.dtype)
    bt = np.full((len(lengths), max(n_pages) + 1), -1, dtype=np.int32)
    nxt = 0
    for b, n in enumerate(lengths):
        base = int(cu[b])
        for p in range(n_pages[b]):
            phys = int(order[nxt])
            nxt += 1
            bt[b, p] = phys
            lo, hi = p * page_size, min(n, (p + 1) * page_size)
            kp[phys, :hi - lo] = k[base + lo:base + hi]
            vp[phys, :hi - lo] = v[base + lo:base + hi]
    return kp, vp, bt


@dataclass
class PagedAppendInputs:
    q: np.ndarray             # uint16 bf16 bits [Tq, Hq, D]
    k_pages: np.ndarray       # uint16 bf16 bits [P, page_size, Hkv, D]
    v_pages: np.ndarray
    block_table: np.ndarray   # int32 [B, max_pages] (-1 past a sequence's pages)
    seq_lens: np.ndarray      # int32 [B] (Lk_b)
    cu_seqlens_q: np.ndarray  # int32 [B+1]
    sinks: np.ndarray         # float32 [Hq]
    page_size: int
    scale: float
    q_lens: list = field(default_factory=list)
    k_lens: list = field(default_factory=list)


def make_paged_append(q_lens, k_lens, page_size: int, hq: int, hkv: int, d: int = 64, seed: int = 0,
                      scale: float = 0.125, spare_pages: int = 3, fill_bits: int = 0x7FC0,
                      rng: Optional[np.random.Generator] = None):
    """The draws of make_append (q -> k -> v -> sinks) with the cache
    scattered into pages as make_paged_decode does (permutation drawn after
    the sinks, unowned slots NaN)."""
    rng = rng if rng is not None else np.random.default_rng(seed)
    a = make_append(q_lens, k_lens, hq, hkv, d, rng=rng, scale=scale)
    kp, vp, bt = _scatter_pages(a.k, a.v, a.cu_seqlens_k, a.k_lens, page_size, rng, spare_pages, fill_bits)
    return PagedAppendInputs(a.q, kp, vp, bt, np.asarray(a.k_lens, dtype=np.int32), a.cu_seqlens_q, a.sinks,
                             page_size, scale, list(a.q_lens), list(a.k_lens))


@dataclass
class RopeInputs:
    qkv: np.ndarray           # uint16 bf16 bits [T, Hq + 2 Hkv, D]
    positions: np.ndarray     # int32 [T]
    slot_mapping: np.ndarray  # int32 [T], distinct rows or -1
    k_cache: np.ndarray       # uint16 bf16 bits [rows, Hkv, D] (initial contents)
    v_cache: np.ndarray


def make_rope(num_tokens: int, hq: int, hkv: int, cache_rows: int, d: int = 64, seed: int = 0,
              max_position: int = 131072, skip_every: int = 7, rng: Optional[np.random.Generator] = None):
    """Inputs of the fused rotary step: qkv and the caches N(0,1) rounded to
    bf16; positions uniform in [0, max_position); distinct cache rows drawn
    without replacement, every skip_every-th token without a row (-1)."""
    rng = rng if rng is not None else np.random.default_rng(seed)
    assert cache_rows >= num_tokens
    qkv = _normal_bf16(rng, (num_tokens, hq + 2 * hkv, d))
    positions = rng.integers(0, max_position, size=num_tokens).astype(np.int32)
    slots = rng.permutation(cache_rows)[:num_tokens].astype(np.int32)
    if skip_every > 0:
        slots[::skip_every] = -1
    kc = _normal_bf16(rng, (cache_rows, hkv, d))
    vc = _normal_bf16(rng, (cache_rows, hkv, d))
    return RopeInputs(qkv, positions, slots, kc, vc)


@dataclass
class DecodeFp8Inputs:
    q: np.ndarray            # uint16 bf16 bits [B, Hq, D]
    k: np.ndarray            # uint8 E4M3 codes [Tk, Hkv, D]
    v: np.ndarray            # uint8 E4M3 codes [Tk, Hkv, D]
    k_scale: float           # K = k_scale * e4m3(k)
    v_scale: float
    sinks: np.ndarray        # float32 [Hq]
    cu_seqlens_k: np.ndarray  # int32 [B+1]
    scale: float
    lengths: list = field(default_factory=list)

    @property
    def max_seqlen(self) -> int:
        return int(max(self.lengths)) if self.lengths else 0


def to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """float32 -> E4M3 codes (uint8), round to nearest even, clamped to the
    largest finite magnitude (448) first.  Encoding is done by torch's
    float8_e4m3fn cast (input generation only)."""
    import torch
    x = np.clip(np.asarray(x, dtype=np.float32), -448.0, 448.0)
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def make_decode_fp8(lengths, hq: int, hkv: int, d: int = 64, seed: int = 0,
                    scale: float = 0.125, sink_std: float = 1.0,
                    k_scale: float = 1.0 / 16, v_scale: float = 1.0 / 16,
                    rng: Optional[np.random.Generator] = None) -> DecodeFp8Inputs:
    """Decode inputs with an E4M3 KV cache: K and V are N(0,1) values divided
    by their per-tensor scale and rounded to E4M3 (the cache then holds
    k_scale * e4m3(code) ~ N(0,1) to within the format's precision).  Draw
    order as make_decode: q, k, v, sinks."""
    rng = rng if rng is not None else np.random.default_rng(seed)
    lengths = [int(x) for x in lengths]
    tk = int(sum(lengths))
    q = _normal_bf16(rng, (len(lengths), hq, d))
    k = to_e4m3_codes(rng.standard_normal(size=(tk, hkv, d), dtype=np.float32) / np.float32(k_scale))
    v = to_e4m3_codes(rng.standard_normal(size=(tk, hkv, d), dtype=np.float32) / np.float32(v_scale))
    sinks = rng.standard_normal(size=hq, dtype=np.float32)
    if sink_std != 1.0:
        sinks = sinks * np.float32(sink_std)
    return DecodeFp8Inputs(q, k, v, float(k_scale), float(v_scale), sinks.astype(np.float32), _cu(lengths), scale,
                           lengths)


@dataclass
class PagedDecodeFp8Inputs:
    q: np.ndarray            # uint16 bf16 bits [B, Hq, D]
    k_pages: np.ndarray      # uint8 E4M3 codes [P, page_size, Hkv, D]
    v_pages: np.ndarray
    k_scale: float
    v_scale: float
    block_table: np.ndarray  # int32 [B, max_pages] (-1 past a sequence's pages)
    seq_lens: np.ndarray     # int32 [B]
    sinks: np.ndarray        # float32 [Hq]
    page_size: int
    scale: float
    lengths: list = field(default_factory=list)


def make_paged_decode_fp8(lengths, page_size: int, hq: int, hkv: int, d: int = 64, seed: int = 0,
                          scale: float = 0.125, spare_pages: int = 3, fill_code: int = 0x7F,
                          rng: Optional[np.random.Generator] = None):
    """The draws of make_decode_fp8 (q -> k -> v -> sinks) with the cache
    scattered into pages as make_paged_decode does (permutation drawn after
    the sinks); unowned slots hold ``fill_code`` (an E4M3 NaN by default)."""
    rng = rng if rng is not None else np.random.default_rng(seed)
    dec = make_decode_fp8(lengths, hq, hkv, d, rng=rng, scale=scale)
    kp, vp, bt = _scatter_pages(dec.k, dec.v, dec.cu_seqlens_k, dec.lengths, page_size, rng, spare_pages, fill_code)
    return PagedDecodeFp8Inputs(dec.q, kp, vp, dec.k_scale, dec.v_scale, bt, np.asarray(dec.lengths, dtype=np.int32),
                                dec.sinks, page_size, scale, list(dec.lengths))


@dataclass
class AppendFp8Inputs:
    q: np.ndarray             # uint16 bf16 bits [Tq, Hq, D]
    k: np.ndarray             # uint8 E4M3 codes [Tk, Hkv, D]
    v: np.ndarray
    k_scale: float
    v_scale: float
    sinks: np.ndarray         # float32 [Hq]
    cu_seqlens_q: np.ndarray  # int32 [B+1]
    cu_seqlens_k: np.ndarray  # int32 [B+1]
    scale: float
    q_lens: list = field(default_factory=list)
    k_lens: list = field(default_factory=list)


def make_append_fp8(q_lens, k_lens, hq: int, hkv: int, d: int = 64, seed: int = 0, scale: float = 0.125,
                    k_scale: float = 1.0 / 16, v_scale: float = 1.0 / 16,
                    rng: Optional[np.random.Generator] = None) -> AppendFp8Inputs:
    """Queries appended to an E4M3 cache: the layout of make_append with the
    cache of make_decode_fp8 (N(0,1) / scale rounded to E4M3).  Draw order
    q -> k -> v -> sinks."""
    rng = rng if rng is not None else np.random.default_rng(seed)
    q_lens = [int(x) for x in q_lens]
    k_lens = [int(x) for x in k_lens]
    assert len(q_lens) == len(k_lens) and all(0 <= a <= b for a, b in zip(q_lens, k_lens))
    tk = sum(k_lens)
    q = _normal_bf16(rng, (sum(q_lens), hq, d))
    k = to_e4m3_codes(rng.standard_normal(size=(tk, hkv, d), dtype=np.float32) / np.float32(k_scale))
    v = to_e4m3_codes(rng.standard_normal(size=(tk, hkv, d), dtype=np.float32) / np.float32(v_scale))
    sinks = rng.standard_normal(size=hq, dtype=np.float32)
    return AppendFp8Inputs(q, k, v, float(k_scale), float(v_scale), sinks.astype(np.float32), _cu(q_lens),
                           _cu(k_lens), scale, q_lens, k_lens)


@dataclass
class PagedAppendFp8Inputs:
    q: np.ndarray             # uint16 bf16 bits [Tq, Hq, D]
    k_pages: np.ndarray       # uint8 E4M3 codes [P, page_size, Hkv, D]
    v_pages: np.ndarray
    k_scale: float
    v_scale: float
    block_table: np.ndarray   # int32 [B, max_pages] (-1 past a sequence's pages)
    seq_lens: np.ndarray      # int32 [B] (key lengths)
    cu_seqlens_q: np.ndarray  # int32 [B+1]
    sinks: np.ndarray         # float32 [Hq]
    page_size: int
    scale: float
    q_lens: list = field(default_factory=list)
    k_lens: list = field(default_factory=list)


def make_paged_append_fp8(q_lens, k_lens, page_size: int, hq: int, hkv: int, d: int = 64, seed: int = 0,
                          scale: float = 0.125, spare_pages: int = 3, fill_code: int = 0x7F,
                          rng: Optional[np.random.Generator] = None) -> PagedAppendFp8Inputs:
    """The draws of make_append_fp8 with the cache scattered into pages as
    make_paged_decode does (permutation drawn after the sinks; unowned slots
    hold ``fill_code``, an E4M3 NaN by default)."""
    rng = rng if rng is not None else np.random.default_rng(seed)
    a = make_append_fp8(q_lens, k_lens, hq, hkv, d, rng=rng, scale=scale)
    kp, vp, bt = _scatter_pages(a.k, a.v, a.cu_seqlens_k, a.k_lens, page_size, rng, spare_pages, fill_code)
    return PagedAppendFp8Inputs(a.q, kp, vp, a.k_scale, a.v_scale, bt, np.asarray(a.k_lens, dtype=np.int32),
                                a.cu_seqlens_q, a.sinks, page_size, scale, list(a.q_lens), list(a.k_lens))


def ragged_lengths(rng: np.random.Generator, n: int = 32, lo: int = 128, hi: int = 32768):
    """Log-uniform lengths round(exp(U[ln lo, ln hi]))."""
    u = rng.uniform(math.log(lo), math.log(hi), size=n)
    return [int(x) for x in np.clip(np.rint(np.exp(u)), lo, hi).astype(np.int64)]


# ---------------------------------------------------------------------------
# The five named workloads
# ---------------------------------------------------------------------------

def tiny_prefill(seed: int = 0) -> PrefillInputs:
    """1 sequence of 256 tokens, 4 query heads / 1 KV head, causal."""
    return make_prefill([256], hq=4, hkv=1, seed=seed)


def gptoss_prefill(seed: int = 0, length: int = 8192) -> PrefillInputs:
    """Batch 1, 8192 tokens, 64/8 heads (run causal and with a 128 window)."""
    return make_prefill([length], hq=64, hkv=8, seed=seed)


def gptoss_decode(seed: int = 0, batch: int = 64, ctx: int = 8192) -> DecodeInputs:
    """64 sequences with 8192 cached tokens each, 64/8 heads, full attention."""
    return make_decode([ctx] * batch, hq=64, hkv=8, seed=seed)


def long_decode(seed: int = 0, batch: int = 16, ctx: int = 32768) -> DecodeInputs:
    """16 sequences with 32768 cached tokens, sinks ~ N(0, 2) (std sqrt 2)."""
    return make_decode([ctx] * batch, hq=64, hkv=8, seed=seed, sink_std=math.sqrt(2.0))


def ragged_prefill(seed: int = 0, n: int = 32) -> PrefillInputs:
    """32 sequences, lengths log-uniform in [128, 32768], 4 heads without sink."""
    rng = np.random.default_rng(seed)
    lengths = ragged_lengths(rng, n)
    return make_prefill(lengths, hq=64, hkv=8, rng=rng, no_sink_heads=NO_SINK_HEADS)
