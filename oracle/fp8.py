"""FP8 (E4M3) KV-cache decode for the float64 oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: vLLM, "GPT-OSS performance optimizations on NVIDIA Blackwell",
section "FlashInfer integration": the KV cache is stored in FP8.  The page
names neither the 8-bit format nor how values are scaled; the readings taken
here are the OCP 8-bit floating-point E4M3 format (the FP8 format of KV
caches; 1 sign, 4 exponent and 3 mantissa bits, bias 7, no infinities, the
two codes with all exponent and mantissa bits set are NaN) and one fp32 scale
per tensor, so a cached element is scale * e4m3(code).  Attention over the
dequantised cache is then the plain definition of ``decode_ref`` (one query
per sequence) or ``prefill_append_ref`` (several query tokens per sequence,
the newest ones: draft tokens of a speculative or multi-token-prediction
decoder; Perplexity, "GPT-OSS on day 0", in-house inference engine).
"""

from __future__ import annotations

import numpy as np

from .append import prefill_append_ref
from .sink_attention import decode_ref


def e4m3_to_float64(codes) -> np.ndarray:
    """Decode E4M3 codes (uint8, any shape) to float64, from the format's
    definition: exponent field e and mantissa field m give
    (-1)^s * 2^(e-7) * (1 + m/8) for e > 0 and (-1)^s * 2^-6 * (m/8) for
    e = 0; e = 15 with m = 7 is NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    normal = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    subnormal = np.ldexp(m / 8.0, -6)
    val = sign * np.where(e == 0, subnormal, normal)
    return np.where((e == 15) & ((c & 7) == 7), np.nan, val)


def decode_fp8_ref(q, k_codes, v_codes, k_scale: float, v_scale: float, cu_seqlens_k, sinks,
                   window: int, scale: float):
    """Single-token decode against an E4M3 KV cache with per-tensor scales:
    K = k_scale * e4m3(k_codes), V = v_scale * e4m3(v_codes), then
    ``decode_ref`` (float64)."""
    k = float(k_scale) * e4m3_to_float64(k_codes)
    v = float(v_scale) * e4m3_to_float64(v_codes)
    return decode_ref(q, k, v, cu_seqlens_k, sinks, window, scale)


def decode_fp8_multi_ref(q, k_codes, v_codes, k_scale: float, v_scale: float, cu_seqlens_q, cu_seqlens_k, sinks,
                         window: int, scale: float, rows=None):
    """Several query tokens per sequence against an E4M3 KV cache with
    per-tensor scales: K = k_scale * e4m3(k_codes), V = v_scale *
    e4m3(v_codes), then ``prefill_append_ref`` (sequence b's queries are its
    newest cu_seqlens_q[b+1] - cu_seqlens_q[b] tokens; float64)."""
    k = float(k_scale) * e4m3_to_float64(k_codes)
    v = float(v_scale) * e4m3_to_float64(v_codes)
    return prefill_append_ref(q, k, v, sinks, cu_seqlens_q, cu_seqlens_k, window, scale, rows=rows)
