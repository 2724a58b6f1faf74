"""Rotary position embedding with YaRN scaling, fused with the Q output and
the KV-cache append, for the float64 oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed: the attention layers rotate query and key heads by their
token's position (NVIDIA's gpt-oss announcement, model description: RoPE;
Perplexity, "GPT-OSS on day 0", Hopper section: YaRN position encoding as in
DeepSeek-V3), and the step before attention applies the rotation to Q and
writes the rotated K and the V of the new tokens into the cache in one pass
(vLLM, "GPT-OSS performance optimizations on NVIDIA Blackwell", minimum
latency: the RoPE + Q + cache fusion).  The pages print no formula and no
parameter.  Readings (all listed in the design notes):

* rotation: the RoFormer rotary embedding; dimension i of the first half of a
  head pairs with dimension i + D/2 (the half-split pairing), frequency
  f_i for i < D/2:  (x_i, x_{i+D/2}) -> (x_i cos a - x_{i+D/2} sin a,
  x_{i+D/2} cos a + x_i sin a), a = position * f_i;
* frequencies: f_i = theta^(-2i/D), rescaled by YaRN's NTK-by-parts rule
  (Peng et al., "YaRN: Efficient Context Window Extension of Large Language
  Models", section 3) as its own code and the GPT-OSS / DeepSeek-V3 models
  apply it: frequency i turns r_i = L f_i / (2 pi) times over the original
  context L; the pair index at which r equals beta is
  c(beta) = (D/2) ln(L / (2 pi beta)) / ln(theta) (solving r_i = beta for
  i); with low = c(beta_fast) and high = c(beta_slow) (floored and ceiled
  when `truncate` is set, as DeepSeek-V3 does; GPT-OSS leaves them
  unrounded), clamped to [0, D - 1], the ramp
  gamma_i = clamp((i - low) / (high - low), 0, 1) is linear in the index,
  i.e. in log r, and the frequency becomes f_i (1 - gamma_i) + gamma_i f_i / s
  for a scale factor s (kept above beta_fast turns, divided by s below
  beta_slow); a factor s <= 1 leaves plain RoPE;
* temperature: YaRN's sqrt(1/t) = 0.1 ln s + 1 multiplies the rotated q and k
  (so the logits scale by its square); 1 for s <= 1;
* fusion: qkv [T, Hq + 2 Hkv, D] holds the q heads, then the k heads, then
  the v heads of each token; q is rotated into q_out [T, Hq, D]; k (rotated)
  and v (unchanged) go to cache row slot_mapping[t] (a row of a contiguous
  cache, or page * page_size + slot of a paged one); slot -1 writes nothing.

Parity status: pinned by CPU tests (tests/test_oracle_rope.py) against the
complex-number form of the rotation, relative-position invariance, norm
preservation, position 0, YaRN's limiting cases (more than beta_fast turns
unchanged, fewer than beta_slow divided by s, factor 1 = plain RoPE),
constructed parameters whose ramp bounds fall on chosen indices (values of
the ramp's interior worked out by hand), the library routine transformers
uses for the GPT-OSS configuration, brute force with the math module, and the
scatter into the cache.
"""

from __future__ import annotations

import math

import numpy as np


def yarn_inv_freq_ref(head_dim: int, theta: float, factor: float = 1.0, original_max_position: float = 4096,
                      beta_fast: float = 32.0, beta_slow: float = 1.0, truncate: bool = False):
    """Frequencies f_i (i < head_dim / 2, float64) after YaRN's NTK-by-parts
    rescaling, and the temperature factor 0.1 ln s + 1 (1 when s <= 1).
    beta_fast / beta_slow are the turn counts over the original context at
    which the ramp over the pair index starts and ends."""
    half = head_dim // 2
    i = np.arange(half, dtype=np.float64)
    base = theta ** (-2.0 * i / head_dim)
    if factor <= 1.0:
        return base, 1.0

    def index_of(turns):
        # the (fractional) pair index whose frequency turns `turns` times
        # over the original context
        return (head_dim / 2.0) * math.log(original_max_position / (2.0 * math.pi * turns)) / math.log(theta)

    low, high = index_of(beta_fast), index_of(beta_slow)
    if truncate:
        low, high = math.floor(low), math.ceil(high)
    low, high = max(low, 0.0), min(high, head_dim - 1.0)
    if high == low:
        high += 0.001   # a zero-width ramp becomes a step
    gamma = np.clip((i - low) / (high - low), 0.0, 1.0)
    freq = base * (1.0 - gamma) + gamma * base / factor
    return freq, 0.1 * math.log(factor) + 1.0


def rope_ref(x, positions, inv_freq, attention_factor: float = 1.0) -> np.ndarray:
    """Rotate x [T, H, D] (float64) by positions [T] with frequencies
    inv_freq [D/2], half-split pairing, times attention_factor."""
    x = np.asarray(x, dtype=np.float64)
    half = x.shape[-1] // 2
    a = np.asarray(positions, dtype=np.float64)[:, None] * np.asarray(inv_freq, dtype=np.float64)[None, :]
    c = np.cos(a)[:, None, :]
    s = np.sin(a)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    out = np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)
    return out * attention_factor


def rope_qkv_append_ref(qkv, positions, num_q_heads: int, num_kv_heads: int, inv_freq, attention_factor: float,
                        slot_mapping, k_cache, v_cache):
    """The fused step: returns q_out [T, Hq, D] (rotated) and copies of
    k_cache / v_cache [rows, Hkv, D] with row slot_mapping[t] set to the
    rotated k / the v of token t (slot -1: nothing written)."""
    qkv = np.asarray(qkv, dtype=np.float64)
    hq, hkv = num_q_heads, num_kv_heads
    q = qkv[:, :hq]
    k = qkv[:, hq:hq + hkv]
    v = qkv[:, hq + hkv:hq + 2 * hkv]
    q_out = rope_ref(q, positions, inv_freq, attention_factor)
    k_rot = rope_ref(k, positions, inv_freq, attention_factor)
    kc = np.array(k_cache, dtype=np.float64, copy=True)
    vc = np.array(v_cache, dtype=np.float64, copy=True)
    for t, slot in enumerate(np.asarray(slot_mapping)):
        if slot >= 0:
            kc[slot] = k_rot[t]
            vc[slot] = v[t]
    return q_out, kc, vc
