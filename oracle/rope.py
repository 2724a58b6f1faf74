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
  Models", section 3): with r_i = L / (2 pi / f_i) the number of turns of
  frequency i over the original context L and the ramp
  gamma(r) = clamp((r - alpha) / (beta - alpha), 0, 1), the frequency
  becomes (1 - gamma_i) f_i / s + gamma_i f_i for a scale factor s; a factor
  s <= 1 leaves plain RoPE;
* temperature: YaRN's sqrt(1/t) = 0.1 ln s + 1 multiplies the rotated q and k
  (so the logits scale by its square); 1 for s <= 1;
* fusion: qkv [T, Hq + 2 Hkv, D] holds the q heads, then the k heads, then
  the v heads of each token; q is rotated into q_out [T, Hq, D]; k (rotated)
  and v (unchanged) go to cache row slot_mapping[t] (a row of a contiguous
  cache, or page * page_size + slot of a paged one); slot -1 writes nothing.

Parity status: pinned by CPU tests (tests/test_oracle_rope.py) against the
complex-number form of the rotation, relative-position invariance, norm
preservation, position 0, YaRN's limiting cases (r > beta unchanged, r < alpha
divided by s, factor 1 = plain RoPE), brute force with the math module, and
the scatter into the cache.
"""

from __future__ import annotations

import math

import numpy as np


def yarn_inv_freq_ref(head_dim: int, theta: float, factor: float = 1.0, original_max_position: int = 4096,
                      beta_fast: float = 32.0, beta_slow: float = 1.0):
    """Frequencies f_i (i < head_dim / 2, float64) after YaRN's NTK-by-parts
    rescaling, and the temperature factor 0.1 ln s + 1 (1 when s <= 1).
    beta_slow and beta_fast are YaRN's alpha and beta (turns over the
    original context)."""
    half = head_dim // 2
    i = np.arange(half, dtype=np.float64)
    base = theta ** (-2.0 * i / head_dim)
    if factor <= 1.0:
        return base, 1.0
    turns = original_max_position * base / (2.0 * math.pi)    # r_i = L / lambda_i
    gamma = np.clip((turns - beta_slow) / (beta_fast - beta_slow), 0.0, 1.0)
    freq = (1.0 - gamma) * base / factor + gamma * base
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
