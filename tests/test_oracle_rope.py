"""Pins for the rotary-embedding / YaRN / fused QKV-append oracle (CPU).

Checked against things other than the functions themselves: the rotation in
complex-number form, the relative-position property of rotary embeddings,
norm preservation, position 0, YaRN's limiting cases (frequencies that turn
more than beta_fast times over the original context are kept, fewer than
beta_slow times divided by the factor; factor 1 is plain RoPE), the ramp's
interior on constructed parameters that put its ends on chosen indices
(values by hand, with and without truncated ends), transformers' YaRN
initialiser for the GPT-OSS configuration, a brute-force evaluation of the
rotation with the math module, and the scatter into the cache.

Sources: the RoFormer rotary embedding and the YaRN method (Peng et al.,
section 3), named by the pages as RoPE (NVIDIA gpt-oss announcement, model
description) and YaRN position encoding (Perplexity, "GPT-OSS on day 0",
Hopper section); the fusion with Q and the cache append (vLLM, "GPT-OSS
performance optimizations on NVIDIA Blackwell", minimum latency).
"""

import cmath
import math

import numpy as np
import pytest

from oracle import rope_qkv_append_ref, rope_ref, yarn_inv_freq_ref


def test_rotation_equals_complex_multiplication():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 3, 8))
    pos = np.array([0, 1, 7, 1000, 131071])
    f = rng.uniform(0.0, 1.0, 4)
    out = rope_ref(x, pos, f, 1.3)
    for t in range(5):
        for h in range(3):
            for i in range(4):
                z = complex(x[t, h, i], x[t, h, i + 4]) * cmath.exp(1j * pos[t] * f[i]) * 1.3
                assert abs(out[t, h, i] - z.real) < 1e-9 and abs(out[t, h, i + 4] - z.imag) < 1e-9


def test_dot_product_depends_on_relative_position_only():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 1, 64))
    k = rng.standard_normal((1, 1, 64))
    f, _ = yarn_inv_freq_ref(64, 150000.0, 32.0, 4096, 32.0, 1.0)
    dots = []
    for p in (0, 17, 5000):
        qr = rope_ref(q, [p + 9], f)
        kr = rope_ref(k, [p], f)
        dots.append(float((qr * kr).sum()))
    assert max(dots) - min(dots) < 1e-9


def test_norm_and_position_zero():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 2, 64))
    f, m = yarn_inv_freq_ref(64, 10000.0, 8.0, 2048, 32.0, 1.0)
    out = rope_ref(x, [0, 3, 99, 123456], f, m)
    assert np.allclose(np.linalg.norm(out, axis=-1), m * np.linalg.norm(x, axis=-1), rtol=1e-12)
    assert np.allclose(out[0], m * x[0], rtol=0, atol=1e-15)


def test_yarn_limits_and_temperature():
    d, theta, s, L = 64, 150000.0, 32.0, 4096
    base, m1 = yarn_inv_freq_ref(d, theta)
    assert m1 == 1.0
    assert np.allclose(base, [theta ** (-2 * i / d) for i in range(d // 2)], rtol=1e-15)
    f, m = yarn_inv_freq_ref(d, theta, s, L, 32.0, 1.0)
    assert m == pytest.approx(0.1 * math.log(32.0) + 1.0, rel=1e-15)
    # a pair whose frequency turns more than beta_fast = 32 times over the
    # original 4096 positions (wavelength below 128 positions) is kept, one
    # turning less than once (wavelength above 4096) is divided by s
    wavelength = 2 * math.pi / base
    fast, slow = wavelength < L / 32.0, wavelength > L
    assert fast.any() and slow.any() and (~fast & ~slow).any()
    assert np.array_equal(f[fast], base[fast])               # high frequencies kept
    assert np.allclose(f[slow], base[slow] / s, rtol=1e-15)  # low frequencies interpolated
    mid = ~fast & ~slow
    assert np.all(f[mid] < base[mid]) and np.all(f[mid] > base[mid] / s)
    f1, m1 = yarn_inv_freq_ref(d, theta, 1.0, L, 32.0, 1.0)
    assert np.array_equal(f1, base) and m1 == 1.0


# theta = e^32 at head_dim 64 gives f_i = e^-i, and the pair index whose
# frequency turns r times over L positions is ln(L / (2 pi r)).  Turn counts
# L / (2 pi e^a) therefore put a ramp end exactly on index a.
E32 = math.exp(32.0)


def _beta_at(index, L=4096):
    return L / (2 * math.pi * math.exp(index))


def test_yarn_ramp_interior_on_constructed_indices():
    """Ramp ends on indices 2 (beta_fast) and 6 (beta_slow), factor 8: the
    ramp is linear in the index, so index 3 is a quarter of the way to the
    interpolated frequency, 4 half, 5 three quarters (values by hand)."""
    f, m = yarn_inv_freq_ref(64, E32, 8.0, 4096, _beta_at(2.0), _beta_at(6.0))
    hand = {0: 1.0, 1: math.exp(-1), 2: math.exp(-2),
            3: math.exp(-3) * (3 / 4 + 1 / 32), 4: math.exp(-4) * (1 / 2 + 1 / 16), 5: math.exp(-5) * (1 / 4 + 3 / 32),
            6: math.exp(-6) / 8, 20: math.exp(-20) / 8, 31: math.exp(-31) / 8}
    for i, want in hand.items():
        assert f[i] == pytest.approx(want, rel=1e-12), i
    assert m == pytest.approx(0.1 * math.log(8.0) + 1.0, rel=1e-15)


def test_yarn_truncated_ramp_on_constructed_indices():
    """Ramp ends on 2.5 and 5.5: unrounded (the GPT-OSS setting) index 3 sits
    a sixth of the way, 4 half, 5 five sixths; with truncation the ends
    become 2 and 6 (floor, ceil) and the quarters of the previous case."""
    bf, bs = _beta_at(2.5), _beta_at(5.5)
    f, _ = yarn_inv_freq_ref(64, E32, 8.0, 4096, bf, bs)
    hand = {2: math.exp(-2), 3: math.exp(-3) * (5 / 6 + 1 / 48), 4: math.exp(-4) * (1 / 2 + 1 / 16),
            5: math.exp(-5) * (1 / 6 + 5 / 48), 6: math.exp(-6) / 8}
    for i, want in hand.items():
        assert f[i] == pytest.approx(want, rel=1e-12), i
    ft, _ = yarn_inv_freq_ref(64, E32, 8.0, 4096, bf, bs, truncate=True)
    hand_t = {2: math.exp(-2), 3: math.exp(-3) * (3 / 4 + 1 / 32), 4: math.exp(-4) * (1 / 2 + 1 / 16),
              5: math.exp(-5) * (1 / 4 + 3 / 32), 6: math.exp(-6) / 8}
    for i, want in hand_t.items():
        assert ft[i] == pytest.approx(want, rel=1e-12), i


@pytest.mark.parametrize("truncate", [False, True])
@pytest.mark.parametrize("params", [dict(), dict(rope_theta=10000.0, factor=8.0, original_max_position_embeddings=2048),
                                    dict(beta_fast=16.0, beta_slow=2.0, factor=4.0)], ids=["gpt_oss", "p1", "p2"])
def test_yarn_matches_transformers_library_routine(truncate, params):
    """transformers' YaRN initialiser (the routine its GPT-OSS model uses;
    float32) on the GPT-OSS configuration (theta 150000, factor 32, 4096
    original positions, beta 32 / 1, no truncation) and variations."""
    transformers = pytest.importorskip("transformers")
    from transformers.modeling_rope_utils import ROPE_INIT_FUNCTIONS
    cfg = transformers.GptOssConfig()
    rp = dict(cfg.rope_parameters)
    rp.update(params)
    rp["truncate"] = truncate
    cfg.rope_parameters = rp
    lib_f, lib_m = ROPE_INIT_FUNCTIONS["yarn"](cfg, "cpu")
    f, m = yarn_inv_freq_ref(cfg.head_dim, rp["rope_theta"], rp["factor"], rp["original_max_position_embeddings"],
                             rp["beta_fast"], rp["beta_slow"], truncate)
    assert np.allclose(f, lib_f.double().numpy(), rtol=1e-6, atol=0)
    assert m == pytest.approx(lib_m, rel=1e-12)


def test_brute_force_rotation():
    d, theta, s, L, bf, bs = 16, 5000.0, 4.0, 64, 8.0, 2.0
    f, m = yarn_inv_freq_ref(d, theta, s, L, bf, bs)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 1, d))
    out = rope_ref(x, [5, 77], f, m)
    for t, p in enumerate((5, 77)):
        for i in range(d // 2):
            a = p * f[i]
            assert out[t, 0, i] == pytest.approx(m * (x[t, 0, i] * math.cos(a) - x[t, 0, i + d // 2] * math.sin(a)),
                                                 abs=1e-12)
            assert out[t, 0, i + d // 2] == pytest.approx(
                m * (x[t, 0, i + d // 2] * math.cos(a) + x[t, 0, i] * math.sin(a)), abs=1e-12)


def test_fused_step_scatters_rows():
    rng = np.random.default_rng(4)
    hq, hkv, d, t = 4, 2, 8, 5
    qkv = rng.standard_normal((t, hq + 2 * hkv, d))
    pos = np.array([3, 4, 5, 6, 7])
    f, m = yarn_inv_freq_ref(d, 100.0, 2.0, 16, 4.0, 1.0)
    kc = rng.standard_normal((10, hkv, d))
    vc = rng.standard_normal((10, hkv, d))
    slots = np.array([9, -1, 0, 4, 2])
    q_out, kc2, vc2 = rope_qkv_append_ref(qkv, pos, hq, hkv, f, m, slots, kc, vc)
    assert np.array_equal(q_out, rope_ref(qkv[:, :hq], pos, f, m))
    for tt, sl in enumerate(slots):
        if sl >= 0:
            assert np.array_equal(kc2[sl], rope_ref(qkv[tt:tt + 1, hq:hq + hkv], pos[tt:tt + 1], f, m)[0])
            assert np.array_equal(vc2[sl], qkv[tt, hq + hkv:])
    untouched = [r for r in range(10) if r not in slots]
    assert np.array_equal(kc2[untouched], kc[untouched]) and np.array_equal(vc2[untouched], vc[untouched])
