"""Pins for the FP8 (E4M3) KV-cache decode oracle (CPU).

The format is the OCP 8-bit floating-point E4M3 (1 sign, 4 exponent, 3
mantissa bits, bias 7, no infinities, S.1111.111 = NaN); the cache holds
scale * e4m3(code) with one fp32 scale per tensor (vLLM, "GPT-OSS performance
optimizations on NVIDIA Blackwell", FlashInfer integration: the KV cache in
FP8; the format and the scale convention are readings, not printed there).
"""

import math

import numpy as np
import pytest
import torch

from attention_gqa_flash_amd import inputs
from oracle import decode_fp8_ref, decode_ref, e4m3_to_float64

ALL = np.arange(256, dtype=np.uint8)


def test_all_codes_match_torch_float8_e4m3fn():
    """Library routine: torch's own E4M3 (fn) decoding, code by code."""
    lib = torch.from_numpy(ALL.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = e4m3_to_float64(ALL)
    assert np.array_equal(np.isnan(lib), np.isnan(ours))
    ok = ~np.isnan(lib)
    assert np.array_equal(lib[ok], ours[ok])
    assert np.array_equal(np.signbit(lib[ok]), np.signbit(ours[ok]))


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0x38, 1.0),
    (0x3F, 1.875), (0x40, 2.0), (0x7E, 448.0), (0xB8, -1.0), (0xFE, -448.0)])
def test_values_from_the_format_definition(code, value):
    assert e4m3_to_float64(np.uint8(code)) == value


def test_nan_codes_negative_zero_and_order():
    v = e4m3_to_float64(ALL)
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and np.isnan(v).sum() == 2
    assert v[0x80] == 0.0 and math.copysign(1.0, v[0x80]) < 0
    assert np.all(np.diff(v[0x00:0x7F]) > 0)          # positive codes increase
    assert np.all(np.diff(v[0x80:0xFF]) < 0)          # negative codes decrease
    assert np.array_equal(v[0x80:0xFF], -v[0x00:0x7F])


def test_scales_apply_to_k_and_v_respectively():
    """K = k_scale * e4m3(k), V = v_scale * e4m3(v): against decode_ref on
    caches dequantised through torch's decoding, with k_scale != v_scale."""
    d = inputs.make_decode_fp8([1, 9, 40], hq=8, hkv=2, seed=3, k_scale=1.0 / 16, v_scale=1.0 / 8)
    qf = inputs.bf16_bits_to_f32(d.q)
    dec = lambda c: torch.from_numpy(c.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for window in (0, 5):
        ro, rl = decode_ref(qf, d.k_scale * dec(d.k), d.v_scale * dec(d.v), d.cu_seqlens_k, d.sinks, window, d.scale)
        o, lse = decode_fp8_ref(qf, d.k, d.v, d.k_scale, d.v_scale, d.cu_seqlens_k, d.sinks, window, d.scale)
        assert np.allclose(o, ro, rtol=0, atol=1e-14) and np.allclose(lse, rl, rtol=0, atol=1e-14)


def test_v_scale_scales_o_only_and_k_scale_acts_as_a_logit_scale():
    d = inputs.make_decode_fp8([17, 30], hq=4, hkv=1, seed=4)
    qf = inputs.bf16_bits_to_f32(d.q)
    o1, l1 = decode_fp8_ref(qf, d.k, d.v, 0.0625, 0.0625, d.cu_seqlens_k, d.sinks, 0, d.scale)
    o2, l2 = decode_fp8_ref(qf, d.k, d.v, 0.0625, 0.25, d.cu_seqlens_k, d.sinks, 0, d.scale)
    assert np.allclose(o2, 4 * o1, rtol=1e-15, atol=0) and np.array_equal(l1, l2)
    # doubling k_scale equals doubling the softmax scale
    o3, l3 = decode_fp8_ref(qf, d.k, d.v, 0.125, 0.0625, d.cu_seqlens_k, d.sinks, 0, d.scale)
    o4, l4 = decode_fp8_ref(qf, d.k, d.v, 0.0625, 0.0625, d.cu_seqlens_k, d.sinks, 0, 2 * d.scale)
    assert np.allclose(o3, o4, rtol=0, atol=1e-15) and np.allclose(l3, l4, rtol=0, atol=1e-13)


def test_generated_cache_is_close_to_its_normal_draw():
    """The generator's codes decode (times the scale) to N(0,1)-sized values:
    E4M3 keeps 3 mantissa bits, so each is within 1/16 relative (or the
    smallest step) of a standard normal draw."""
    d = inputs.make_decode_fp8([4096], hq=8, hkv=2, seed=5)
    k = d.k_scale * e4m3_to_float64(d.k)
    assert np.isfinite(k).all()
    assert 0.95 < k.std() < 1.05 and abs(k.mean()) < 0.02


# --- several query tokens per sequence (draft tokens) against an E4M3 cache ---

from oracle import decode_fp8_multi_ref  # noqa: E402


def _e4m3_by_hand(code: int) -> float:
    """E4M3 from the format definition with the math module (independent of
    the oracle's vectorised decoding): bias 7, subnormals 2^-6 * m / 8."""
    s = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 15, code & 7
    return s * (math.ldexp(m / 8.0, -6) if e == 0 else math.ldexp(1.0 + m / 8.0, e - 7))


def test_multi_with_one_query_is_the_single_token_decode():
    a = inputs.make_append_fp8([1, 1, 1], [1, 37, 300], hq=8, hkv=2, seed=6, k_scale=0.0625, v_scale=0.125)
    d_cu = a.cu_seqlens_k
    qf = inputs.bf16_bits_to_f32(a.q)
    for window in (0, 1, 16):
        o1, l1 = decode_fp8_multi_ref(qf, a.k, a.v, a.k_scale, a.v_scale, a.cu_seqlens_q, d_cu, a.sinks, window, a.scale)
        o2, l2 = decode_fp8_ref(qf, a.k, a.v, a.k_scale, a.v_scale, d_cu, a.sinks, window, a.scale)
        assert np.allclose(o1, o2, rtol=0, atol=1e-14) and np.allclose(l1, l2, rtol=0, atol=1e-13)


@pytest.mark.parametrize("window", [0, 1, 2, 5, 40])
def test_multi_brute_force(window):
    """Python loops over the codes decoded by hand, the bottom-right causal /
    window mask written out, math.fsum for the sums."""
    q_lens, k_lens = [3, 1, 4], [5, 9, 12]
    hq, hkv, d = 4, 2, 8
    a = inputs.make_append_fp8(q_lens, k_lens, hq=hq, hkv=hkv, d=d, seed=7, k_scale=0.125, v_scale=0.25)
    qf = inputs.bf16_bits_to_f32(a.q).astype(np.float64)
    o, lse = decode_fp8_multi_ref(qf, a.k, a.v, a.k_scale, a.v_scale, a.cu_seqlens_q, a.cu_seqlens_k, a.sinks, window,
                                  a.scale)
    g = hq // hkv
    for b in range(len(q_lens)):
        for r in range(q_lens[b]):
            row = a.cu_seqlens_q[b] + r
            pos = k_lens[b] - q_lens[b] + r
            keys = [j for j in range(k_lens[b]) if j <= pos and (window <= 0 or j > pos - window)]
            for h in range(hq):
                kh = h // g
                logits = []
                for j in keys:
                    kr = a.cu_seqlens_k[b] + j
                    dot = math.fsum(qf[row, h, c] * a.k_scale * _e4m3_by_hand(int(a.k[kr, kh, c])) for c in range(d))
                    logits.append(a.scale * dot)
                z = float(a.sinks[h])
                big = max(logits + [z])
                w = [math.exp(x - big) for x in logits]
                den = math.fsum(w) + math.exp(z - big)
                for c in range(d):
                    num = math.fsum(wj * a.v_scale * _e4m3_by_hand(int(a.v[a.cu_seqlens_k[b] + j, kh, c]))
                                    for wj, j in zip(w, keys))
                    assert abs(o[row, h, c] - num / den) < 1e-12
                assert abs(lse[row, h] - (big + math.log(den))) < 1e-12


def test_multi_scales_act_on_logits_and_outputs():
    a = inputs.make_append_fp8([2, 3], [20, 33], hq=8, hkv=2, seed=8)
    qf = inputs.bf16_bits_to_f32(a.q)
    args = (a.cu_seqlens_q, a.cu_seqlens_k, a.sinks, 7)
    o1, l1 = decode_fp8_multi_ref(qf, a.k, a.v, 0.0625, 0.0625, *args, a.scale)
    o2, l2 = decode_fp8_multi_ref(qf, a.k, a.v, 0.0625, 0.5, *args, a.scale)
    assert np.allclose(o2, 8 * o1, rtol=1e-15, atol=0) and np.array_equal(l1, l2)
    o3, l3 = decode_fp8_multi_ref(qf, a.k, a.v, 0.125, 0.0625, *args, a.scale)
    o4, l4 = decode_fp8_multi_ref(qf, a.k, a.v, 0.0625, 0.0625, *args, 2 * a.scale)
    assert np.allclose(o3, o4, rtol=0, atol=1e-15) and np.allclose(l3, l4, rtol=0, atol=1e-13)
