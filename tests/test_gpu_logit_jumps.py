"""GPU parity when logits rise late and far above the running maximum.

Every path keeps its online softmax against a reference maximum that moves
only past a margin (decode: a tile maximum more than 2^8 above it; prefill: a
partial denominator past 2^32), rescaling the accumulators when it does.
Random N(0,1) inputs seldom take those branches after the first tile.  Here
keys are planted as multiples alpha of one query head's own vector, so that
head's logit at the planted position is about alpha * |q|^2 * scale: with
|q|^2 ~ 64 and scale 1/8, alpha = 1, 2, 3.5, 6 give jumps of roughly 11, 23,
40 and 69 in log2 units over logits whose running maximum is near 5.  Later
plants sit below an earlier, larger one as well, so the reference both moves
and stays.  The other heads of the group see the same keys at random angles
to their own queries.

Bar as everywhere: max |err| <= 2e-2 and mean |err| <= 2e-3 on the bf16
outputs against the float64 oracle; lse within 4e-3 with an identical -inf
pattern.
"""

import numpy as np
import pytest
import torch

from attention_gqa_flash_amd import binding, inputs
from oracle import decode_fp8_multi_ref, decode_fp8_ref, decode_ref, prefill_append_ref, prefill_varlen_ref
from tests.helpers import (assert_close_lse, assert_close_out, bf16_to_device, f32_to_device, i32_to_device,
                           to_f64)

pytestmark = pytest.mark.gpu

ALPHAS = (1.0, 2.0, 3.5, 6.0, 3.0, 1.5)  # the last two sit below the third and fourth


def _u8(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def _plant_rows(k_f32, rows, q_vec, alpha):
    """K rows `rows` (sequence positions already offset) of one KV head:
    alpha times the query vector."""
    for r in rows:
        k_f32[r] = np.float32(alpha) * q_vec


def _plants(length, n):
    """n positions spread over [length / 8, length), increasing."""
    return [int(length * (1 + 7 * i / n) / 8) for i in range(n)]


def _decode_plant(q_bits, k_bits, cu_k, lengths, group, q_row_of, encode):
    """Plant the ALPHAS ladder into every sequence of at least 64 keys, for
    one head per KV head (varying with the sequence).  q_row_of(b) gives the
    query row whose vector is planted; encode(values) returns the cache's
    storage for float32 values."""
    hkv = k_bits.shape[1]
    qf = inputs.bf16_bits_to_f32(q_bits)
    k_new = k_bits.copy()
    for b, length in enumerate(lengths):
        if length < 64:
            continue
        pos = _plants(length, len(ALPHAS))
        for g in range(hkv):
            h0 = g * group + (b + g) % group
            q_vec = qf[q_row_of(b), h0]
            for p, alpha in zip(pos, ALPHAS):
                k_new[cu_k[b] + p, g] = encode((np.float32(alpha) * q_vec).astype(np.float32))
    return k_new


@pytest.mark.parametrize("hq,hkv", [(64, 8), (16, 2), (32, 1)])
@pytest.mark.parametrize("splits", [1, 2, 4, 16])
def test_decode_logit_jumps(hq, hkv, splits):
    lengths = [64, 700, 3000, 8200]
    d = inputs.make_decode(lengths, hq=hq, hkv=hkv, seed=500 + hq + splits)
    d.k = _decode_plant(d.q, d.k, d.cu_seqlens_k, lengths, hq // hkv, lambda b: b, inputs.round_to_bf16_bits)
    qf, kf, vf = (inputs.bf16_bits_to_f32(x) for x in (d.q, d.k, d.v))
    for window in (0, 1000):
        o, lse = binding.decode_splitkv(bf16_to_device(d.q), bf16_to_device(d.k), bf16_to_device(d.v),
                                        i32_to_device(d.cu_seqlens_k), max(lengths), f32_to_device(d.sinks), window,
                                        d.scale, splits, return_lse=True)
        torch.cuda.synchronize()
        ro, rl = decode_ref(qf, kf, vf, d.cu_seqlens_k, d.sinks, window, d.scale)
        what = "decode jumps G=%d S=%d W=%d" % (hq // hkv, splits, window)
        assert_close_out(to_f64(o), ro, what)
        assert_close_lse(lse.cpu().numpy(), rl, what)


@pytest.mark.parametrize("hq,hkv", [(64, 8), (20, 5)])
@pytest.mark.parametrize("splits", [1, 4, 16])
def test_fp8_decode_logit_jumps(hq, hkv, splits):
    """The E4M3 cache: the KV-head-pair kernels (64 / 8) and the generic
    FP8 kernels (an odd number of KV heads)."""
    lengths = [64, 700, 3000, 8200]
    d = inputs.make_decode_fp8(lengths, hq=hq, hkv=hkv, seed=600 + hq + splits)
    d.k = _decode_plant(d.q, d.k, d.cu_seqlens_k, lengths, hq // hkv, lambda b: b,
                        lambda x: inputs.to_e4m3_codes(x / np.float32(d.k_scale)))
    o, lse = binding.decode_splitkv_fp8(bf16_to_device(d.q), _u8(d.k), _u8(d.v), d.k_scale, d.v_scale,
                                        i32_to_device(d.cu_seqlens_k), max(lengths), f32_to_device(d.sinks), 0,
                                        d.scale, splits, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = decode_fp8_ref(inputs.bf16_bits_to_f32(d.q), d.k, d.v, d.k_scale, d.v_scale, d.cu_seqlens_k, d.sinks,
                            0, d.scale)
    what = "fp8 decode jumps G=%d S=%d" % (hq // hkv, splits)
    assert_close_out(to_f64(o), ro, what)
    assert_close_lse(lse.cpu().numpy(), rl, what)


@pytest.mark.parametrize("n_tok", [1, 4, 8])
@pytest.mark.parametrize("splits", [1, 4])
@pytest.mark.parametrize("fp8", [False, True])
def test_multi_decode_logit_jumps(n_tok, splits, fp8):
    """Draft tokens (16-, 32- and 64-column layouts): the planted vector is the
    newest token's query; every token sees the planted keys (all before the
    first query position)."""
    k_lens = [64, 700, 3000, 8200]
    q_lens = [n_tok] * len(k_lens)
    hq, hkv = 64, 8
    seed = 700 + 10 * n_tok + splits
    a = (inputs.make_append_fp8 if fp8 else inputs.make_append)(q_lens, k_lens, hq=hq, hkv=hkv, seed=seed)
    lengths = [L - n_tok for L in k_lens]  # plants stay before the first query position
    if fp8:
        encode = lambda x: inputs.to_e4m3_codes(x / np.float32(a.k_scale))  # noqa: E731
    else:
        encode = inputs.round_to_bf16_bits
    a.k = _decode_plant(a.q, a.k, a.cu_seqlens_k, lengths, hq // hkv, lambda b: a.cu_seqlens_q[b + 1] - 1, encode)
    q = bf16_to_device(a.q)
    cq, ck = i32_to_device(a.cu_seqlens_q), i32_to_device(a.cu_seqlens_k)
    if fp8:
        o, lse = binding.decode_splitkv_multi_fp8(q, _u8(a.k), _u8(a.v), a.k_scale, a.v_scale, cq, ck, n_tok,
                                                  max(k_lens), f32_to_device(a.sinks), 0, a.scale, splits,
                                                  return_lse=True)
        ro, rl = decode_fp8_multi_ref(inputs.bf16_bits_to_f32(a.q), a.k, a.v, a.k_scale, a.v_scale, a.cu_seqlens_q,
                                      a.cu_seqlens_k, a.sinks, 0, a.scale)
    else:
        o, lse = binding.decode_splitkv_multi(q, bf16_to_device(a.k), bf16_to_device(a.v), cq, ck, n_tok, max(k_lens),
                                              f32_to_device(a.sinks), 0, a.scale, splits, return_lse=True)
        qf, kf, vf = (inputs.bf16_bits_to_f32(x) for x in (a.q, a.k, a.v))
        ro, rl = prefill_append_ref(qf, kf, vf, a.sinks, a.cu_seqlens_q, a.cu_seqlens_k, 0, a.scale)
    torch.cuda.synchronize()
    what = "multi jumps n=%d S=%d fp8=%s" % (n_tok, splits, fp8)
    assert_close_out(to_f64(o), ro, what)
    assert_close_lse(lse.cpu().numpy(), rl, what)


@pytest.mark.parametrize("window", [0, 128])
def test_prefill_logit_jumps(window):
    """Prefill (the partial-denominator margin of 2^32): for every 7th query
    row of a head per KV head, the ladder is planted at keys before it (inside
    the window for W = 128), so its logits jump as the key tiles arrive."""
    lengths = [300, 1100]
    hq, hkv = 64, 8
    group = hq // hkv
    p = inputs.make_prefill(lengths, hq=hq, hkv=hkv, seed=800 + window)
    qf = inputs.bf16_bits_to_f32(p.q)
    kf = inputs.bf16_bits_to_f32(p.k)
    reach = (window - 1) if window else None
    for b, length in enumerate(lengths):
        s0 = int(p.cu_seqlens[b])
        for i in range(40, length, 7):
            lo = max(0, i - reach) if reach else 0
            span = i - lo
            g = i % hkv
            h0 = g * group + (i // 7) % group
            pos = [lo + int(span * (j + 1) / (len(ALPHAS) + 1)) for j in range(len(ALPHAS))]
            for pp, alpha in zip(pos, ALPHAS):
                _plant_rows(kf[:, g], [s0 + pp], qf[s0 + i, h0], alpha)
    p.k = inputs.round_to_bf16_bits(kf)
    kf = inputs.bf16_bits_to_f32(p.k)
    vf = inputs.bf16_bits_to_f32(p.v)
    o, lse = binding.prefill_varlen(bf16_to_device(p.q), bf16_to_device(p.k), bf16_to_device(p.v),
                                    f32_to_device(p.sinks), i32_to_device(p.cu_seqlens), max(lengths), window,
                                    p.scale, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = prefill_varlen_ref(qf, kf, vf, p.sinks, p.cu_seqlens, window, p.scale)
    what = "prefill jumps W=%d" % window
    assert_close_out(to_f64(o), ro, what)
    assert_close_lse(lse.cpu().numpy(), rl, what)
