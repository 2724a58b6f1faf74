"""GPU parity: the HIP library against the float64 CPU oracle, element by
element, at sizes the oracle finishes in seconds (several tiles, ragged
tails, empty and one-token sequences, every layer kind).

Bar: max |err| <= 2e-2 and mean |err| <= 2e-3 on the bf16 outputs (the
contract); lse within tests.helpers.LSE_ABS with an identical -inf pattern
(a bound derived from the kernels' arithmetic, not part of the contract).
"""

import numpy as np
import pytest
import torch

from attention_gqa_flash_amd import binding, inputs
from oracle import decode_ref, decode_split_partials_ref, merge_ref, prefill_varlen_ref
from tests.helpers import (assert_close_lse, assert_close_out, bf16_to_device, f32_to_device, i32_to_device,
                           to_f64)

pytestmark = pytest.mark.gpu


def _prefill_case(p, window, with_sinks=True):
    q, k, v = (bf16_to_device(x) for x in (p.q, p.k, p.v))
    sinks = f32_to_device(p.sinks) if with_sinks else None
    cu = i32_to_device(p.cu_seqlens)
    o, lse = binding.prefill_varlen(q, k, v, sinks, cu, max(p.lengths), window, p.scale, return_lse=True)
    torch.cuda.synchronize()
    qf, kf, vf = (inputs.bf16_bits_to_f32(x) for x in (p.q, p.k, p.v))
    ro, rl = prefill_varlen_ref(qf, kf, vf, p.sinks if with_sinks else None, p.cu_seqlens, window, p.scale)
    return to_f64(o), lse.cpu().numpy(), ro, rl


def test_tiny_prefill_config():
    """1 sequence of 256, 4 q heads / 1 KV head, causal, seed 0."""
    p = inputs.tiny_prefill(seed=0)
    o, lse, ro, rl = _prefill_case(p, 0)
    print("tiny: max|err| %.3g mean|err| %.3g" % assert_close_out(o, ro, "tiny"))
    assert_close_lse(lse, rl, "tiny")


@pytest.mark.parametrize("window", [0, 1, 5, 31, 32, 64, 127, 128, 129, 1000])
@pytest.mark.parametrize("hq,hkv", [(8, 2), (16, 2), (24, 2), (64, 8), (8, 8), (32, 1), (32, 16)])
def test_varlen_prefill_small(window, hq, hkv):
    lengths = [1, 31, 32, 33, 64, 65, 127, 200, 517]
    if hq == 64:
        lengths = [1, 33, 130, 300]
    p = inputs.make_prefill(lengths, hq=hq, hkv=hkv, seed=window + 100 * hq + hkv)
    o, lse, ro, rl = _prefill_case(p, window)
    assert_close_out(o, ro, "varlen W=%d G=%d" % (window, hq // hkv))
    assert_close_lse(lse, rl, "varlen")


def test_prefill_without_sinks_and_neg_inf_heads():
    p = inputs.make_prefill([70, 129], hq=16, hkv=2, seed=3, no_sink_heads=(0, 5, 9, 15))
    for window in (0, 128):
        o, lse, ro, rl = _prefill_case(p, window)
        assert_close_out(o, ro, "-inf heads")
        assert_close_lse(lse, rl, "-inf heads")
        o, lse, ro, rl = _prefill_case(p, window, with_sinks=False)
        assert_close_out(o, ro, "no sinks")
        assert_close_lse(lse, rl, "no sinks")


def test_prefill_large_sink_gives_zero():
    p = inputs.make_prefill([96], hq=8, hkv=1, seed=4)
    p.sinks[:] = 40.0  # exp(40 - s) dwarfs every key for N(0,1) data at scale 1/8
    o, lse, ro, rl = _prefill_case(p, 0)
    assert np.abs(o).max() < 1e-10
    assert_close_out(o, ro, "sink=+40")
    assert_close_lse(lse, rl, "sink=+40")


def test_prefill_empty_sequences_in_pack():
    p = inputs.make_prefill([0, 45, 0, 0, 70, 0], hq=16, hkv=2, seed=6)
    o, lse, ro, rl = _prefill_case(p, 0)
    assert_close_out(o, ro, "empty seqs")
    assert_close_lse(lse, rl, "empty seqs")


@pytest.mark.parametrize("n_seqs,max_len", [(150, 90), (4100, 3)])
def test_prefill_many_sequences(n_seqs, max_len):
    """Batches past 64 sequences: the work-item search takes two and three
    rounds (up to 64 sequences take one)."""
    rng = np.random.default_rng(n_seqs)
    lengths = [int(x) for x in rng.integers(0, max_len + 1, size=n_seqs)]
    p = inputs.make_prefill(lengths, hq=8, hkv=2, seed=n_seqs)
    for window in (0, 2):
        o, lse, ro, rl = _prefill_case(p, window)
        assert_close_out(o, ro, "%d seqs W=%d" % (n_seqs, window))
        assert_close_lse(lse, rl, "%d seqs" % n_seqs)


def test_prefill_rows_past_the_last_sequence_untouched():
    """Buffers longer than cu_seqlens[batch]: rows past it are not written."""
    p = inputs.make_prefill([40, 0, 97], hq=16, hkv=2, seed=8)
    pad = 75
    q, k, v = (bf16_to_device(np.concatenate([x, np.zeros((pad,) + x.shape[1:], x.dtype)])) for x in (p.q, p.k, p.v))
    out = torch.full(q.shape, 3.0, dtype=torch.bfloat16, device=q.device)
    binding.prefill_varlen(q, k, v, f32_to_device(p.sinks), i32_to_device(p.cu_seqlens), 97, 0, p.scale, out=out)
    torch.cuda.synchronize()
    t = int(p.cu_seqlens[-1])
    assert bool((out[t:] == 3.0).all())
    qf, kf, vf = (inputs.bf16_bits_to_f32(x) for x in (p.q, p.k, p.v))
    ro, _ = prefill_varlen_ref(qf, kf, vf, p.sinks, p.cu_seqlens, 0, p.scale)
    assert_close_out(to_f64(out[:t]), ro, "padded buffers")


def test_prefill_deterministic():
    p = inputs.make_prefill([300, 77], hq=64, hkv=8, seed=7)
    q, k, v = (bf16_to_device(x) for x in (p.q, p.k, p.v))
    sinks, cu = f32_to_device(p.sinks), i32_to_device(p.cu_seqlens)
    ref = binding.prefill_varlen(q, k, v, sinks, cu, 300, 0, p.scale)
    for _ in range(10):
        again = binding.prefill_varlen(q, k, v, sinks, cu, 300, 0, p.scale)
        assert torch.equal(again.view(torch.int16), ref.view(torch.int16))


# ---------------------------------------------------------------------------
# Decode and merge
# ---------------------------------------------------------------------------

def _decode_case(d, window, splits):
    q, k, v = (bf16_to_device(x) for x in (d.q, d.k, d.v))
    o, lse = binding.decode_splitkv(q, k, v, i32_to_device(d.cu_seqlens_k), max(d.lengths),
                                    f32_to_device(d.sinks), window, d.scale, splits, return_lse=True)
    torch.cuda.synchronize()
    return to_f64(o), lse.cpu().numpy()


@pytest.mark.parametrize("window", [0, 1, 128])
def test_decode_small_all_splits(window):
    lengths = [1, 5, 31, 32, 33, 100, 1000, 4097]
    d = inputs.make_decode(lengths, hq=64, hkv=8, seed=11 + window)
    qf, kf, vf = (inputs.bf16_bits_to_f32(x) for x in (d.q, d.k, d.v))
    ro, rl = decode_ref(qf, kf, vf, d.cu_seqlens_k, d.sinks, window, d.scale)
    outs = []
    for s in (1, 2, 3, 4, 16, 32, 100):
        o, lse = _decode_case(d, window, s)
        assert_close_out(o, ro, "decode W=%d S=%d" % (window, s))
        assert_close_lse(lse, rl, "decode W=%d S=%d" % (window, s))
        outs.append(o)
    for a in outs[1:]:
        assert_close_out(a, outs[0], "split agreement")


@pytest.mark.parametrize("hq,hkv", [(4, 1), (8, 8), (32, 1), (12, 4)])
def test_decode_group_shapes(hq, hkv):
    d = inputs.make_decode([7, 64, 300], hq=hq, hkv=hkv, seed=hq * 10 + hkv)
    qf, kf, vf = (inputs.bf16_bits_to_f32(x) for x in (d.q, d.k, d.v))
    for window, s in ((0, 1), (0, 5), (16, 3)):
        ro, rl = decode_ref(qf, kf, vf, d.cu_seqlens_k, d.sinks, window, d.scale)
        o, lse = _decode_case(d, window, s)
        assert_close_out(o, ro, "decode G=%d" % (hq // hkv))
        assert_close_lse(lse, rl, "decode G=%d" % (hq // hkv))


@pytest.mark.parametrize("hq,hkv", [(64, 8), (32, 1), (8, 8)])
@pytest.mark.parametrize("window,splits", [(0, 4), (0, 64), (128, 32), (128, 200), (7, 3), (1, 2)])
def test_decode_short_splits(hq, hkv, window, splits):
    """Splits of at most 32 keys, which the library evaluates as one range
    (the merge is exact): short caches, window layers, more splits than
    keys, sinks of -inf on some heads and no sink tensor."""
    lengths = [1, 2, 17, 32, 33, 64, 127, 128, 129, 500]
    if window == 0:
        lengths = [x for x in lengths if x <= 128]
    nos = tuple(h for h in (0, 5, hq - 1) if h < hq)
    d = inputs.make_decode(lengths, hq=hq, hkv=hkv, seed=window * 7 + splits + hq)
    d.sinks[list(nos)] = -np.inf
    qf, kf, vf = (inputs.bf16_bits_to_f32(x) for x in (d.q, d.k, d.v))
    ro, rl = decode_ref(qf, kf, vf, d.cu_seqlens_k, d.sinks, window, d.scale)
    o, lse = _decode_case(d, window, splits)
    assert_close_out(o, ro, "short splits W=%d S=%d" % (window, splits))
    assert_close_lse(lse, rl, "short splits")
    q, k, v = (bf16_to_device(x) for x in (d.q, d.k, d.v))
    o2 = binding.decode_splitkv(q, k, v, i32_to_device(d.cu_seqlens_k), max(d.lengths), None, window, d.scale,
                                splits)
    torch.cuda.synchronize()
    ro2, _ = decode_ref(qf, kf, vf, d.cu_seqlens_k, None, window, d.scale)
    assert_close_out(to_f64(o2), ro2, "short splits, no sinks")


@pytest.mark.parametrize("hq,hkv", [(16, 4), (20, 5), (48, 6), (56, 7), (64, 8), (128, 4)])
@pytest.mark.parametrize("splits", [4, 6, 13])
def test_decode_one_wave_per_kv_head(hq, hkv, splits):
    """Four or more splits of at least 128 keys over 4 to 8 KV heads: one
    workgroup per (sequence, split), one wave per KV head; ragged lengths so
    some splits are short or empty, and a -inf sink."""
    d = inputs.make_decode([1, 200, 1500, 2600], hq=hq, hkv=hkv, seed=hq + splits)
    d.sinks[1] = -np.inf
    qf, kf, vf = (inputs.bf16_bits_to_f32(x) for x in (d.q, d.k, d.v))
    for window in (0, 1200):  # 1200 keys: >= 128 per split at S = 4 and 6, not at 13
        ro, rl = decode_ref(qf, kf, vf, d.cu_seqlens_k, d.sinks, window, d.scale)
        o, lse = _decode_case(d, window, splits)
        assert_close_out(o, ro, "wave per head G=%d S=%d W=%d" % (hq // hkv, splits, window))
        assert_close_lse(lse, rl, "wave per head")


def test_decode_one_wave_per_kv_head_several_splits_per_workgroup():
    """Enough (sequence, split) pairs that consecutive splits share a
    workgroup (40 x 32 here): partials of every split, empty ones included,
    merged."""
    rng = np.random.default_rng(41)
    lengths = [4200 if i % 3 == 0 else int(rng.integers(1, 5000)) for i in range(40)]
    d = inputs.make_decode(lengths, hq=16, hkv=4, seed=41)
    qf, kf, vf = (inputs.bf16_bits_to_f32(x) for x in (d.q, d.k, d.v))
    ro, rl = decode_ref(qf, kf, vf, d.cu_seqlens_k, d.sinks, 0, d.scale)
    for splits in (32, 27):
        o, lse = _decode_case(d, 0, splits)
        assert_close_out(o, ro, "several splits per workgroup S=%d" % splits)
        assert_close_lse(lse, rl, "several splits per workgroup")


@pytest.mark.parametrize("hq,hkv", [(16, 2), (24, 6), (64, 8), (40, 10)])
def test_decode_single_split_kv_head_pairs(hq, hkv):
    """One split of more than 1024 keys over an even number of KV heads:
    eight-wave workgroups serving two KV heads each (four interleaved waves
    per head, merged through LDS); full and 2000-key window layers."""
    d = inputs.make_decode([1, 1100, 3000, 5000], hq=hq, hkv=hkv, seed=hq * 3 + hkv)
    d.sinks[hq - 1] = -np.inf
    qf, kf, vf = (inputs.bf16_bits_to_f32(x) for x in (d.q, d.k, d.v))
    for window in (0, 2000):
        ro, rl = decode_ref(qf, kf, vf, d.cu_seqlens_k, d.sinks, window, d.scale)
        o, lse = _decode_case(d, window, 1)
        assert_close_out(o, ro, "head pairs G=%d W=%d" % (hq // hkv, window))
        assert_close_lse(lse, rl, "head pairs")


def test_decode_partials_match_oracle_partials():
    """Run decode with S = 4 and check the merged result against the oracle's
    own split partials merged on the CPU (sink in chunk 0 only)."""
    d = inputs.make_decode([3, 50, 129, 513], hq=16, hkv=2, seed=12)
    qf, kf, vf = (inputs.bf16_bits_to_f32(x) for x in (d.q, d.k, d.v))
    op, lp = decode_split_partials_ref(qf, kf, vf, d.cu_seqlens_k, d.sinks, 0, d.scale, 4)
    mo, ml = merge_ref(op, lp)
    o, lse = _decode_case(d, 0, 4)
    assert_close_out(o, mo, "partials")
    assert_close_lse(lse, ml, "partials")


def test_merge_kernel():
    rng = np.random.default_rng(13)
    s, n, h, dim = 5, 37, 6, 64
    o_parts = rng.standard_normal((s, n, h, dim)).astype(np.float32)
    lse_parts = (3.0 * rng.standard_normal((s, n, h))).astype(np.float32)
    lse_parts[1, :5] = -np.inf          # some empty partials
    lse_parts[:, 7, 2] = -np.inf        # one row entirely empty
    o_parts[1, :5] = 0.0
    o_parts[:, 7, 2] = 0.0
    o, lse = binding.merge_lse(f32_to_device(o_parts), f32_to_device(lse_parts), return_lse=True)
    torch.cuda.synchronize()
    ro, rl = merge_ref(o_parts.astype(np.float64), lse_parts.astype(np.float64))
    assert_close_out(to_f64(o), ro, "merge")
    assert_close_lse(lse.cpu().numpy(), rl, "merge")
    assert np.all(to_f64(o)[7, 2] == 0.0)


def test_decode_deterministic():
    d = inputs.make_decode([4000, 17], hq=64, hkv=8, seed=14)
    q, k, v = (bf16_to_device(x) for x in (d.q, d.k, d.v))
    cu, sinks = i32_to_device(d.cu_seqlens_k), f32_to_device(d.sinks)
    for s in (1, 8):
        ref = binding.decode_splitkv(q, k, v, cu, 4000, sinks, 0, d.scale, s)
        for _ in range(5):
            again = binding.decode_splitkv(q, k, v, cu, 4000, sinks, 0, d.scale, s)
            assert torch.equal(again.view(torch.int16), ref.view(torch.int16))
