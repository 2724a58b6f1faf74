"""GPU parity of the FP8 (E4M3) KV-cache decode against the float64 oracle
(K = k_scale * e4m3(code), V = v_scale * e4m3(code); vLLM, "GPT-OSS
performance optimizations on NVIDIA Blackwell", FlashInfer integration).

Every decode kernel shape is reached: one short or long split (two-wave,
head-pair and four-wave workgroups), long splits per wave, a wave per KV
head, the KV-head-pair kernel (G <= 8 over an even number of KV heads: a
wave streams both heads of a pair), and window layers whose splits are
evaluated as one range.  Bar as the
bf16 path: max |err| <= 2e-2, mean |err| <= 2e-3, lse within 4e-3.
"""

import numpy as np
import pytest
import torch

from attention_gqa_flash_amd import binding, inputs
from oracle import decode_fp8_ref
from tests.helpers import assert_close_lse, assert_close_out, bf16_to_device, f32_to_device, i32_to_device, to_f64

pytestmark = pytest.mark.gpu


def _u8(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def _case(d, window, splits, sinks=True):
    q = bf16_to_device(d.q)
    o, lse = binding.decode_splitkv_fp8(q, _u8(d.k), _u8(d.v), d.k_scale, d.v_scale, i32_to_device(d.cu_seqlens_k),
                                        max(d.lengths), f32_to_device(d.sinks) if sinks else None, window, d.scale,
                                        splits, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = decode_fp8_ref(inputs.bf16_bits_to_f32(d.q), d.k, d.v, d.k_scale, d.v_scale, d.cu_seqlens_k,
                            d.sinks if sinks else None, window, d.scale)
    return to_f64(o), lse.cpu().numpy(), ro, rl


@pytest.mark.parametrize("hq,hkv", [(64, 8), (8, 1), (16, 2), (32, 1), (20, 5)])
@pytest.mark.parametrize("splits", [1, 2, 4, 16])
def test_fp8_decode_kernel_shapes(hq, hkv, splits):
    d = inputs.make_decode_fp8([1, 31, 300, 1500, 2100], hq=hq, hkv=hkv, seed=hq * 7 + hkv + splits)
    d.sinks[0] = -np.inf
    for window in (0, 128, 1800):
        o, lse, ro, rl = _case(d, window, splits)
        assert_close_out(o, ro, "fp8 G=%d S=%d W=%d" % (hq // hkv, splits, window))
        assert_close_lse(lse, rl, "fp8")


@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 8), (24, 4), (64, 8), (128, 16), (4, 2)])
@pytest.mark.parametrize("splits", [1, 3, 16, 64])
def test_fp8_pair_kernel(hq, hkv, splits):
    """The KV-head-pair kernel (one query token, G <= 8, an even number of KV
    heads) at G = 1, 2, 6 and 8, with 1-, 2-, 4- and 8-wave workgroups (the
    wave count follows sequences x pairs x splits and the tiles per split),
    ragged lengths with more splits than some sequences have tiles, and
    window layers (evaluated as one range)."""
    d = inputs.make_decode_fp8([1, 33, 700, 4100, 32, 2049], hq=hq, hkv=hkv, seed=hq * 11 + hkv + splits)
    d.sinks[1] = -np.inf
    for window in (0, 128, 1800):
        o, lse, ro, rl = _case(d, window, splits)
        assert_close_out(o, ro, "fp8 pair G=%d Hkv=%d S=%d W=%d" % (hq // hkv, hkv, splits, window))
        assert_close_lse(lse, rl, "fp8 pair")


@pytest.mark.parametrize("k_scale,v_scale", [(1.0 / 16, 1.0 / 8), (0.0371, 0.0213), (1.0, 1.0 / 64)])
def test_fp8_decode_scales(k_scale, v_scale):
    d = inputs.make_decode_fp8([700, 64, 1200], hq=16, hkv=4, seed=9, k_scale=k_scale, v_scale=v_scale)
    for splits in (1, 5):
        o, lse, ro, rl = _case(d, 0, splits)
        assert_close_out(o, ro, "fp8 scales %g %g" % (k_scale, v_scale))
        assert_close_lse(lse, rl, "fp8 scales")


@pytest.mark.parametrize("hq,hkv", [(64, 8), (16, 2)])
def test_fp8_decode_without_sinks_and_long_context(hq, hkv):
    """Includes long splits per wave (16/2 heads, 4 splits of 1250+ keys)."""
    d = inputs.make_decode_fp8([32768, 5000], hq=hq, hkv=hkv, seed=10, sink_std=2 ** 0.5)
    for splits in (1, 4, 32):
        o, lse, ro, rl = _case(d, 0, splits, sinks=False)
        assert_close_out(o, ro, "fp8 no sinks S=%d" % splits)
        assert_close_lse(lse, rl, "fp8 no sinks")


def test_fp8_debug_check_reports_nan_codes(monkeypatch):
    monkeypatch.setenv("SINKATTN_DEBUG_CHECKS", "1")
    d = inputs.make_decode_fp8([40, 70], hq=8, hkv=2, seed=11)
    o, lse, ro, rl = _case(d, 0, 1)  # valid codes pass the checks
    assert_close_out(o, ro, "fp8 debug valid")
    k = d.k.copy()
    k[50, 1, 3] = 0x7F  # E4M3 NaN
    with pytest.raises(binding.SinkAttnError) as err:
        binding.decode_splitkv_fp8(bf16_to_device(d.q), _u8(k), _u8(d.v), d.k_scale, d.v_scale,
                                   i32_to_device(d.cu_seqlens_k), 70, f32_to_device(d.sinks), 0, d.scale, 1)
    assert err.value.status == 1 and "k" in str(err.value)
