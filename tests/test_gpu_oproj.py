"""GPU parity of the output projection with bias (y = o W^T + b) against the
float64 oracle, on the same bf16 o and W.

Bar (derived): fp32 accumulation over K = 4096 products of N(0,1) o and
N(0, 1/K) W, then one rounding to bf16: |gpu - oracle| <= 2^-8 |y| (half a
bf16 ulp) + 1e-3 (fp32 accumulation, far above its typical 1e-5 here).
Row counts on and off the 32- and 64-row blocks, K from 128 to 4096, with and
without bias, and the projection of a real decode output.
"""

import numpy as np
import pytest
import torch

from attention_gqa_flash_amd import binding, inputs
from oracle import oproj_ref
from tests.helpers import bf16_to_device, f32_to_device, i32_to_device, to_f64

pytestmark = pytest.mark.gpu


def _case(n, k, e, seed, with_bias=True):
    rng = np.random.default_rng(seed)
    o = inputs.round_to_bf16_bits(rng.standard_normal((n, k), dtype=np.float32))
    w = inputs.round_to_bf16_bits((rng.standard_normal((e, k)) / np.sqrt(k)).astype(np.float32))
    b = rng.standard_normal(e).astype(np.float32) if with_bias else None
    return o, w, b


def _check(o_bits, w_bits, b, y):
    ref = oproj_ref(inputs.bf16_bits_to_f32(o_bits), inputs.bf16_bits_to_f32(w_bits), b)
    got = to_f64(y)
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-3
    assert np.all(err <= bound), "worst %.3g" % err.max()


@pytest.mark.parametrize("n", [1, 31, 32, 63, 64, 65, 200])
@pytest.mark.parametrize("k,e", [(4096, 2880), (128, 32), (640, 96)])
def test_oproj(n, k, e):
    o, w, b = _case(n, k, e, seed=n + k + e)
    y = binding.oproj_bias(bf16_to_device(o), bf16_to_device(w), f32_to_device(b))
    torch.cuda.synchronize()
    _check(o, w, b, y)


def test_oproj_without_bias_and_prefill_rows():
    o, w, _ = _case(2000, 4096, 2880, seed=5, with_bias=False)
    y = binding.oproj_bias(bf16_to_device(o), bf16_to_device(w), None)
    torch.cuda.synchronize()
    _check(o, w, None, y)


def test_oproj_of_a_decode_output():
    """Decode 64 x 4096 (64/8 heads), then project its [64, 4096] output."""
    d = inputs.make_decode([4096] * 64, hq=64, hkv=8, seed=6)
    o = binding.decode_splitkv(bf16_to_device(d.q), bf16_to_device(d.k), bf16_to_device(d.v),
                               i32_to_device(d.cu_seqlens_k), 4096, f32_to_device(d.sinks), 0, d.scale, 4)
    _, w, b = _case(1, 4096, 2880, seed=7)
    y = binding.oproj_bias(o, bf16_to_device(w), f32_to_device(b))
    torch.cuda.synchronize()
    o_bits = o.view(torch.int16).cpu().numpy().view(np.uint16).reshape(64, 4096)
    _check(o_bits, w, b, y)


def test_oproj_debug_check_names_the_operand(monkeypatch):
    monkeypatch.setenv("SINKATTN_DEBUG_CHECKS", "1")
    o, w, b = _case(64, 4096, 2880, seed=8)
    y = binding.oproj_bias(bf16_to_device(o), bf16_to_device(w), f32_to_device(b))
    torch.cuda.synchronize()
    _check(o, w, b, y)
    w_bad = w.copy()
    w_bad[5, 17] = 0x7FC0  # bf16 NaN
    with pytest.raises(binding.SinkAttnError) as err:
        binding.oproj_bias(bf16_to_device(o), bf16_to_device(w_bad), f32_to_device(b))
    assert err.value.status == 1 and "w holds NaN" in str(err.value)
