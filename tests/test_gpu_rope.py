"""GPU parity of the fused rotary step (RoPE with YaRN, Q out, K/V cache
append) against the float64 oracle.

Bar (derived): the kernel computes each rotated value in fp32 from exact
inputs and rounds it to bf16 once, so |gpu - oracle| <= 2^-8 |oracle| (half a
bf16 unit in the last place) plus fp32 rounding of the sum and of sin / cos
(<= 1e-5 at these magnitudes).  V rows are copied bit for bit; cache rows no
token names keep their contents bit for bit; tokens with slot -1 write
nothing.  Positions reach 2^31 - 1 (phases reduced in fp64).
"""

import numpy as np
import pytest
import torch

from attention_gqa_flash_amd import binding, inputs
from oracle import rope_qkv_append_ref, yarn_inv_freq_ref
from tests.helpers import bf16_to_device, i32_to_device, to_f64

pytestmark = pytest.mark.gpu

YARN = dict(rope_theta=150000.0, yarn_factor=32.0, yarn_original_max_position=4096, yarn_beta_fast=32.0,
            yarn_beta_slow=1.0)
PLAIN = dict(rope_theta=10000.0, yarn_factor=1.0)
# the same YaRN setting with the ramp ends rounded outwards (DeepSeek-V3's
# form), and a setting whose ramp spans most of the pairs
YARN_TRUNC = dict(YARN, yarn_truncate=True)
YARN_WIDE = dict(rope_theta=10000.0, yarn_factor=8.0, yarn_original_max_position=2048, yarn_beta_fast=64.0,
                 yarn_beta_slow=0.5)


def _close(got, ref, what):
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-5
    bad = err > bound
    assert not bad.any(), "%s: %d values off, worst %.3g (bound %.3g)" % (what, bad.sum(), err.max(),
                                                                         bound[np.unravel_index(err.argmax(),
                                                                                                err.shape)])


def _run_and_check(r, hq, hkv, params):
    qkv = bf16_to_device(r.qkv)
    kc = bf16_to_device(r.k_cache)
    vc = bf16_to_device(r.v_cache)
    q_out = binding.rope_qkv_append(qkv, i32_to_device(r.positions), i32_to_device(r.slot_mapping), hq, hkv, kc, vc,
                                    **params)
    torch.cuda.synchronize()
    f, m = yarn_inv_freq_ref(64, params["rope_theta"], params.get("yarn_factor", 1.0),
                             params.get("yarn_original_max_position", 4096), params.get("yarn_beta_fast", 32.0),
                             params.get("yarn_beta_slow", 1.0), params.get("yarn_truncate", False))
    rq, rk, rv = rope_qkv_append_ref(inputs.bf16_bits_to_f32(r.qkv), r.positions, hq, hkv, f, m, r.slot_mapping,
                                     inputs.bf16_bits_to_f32(r.k_cache), inputs.bf16_bits_to_f32(r.v_cache))
    _close(to_f64(q_out), rq, "q")
    _close(to_f64(kc), rk, "k cache")
    # V: copied exactly; untouched rows: unchanged bit for bit
    got_v = vc.view(torch.int16).cpu().numpy().view(np.uint16)
    want_v = r.v_cache.copy()
    hv = r.qkv[:, hq + hkv:]
    for t, sl in enumerate(r.slot_mapping):
        if sl >= 0:
            want_v[sl] = hv[t]
    assert np.array_equal(got_v, want_v)
    got_k = kc.view(torch.int16).cpu().numpy().view(np.uint16)
    untouched = np.setdiff1d(np.arange(r.k_cache.shape[0]), r.slot_mapping[r.slot_mapping >= 0])
    assert np.array_equal(got_k[untouched], r.k_cache[untouched])


@pytest.mark.parametrize("hq,hkv", [(64, 8), (8, 1), (16, 16)])
@pytest.mark.parametrize("params", [YARN, PLAIN, YARN_TRUNC, YARN_WIDE], ids=["yarn", "plain", "yarn_trunc", "yarn_wide"])
def test_rope_qkv_append(hq, hkv, params):
    r = inputs.make_rope(1000, hq, hkv, cache_rows=1500, seed=hq + hkv)
    _run_and_check(r, hq, hkv, params)


def test_rope_large_positions_and_single_token():
    r = inputs.make_rope(300, 64, 8, cache_rows=300, seed=3, max_position=2 ** 31 - 1, skip_every=0)
    r.positions[:4] = [0, 1, 2 ** 31 - 1, 131071]
    _run_and_check(r, 64, 8, YARN)
    one = inputs.make_rope(1, 64, 8, cache_rows=5, seed=4)
    _run_and_check(one, 64, 8, YARN)


def test_rope_into_paged_cache_rows():
    """Slots of a paged cache (page * page_size + slot) name rows of the
    [pages * page_size, Hkv, 64] view; the paged decode then reads them."""
    page_size, pages = 16, 40
    r = inputs.make_rope(200, 64, 8, cache_rows=page_size * pages, seed=5, skip_every=0)
    _run_and_check(r, 64, 8, YARN)


def test_rope_debug_check_reports_repeated_slot(monkeypatch):
    monkeypatch.setenv("SINKATTN_DEBUG_CHECKS", "1")
    r = inputs.make_rope(50, 16, 2, cache_rows=60, seed=6)
    _run_and_check(r, 16, 2, YARN)
    slots = r.slot_mapping.copy()
    slots[3] = slots[10] = 7
    with pytest.raises(binding.SinkAttnError) as err:
        binding.rope_qkv_append(bf16_to_device(r.qkv), i32_to_device(r.positions), i32_to_device(slots), 16, 2,
                                bf16_to_device(r.k_cache), bf16_to_device(r.v_cache), **YARN)
    assert err.value.status == 1 and "slot" in str(err.value)
