"""SINKATTN_DEBUG_CHECKS=1: the device-side preconditions of the C ABI are
checked before any attention kernel runs.

Valid inputs pass and give the same result as without the checks; each
violated precondition (offsets, decode length, sinks, NaN/Inf in q/k, merge
partials) returns SINKATTN_ERR_INVALID_ARG with a message naming it.  No
attention kernel is launched on the invalid inputs.
"""

import numpy as np
import pytest
import torch

from attention_gqa_flash_amd import binding, inputs
from tests.helpers import bf16_to_device, f32_to_device, i32_to_device

pytestmark = pytest.mark.gpu

INVALID_ARG = 1


@pytest.fixture
def debug_checks(monkeypatch):
    monkeypatch.setenv("SINKATTN_DEBUG_CHECKS", "1")


def _prefill(p, cu=None, sinks=None, q=None, k=None):
    qd = q if q is not None else bf16_to_device(p.q)
    kd = k if k is not None else bf16_to_device(p.k)
    return binding.prefill_varlen(qd, kd, bf16_to_device(p.v),
                                  f32_to_device(p.sinks if sinks is None else sinks),
                                  i32_to_device(p.cu_seqlens if cu is None else cu), max(p.lengths), 0, p.scale)


def _status(fn):
    with pytest.raises(binding.SinkAttnError) as err:
        fn()
        torch.cuda.synchronize()
    assert err.value.status == INVALID_ARG, err.value
    return str(err.value)


def test_valid_inputs_pass_and_match(debug_checks, monkeypatch):
    p = inputs.make_prefill([40, 90], hq=16, hkv=2, seed=21)
    checked = _prefill(p)
    torch.cuda.synchronize()
    monkeypatch.setenv("SINKATTN_DEBUG_CHECKS", "0")
    plain = _prefill(p)
    torch.cuda.synchronize()
    assert torch.equal(checked, plain)


def test_prefill_offsets(debug_checks):
    p = inputs.make_prefill([40, 90], hq=16, hkv=2, seed=22)
    assert "non-decreasing" in _status(lambda: _prefill(p, cu=np.array([0, 100, 90], np.int32)))
    assert "cu_seqlens[0]" in _status(lambda: _prefill(p, cu=np.array([5, 40, 130], np.int32)))
    assert "total_tokens" in _status(lambda: _prefill(p, cu=np.array([0, 40, 131], np.int32)))


def test_prefill_sinks_and_values(debug_checks):
    p = inputs.make_prefill([40, 90], hq=16, hkv=2, seed=23)
    bad = p.sinks.copy()
    bad[3] = np.inf
    assert "sink" in _status(lambda: _prefill(p, sinks=bad))
    bad[3] = np.nan
    assert "sink" in _status(lambda: _prefill(p, sinks=bad))
    ok = p.sinks.copy()
    ok[3] = -np.inf  # a head without sink is valid
    _prefill(p, sinks=ok)
    torch.cuda.synchronize()
    q = bf16_to_device(p.q)
    q.view(torch.int16)[7, 2, 5] = 0x7fc0  # NaN
    assert "q holds" in _status(lambda: _prefill(p, q=q))
    k = bf16_to_device(p.k)
    k.view(torch.int16)[100, 1, 0] = 0x7f80  # +Inf
    assert "k holds" in _status(lambda: _prefill(p, k=k))


def test_decode_offsets_and_lengths(debug_checks):
    d = inputs.make_decode([5, 70, 33], hq=16, hkv=2, seed=24)
    q, k, v = (bf16_to_device(x) for x in (d.q, d.k, d.v))
    sinks = f32_to_device(d.sinks)

    def run(cu, max_len=70, splits=1):
        return binding.decode_splitkv(q, k, v, i32_to_device(cu), max_len, sinks, 0, d.scale, splits)

    run(d.cu_seqlens_k)
    torch.cuda.synchronize()
    assert "empty" in _status(lambda: run(np.array([0, 5, 5, 108], np.int32)))
    assert "longer" in _status(lambda: run(d.cu_seqlens_k, max_len=40, splits=4))
    assert "non-decreasing" in _status(lambda: run(np.array([0, 75, 70, 108], np.int32)))


def test_merge_partials(debug_checks):
    rng = np.random.default_rng(25)
    parts, n, h = 3, 4, 8
    o_parts = torch.from_numpy(rng.standard_normal((parts, n, h, 64)).astype(np.float32)).cuda()
    lse_parts = torch.from_numpy(rng.standard_normal((parts, n, h)).astype(np.float32)).cuda()
    lse_parts[1, 2, 3] = float("-inf")  # an empty part is valid
    binding.merge_lse(o_parts, lse_parts)
    torch.cuda.synchronize()
    bad = lse_parts.clone()
    bad[0, 0, 0] = float("nan")
    assert "lse_parts" in _status(lambda: binding.merge_lse(o_parts, bad))
    bad_o = o_parts.clone()
    bad_o[2, 1, 1, 7] = float("inf")
    assert "o_parts" in _status(lambda: binding.merge_lse(bad_o, lse_parts))
