"""The allocation-free decode (sinkattn_decode_splitkv_noalloc, for callers
that cannot allocate device memory) against the workspace decode
(sinkattn_decode_splitkv) it shares its kernels with: the same outputs bit
for bit on two calls in a row, the second with a smaller input (the static
scratch keeps the first call's partials), and both within the oracle bar.
"""

import numpy as np
import pytest
import torch

from attention_gqa_flash_amd import binding, inputs
from oracle import decode_ref
from tests.helpers import assert_close_lse, assert_close_out, bf16_to_device, f32_to_device, i32_to_device, to_f64

pytestmark = pytest.mark.gpu


def _case(lengths, seed):
    d = inputs.make_decode(lengths, 64, 8, 64, seed=seed)
    dev = dict(q=bf16_to_device(d.q), k=bf16_to_device(d.k), v=bf16_to_device(d.v), sinks=f32_to_device(d.sinks),
               cu=i32_to_device(d.cu_seqlens_k))
    return d, dev


def _both(dev, max_len, window, splits, scale):
    o1, l1 = binding.decode_splitkv(dev["q"], dev["k"], dev["v"], dev["cu"], max_len, dev["sinks"], window, scale,
                                    splits, return_lse=True)
    o2 = torch.empty_like(dev["q"])
    l2 = torch.empty((dev["q"].shape[0], dev["q"].shape[1]), dtype=torch.float32, device=dev["q"].device)
    binding.decode_splitkv_noalloc(dev["q"], dev["k"], dev["v"], dev["cu"], max_len, dev["sinks"], window, scale,
                                   splits, out=o2, lse=l2)
    torch.cuda.synchronize()
    return o1, l1, o2, l2


def _check(d, dev, window, splits):
    max_len = int(max(d.lengths))
    o1, l1, o2, l2 = _both(dev, max_len, window, splits, d.scale)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), (window, splits)
    assert torch.equal(l1, l2), (window, splits)
    qf, kf, vf = (inputs.bf16_bits_to_f32(x) for x in (d.q, d.k, d.v))
    ro, rl = decode_ref(qf, kf, vf, d.cu_seqlens_k, d.sinks, window, d.scale)
    assert_close_out(to_f64(o2), ro, "noalloc S=%d W=%d" % (splits, window))
    assert_close_lse(l2.cpu().numpy().astype(np.float64), rl, "noalloc S=%d W=%d" % (splits, window))


def test_noalloc_matches_workspace_decode_on_two_calls():
    """First call: 24 sequences of 600-5000 keys at 16 splits (partials fill
    part of the scratch); second call: 5 shorter sequences at 4 splits, which
    must not see the first call's partials."""
    rng = np.random.default_rng(11)
    big, dev_big = _case([int(x) for x in rng.integers(600, 5000, 24)], seed=31)
    small, dev_small = _case([300, 77, 1500, 1, 640], seed=32)
    _check(big, dev_big, 0, 16)
    _check(small, dev_small, 0, 4)
    _check(small, dev_small, 128, 4)
    _check(big, dev_big, 0, 1)          # one split: no scratch involved


def test_noalloc_full_size_decode_and_limit():
    """The 64 x 8192 decode at 16 splits (17 MB of partials), then a request
    above the 32 MiB scratch, which is refused before any launch."""
    d, dev = _case([8192] * 64, seed=0)
    o1, l1, o2, l2 = _both(dev, 8192, 0, 16, d.scale)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
    with pytest.raises(binding.SinkAttnError) as err:
        binding.decode_splitkv_noalloc(dev["q"], dev["k"], dev["v"], dev["cu"], 8192, dev["sinks"], 0, d.scale, 32)
    assert err.value.status == 3 and "static scratch" in str(err.value)
