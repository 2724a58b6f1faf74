"""Bit-identical masking: which keys reach each output row.

Probe: q = 0 (every logit is 0, so every visible key gets weight
1 / (|J(i)| + e^z) > 0), sinks = 0, and a one-hot V with V[j, :, c] = 1 iff
the key's local position j equals 64 r + c (probe round r).  Output element
(i, h, c) is then exactly 0.0 iff key 64 r + c is not in J(i).  The zero
pattern is compared bit for bit with the oracle's integer mask (causal,
128-token-style windows of every width around the tile sizes, varlen packs,
decode key ranges under every split count).
"""

import numpy as np
import pytest
import torch

from attention_gqa_flash_amd import binding
from oracle import decode_key_range, prefill_mask_ref
from tests.helpers import i32_to_device

pytestmark = pytest.mark.gpu

LENGTHS = [1, 2, 63, 64, 65, 127, 128, 129, 255, 256, 257, 1000]
WINDOWS = [0, 1, 63, 64, 65, 127, 128, 129, 1000, 1001]


def _one_hot_v(lengths, hkv, r):
    t = sum(lengths)
    v = torch.zeros((t, hkv, 64), dtype=torch.bfloat16)
    base = 0
    for length in lengths:
        for c in range(64):
            j = 64 * r + c
            if j < length:
                v[base + j, :, c] = 1.0
        base += length
    return v.cuda()


@pytest.mark.parametrize("window", WINDOWS)
def test_prefill_mask_pattern(window):
    hq, hkv = 16, 2
    lengths = LENGTHS
    t = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    q = torch.zeros((t, hq, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.randn((t, hkv, 64), device="cuda").to(torch.bfloat16)
    sinks = torch.zeros(hq, dtype=torch.float32, device="cuda")
    cu_d = i32_to_device(cu)
    masks = [prefill_mask_ref(length, window) for length in lengths]
    for r in range((max(lengths) + 63) // 64):
        v = _one_hot_v(lengths, hkv, r)
        o = binding.prefill_varlen(q, k, v, sinks, cu_d, max(lengths), window, 0.125)
        nz = (o.float() != 0).cpu().numpy()              # [T, Hq, 64]
        for b, length in enumerate(lengths):
            keys = 64 * r + np.arange(64)
            inside = keys < length
            expect = np.zeros((length, 64), dtype=bool)
            expect[:, inside] = masks[b][:, keys[inside]]
            got = nz[cu[b]:cu[b + 1]]                     # [L, Hq, 64]
            for h in range(hq):
                assert np.array_equal(got[:, h, :], expect), (window, r, length, h)


@pytest.mark.parametrize("splits", [1, 4, 32])
def test_decode_mask_pattern(splits):
    hq, hkv = 64, 8
    lengths = [1, 127, 128, 129, 8192]
    t = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    cu_d = i32_to_device(cu)
    q = torch.zeros((len(lengths), hq, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.randn((t, hkv, 64), device="cuda").to(torch.bfloat16)
    sinks = torch.zeros(hq, dtype=torch.float32, device="cuda")
    for window in (0, 1, 127, 128, 129):
        rounds = sorted(set([0, 1, 2] + [(8192 - window) // 64 + d for d in (-1, 0, 1)] + [127]))
        for r in rounds:
            if r < 0 or 64 * r >= max(lengths):
                continue
            v = _one_hot_v(lengths, hkv, r)
            o = binding.decode_splitkv(q, k, v, cu_d, max(lengths), sinks, window, 0.125, splits)
            nz = (o.float() != 0).cpu().numpy()          # [B, Hq, 64]
            for b, length in enumerate(lengths):
                lo, hi = decode_key_range(length, window)
                keys = 64 * r + np.arange(64)
                expect = (keys >= lo) & (keys < hi)
                for h in range(hq):
                    assert np.array_equal(nz[b, h], expect), (splits, window, r, length, h)
