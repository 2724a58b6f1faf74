"""Shared test helpers: host<->device marshalling and error metrics."""

import numpy as np

# Tolerances on bf16 outputs against the float64 oracle (fp32 accumulation).
MAX_ABS = 2e-2
MEAN_ABS = 2e-3
# lse is fp32, but the prefill kernel sums the bf16-rounded probabilities it
# also feeds to P.V (so the output weights stay consistent with their
# normaliser).  Each weight carries a relative rounding error of at most
# 2^-9 (bf16 round-to-nearest-even), so ln(den) may move by up to
# 2^-9 = 1.95e-3; twice that covers the fp32 exp2/log2 approximations.
LSE_ABS = 4e-3


def bf16_to_device(bits, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def f32_to_device(x, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def i32_to_device(x, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(device)


def to_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def err_stats(got, ref):
    diff = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    return float(diff.max()) if diff.size else 0.0, float(diff.mean()) if diff.size else 0.0


def assert_close_out(got, ref, what=""):
    assert np.all(np.isfinite(got)), "%s: non-finite output" % what
    mx, mean = err_stats(got, ref)
    assert mx <= MAX_ABS and mean <= MEAN_ABS, "%s: max|err| %.3g (<= %.0e), mean|err| %.3g (<= %.0e)" % (
        what, mx, MAX_ABS, mean, MEAN_ABS)
    return mx, mean


def assert_close_lse(got, ref, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), "%s: -inf pattern of lse differs" % what
    fin = np.isfinite(ref)
    mx = float(np.abs(got[fin] - ref[fin]).max()) if fin.any() else 0.0
    assert mx <= LSE_ABS, "%s: lse max|err| %.3g" % (what, mx)
