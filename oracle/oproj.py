"""Output projection with bias after attention, for the float64 oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed: the attention output of a token, its query heads
concatenated (o [N, Hq * D]), times the projection weight plus a bias:
y = o W^T + b, with W [E, Hq * D] (one row per output feature) and b [E]
(Perplexity, "GPT-OSS on day 0", section "GPT-OSS on Hopper": the output
projection carries a bias).  The pages give neither the width E nor the
weights; both are synthetic here.

Parity status: pinned by CPU tests (tests/test_oracle_oproj.py) against the
bias alone (o = 0), one-hot rows (a row of W plus b, exactly), linearity and
brute force with math.fsum.
"""

from __future__ import annotations

import numpy as np


def oproj_ref(o, w, bias) -> np.ndarray:
    """y [N, E] = o [N, K] @ w[E, K]^T + bias [E] (None = no bias), float64."""
    o = np.asarray(o, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    y = o @ w.T
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    return y
