"""The oracle's pins catch plausible mistakes.

Each case copies the oracle into a temporary directory, plants one mistake in
the copy (never in the repository) and checks that the pin suite
(tests/test_oracle_pins.py) then fails.  The mistakes: the sink multiplied by
the softmax scale (in the max or in the denominator), the sink dropped, the
window one key too wide, the sink in every split, the decode window one key
too wide, the wrong GQA grouping, a base-2 lse, an unweighted merge; and
for the FP8 oracle (checked by tests/test_oracle_fp8.py): exponent bias 8
instead of 7, subnormals scaled like normals, the two scales swapped, and
with several query tokens the window dropped or the query offsets read as
the key offsets; and
for the append oracle (tests/test_oracle_append.py): top-left causal
alignment, the window one key too wide, queries one position late; and for
the paged oracle (tests/test_oracle_paged.py): page and slot swapped, the
slot off by one, K and V swapped in the E4M3 multi-token form; and for the rotary oracle (tests/test_oracle_rope.py): the
rotation the wrong way, the YaRN ramp reversed, the ramp linear in the turn
count instead of the pair index, the 2 pi of the turn count dropped, the
truncated ramp ends rounded inwards, the temperature without its 0.1, V
rotated as well; and for the projection oracle
(tests/test_oracle_oproj.py): output features reversed, the bias reversed.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTATIONS = [
    ("big_m = np.maximum(row_max, z)", "big_m = np.maximum(row_max, z * scale)"),
    ("den = np.exp(z - m_safe) + e.sum(axis=1)", "den = np.exp(z * scale - m_safe) + e.sum(axis=1)"),
    ("den = np.exp(z - m_safe) + e.sum(axis=1)", "den = e.sum(axis=1)"),
    ("valid &= jj > ii - window", "valid &= jj >= ii - window"),
    ("zs = z[h] if s == 0 else -np.inf", "zs = z[h]"),
    ("lo = max(0, length - window) if window > 0 else 0", "lo = max(0, length - window - 1) if window > 0 else 0"),
    ("g = h // group", "g = h % (hq // group)"),
    ("m_safe + np.log(np.where(has, den, 1.0))", "m_safe + np.log2(np.where(has, den, 1.0))"),
    ("num = (w[..., None] * o_parts).sum(axis=0)", "num = o_parts.sum(axis=0)"),
]


FP8_MUTATIONS = [
    ("np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))", "np.ldexp(1.0 + m / 8.0, (e - 8).astype(np.int64))"),
    ("subnormal = np.ldexp(m / 8.0, -6)", "subnormal = np.ldexp(1.0 + m / 8.0, -7)"),
    ("k = float(k_scale) * e4m3_to_float64(k_codes)", "k = float(v_scale) * e4m3_to_float64(k_codes)"),
    # several query tokens: the window dropped, the queries aligned top-left
    ("return prefill_append_ref(q, k, v, sinks, cu_seqlens_q, cu_seqlens_k, window, scale, rows=rows)",
     "return prefill_append_ref(q, k, v, sinks, cu_seqlens_q, cu_seqlens_k, 0, scale, rows=rows)"),
    ("return prefill_append_ref(q, k, v, sinks, cu_seqlens_q, cu_seqlens_k, window, scale, rows=rows)",
     "return prefill_append_ref(q, k, v, sinks, cu_seqlens_q, cu_seqlens_q, window, scale, rows=rows)"),
]


APPEND_MUTATIONS = [
    ("off = lk - lq", "off = 0"),                                   # top-left causal alignment
    ("valid &= jj > pos[:, None] - window", "valid &= jj >= pos[:, None] - window"),
    ("pos = off + blk ", "pos = off + blk + 1 "),                   # query one position late
]


PAGED_MUTATIONS = [
    ("pages[bt[b, j // page_size], j % page_size]", "pages[bt[b, j % page_size], j // page_size]"),
    ("pages[bt[b, j // page_size], j % page_size]", "pages[bt[b, j // page_size], (j + 1) % page_size]"),
    ("return prefill_append_ref(q, k, v, sinks, cu_seqlens_q, cu, window, scale, rows=rows)",
     "return prefill_append_ref(q, v, k, sinks, cu_seqlens_q, cu, window, scale, rows=rows)"),
    ("return prefill_append_ref(q, k, v, sinks, cu_seqlens_q, cu, window, scale, rows=rows)",
     "return prefill_append_ref(q, k, v, sinks, cu_seqlens_q, cu, 0, scale, rows=rows)"),
    ("return decode_fp8_ref(q, k, v, k_scale, v_scale, cu, sinks, window, scale)",
     "return decode_fp8_ref(q, k, v, v_scale, k_scale, cu, sinks, window, scale)"),
    ("return decode_fp8_multi_ref(q, k, v, k_scale, v_scale, cu_seqlens_q, cu, sinks, window, scale, rows=rows)",
     "return decode_fp8_multi_ref(q, v, k, k_scale, v_scale, cu_seqlens_q, cu, sinks, window, scale, rows=rows)"),
]


ROPE_MUTATIONS = [
    ("out = np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)",
     "out = np.concatenate([x1 * c + x2 * s, x2 * c - x1 * s], axis=-1)"),      # rotation the wrong way
    ("freq = base * (1.0 - gamma) + gamma * base / factor",
     "freq = base * gamma + (1.0 - gamma) * base / factor"),                     # ramp reversed
    ("gamma = np.clip((i - low) / (high - low), 0.0, 1.0)",                      # ramp linear in turns
     "gamma = 1.0 - np.clip((original_max_position * base / (2.0 * math.pi) - beta_slow) / (beta_fast - beta_slow), "
     "0.0, 1.0)"),
    ("original_max_position / (2.0 * math.pi * turns)", "original_max_position / turns"),   # 2 pi dropped
    ("low, high = math.floor(low), math.ceil(high)", "low, high = math.ceil(low), math.floor(high)"),
    ("return freq, 0.1 * math.log(factor) + 1.0", "return freq, math.log(factor) + 1.0"),
    ("vc[slot] = v[t]", "vc[slot] = rope_ref(v[t:t + 1], positions[t:t + 1], inv_freq, attention_factor)[0]"),
]


OPROJ_MUTATIONS = [
    ("y = o @ w.T", "y = o @ w.T[::-1]"),                          # output features reversed
    ("y = y + np.asarray(bias, dtype=np.float64)[None, :]", "y = y + np.asarray(bias, dtype=np.float64)[None, ::-1]"),
]


def _run_pins(tmp_path, module, old, new, pin_file):
    for sub in ("oracle", "tests", "attention_gqa_flash_amd"):
        shutil.copytree(os.path.join(ROOT, sub), tmp_path / sub,
                        ignore=shutil.ignore_patterns("__pycache__", "*.so", "csrc"))
    src = tmp_path / "oracle" / module
    text = src.read_text()
    assert old in text, "mutation anchor not found in the oracle"
    src.write_text(text.replace(old, new))
    proc = subprocess.run(
        [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", pin_file],
        cwd=tmp_path, capture_output=True, text=True, timeout=600)
    assert proc.returncode != 0, "pins did not catch: %s -> %s\n%s" % (old, new, proc.stdout[-2000:])


@pytest.mark.parametrize("old,new", MUTATIONS, ids=[str(i) for i in range(len(MUTATIONS))])
def test_pins_catch_planted_mistake(tmp_path, old, new):
    _run_pins(tmp_path, "sink_attention.py", old, new, "tests/test_oracle_pins.py")


@pytest.mark.parametrize("old,new", FP8_MUTATIONS, ids=["fp8_%d" % i for i in range(len(FP8_MUTATIONS))])
def test_fp8_pins_catch_planted_mistake(tmp_path, old, new):
    _run_pins(tmp_path, "fp8.py", old, new, "tests/test_oracle_fp8.py")


@pytest.mark.parametrize("old,new", APPEND_MUTATIONS, ids=["append_%d" % i for i in range(len(APPEND_MUTATIONS))])
def test_append_pins_catch_planted_mistake(tmp_path, old, new):
    _run_pins(tmp_path, "append.py", old, new, "tests/test_oracle_append.py")


@pytest.mark.parametrize("old,new", PAGED_MUTATIONS, ids=["paged_%d" % i for i in range(len(PAGED_MUTATIONS))])
def test_paged_pins_catch_planted_mistake(tmp_path, old, new):
    _run_pins(tmp_path, "paged.py", old, new, "tests/test_oracle_paged.py")


@pytest.mark.parametrize("old,new", ROPE_MUTATIONS, ids=["rope_%d" % i for i in range(len(ROPE_MUTATIONS))])
def test_rope_pins_catch_planted_mistake(tmp_path, old, new):
    _run_pins(tmp_path, "rope.py", old, new, "tests/test_oracle_rope.py")


@pytest.mark.parametrize("old,new", OPROJ_MUTATIONS, ids=["oproj_%d" % i for i in range(len(OPROJ_MUTATIONS))])
def test_oproj_pins_catch_planted_mistake(tmp_path, old, new):
    _run_pins(tmp_path, "oproj.py", old, new, "tests/test_oracle_oproj.py")
