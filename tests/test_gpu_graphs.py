"""HIP graph capture of the entry points (the library launches kernels on
the caller's stream and, given its buffers, allocates and clears nothing, so
a serving loop can capture a step once and replay it).

Each case captures one call into a graph with every buffer preallocated,
then replays it three times.  Before each replay the program's own eager
work writes new query values into the captured input (and synchronises);
every replay is compared with an eager call on the same inputs, bit for bit
(the same kernels over the same data), and the last one also against the
float64 oracle.
"""

import numpy as np
import pytest
import torch

from attention_gqa_flash_amd import binding, inputs
from oracle import decode_ref, prefill_append_ref, prefill_varlen_ref
from tests.helpers import assert_close_out, bf16_to_device, f32_to_device, i32_to_device, to_f64

pytestmark = pytest.mark.gpu


def _replays(run, q_dev, fresh_q, out):
    """Capture run() (which writes `out`), replay it with three query sets
    written eagerly before each replay; return the last query set."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()  # warm-up outside the capture (library load, first launch)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    last = None
    for i in range(3):
        last = fresh_q(i)
        q_dev.copy_(last)  # the program's own eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        run()  # eager, same inputs
        torch.cuda.synchronize()
        assert torch.equal(got, out), "replay %d differs from the eager call" % i
    return last


def _bf16_from(seed, shape):
    rng = np.random.default_rng(seed)
    return bf16_to_device(inputs.round_to_bf16_bits(rng.standard_normal(size=shape, dtype=np.float32)))


def test_graph_decode_splitkv_and_merge():
    d = inputs.make_decode([1000, 37, 4096, 64], hq=64, hkv=8, seed=1000)
    q, k, v = (bf16_to_device(x) for x in (d.q, d.k, d.v))
    cu, sinks = i32_to_device(d.cu_seqlens_k), f32_to_device(d.sinks)
    ws = torch.empty(binding.decode_workspace_bytes(4, 64, 64, 4), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    run = lambda: binding.decode_splitkv(q, k, v, cu, 4096, sinks, 0, d.scale, 4, workspace=ws, out=out)  # noqa: E731
    last = _replays(run, q, lambda i: _bf16_from(1001 + i, tuple(q.shape)), out)
    qf = last.float().cpu().numpy()
    kf, vf = (inputs.bf16_bits_to_f32(x) for x in (d.k, d.v))
    ro, _ = decode_ref(qf, kf, vf, d.cu_seqlens_k, d.sinks, 0, d.scale)
    assert_close_out(to_f64(out), ro, "graph decode S=4")


@pytest.mark.parametrize("window", [0, 128])
def test_graph_prefill(window):
    p = inputs.make_prefill([300, 64], hq=16, hkv=2, seed=1010 + window)
    q, k, v = (bf16_to_device(x) for x in (p.q, p.k, p.v))
    cu, sinks = i32_to_device(p.cu_seqlens), f32_to_device(p.sinks)
    out = torch.empty_like(q)
    run = lambda: binding.prefill_varlen(q, k, v, sinks, cu, 300, window, p.scale, out=out)  # noqa: E731
    last = _replays(run, q, lambda i: _bf16_from(1011 + i, tuple(q.shape)), out)
    kf, vf = (inputs.bf16_bits_to_f32(x) for x in (p.k, p.v))
    ro, _ = prefill_varlen_ref(last.float().cpu().numpy(), kf, vf, p.sinks, p.cu_seqlens, window, p.scale)
    assert_close_out(to_f64(out), ro, "graph prefill W=%d" % window)


def test_graph_split_append_prefill_and_merge():
    a = inputs.make_append([40, 7], [3000, 500], hq=16, hkv=2, seed=1020)
    q, k, v = (bf16_to_device(x) for x in (a.q, a.k, a.v))
    cq, ck, sinks = i32_to_device(a.cu_seqlens_q), i32_to_device(a.cu_seqlens_k), f32_to_device(a.sinks)
    ws = torch.empty(binding.decode_workspace_bytes(47, 16, 64, 6), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    run = lambda: binding.prefill_append(q, k, v, sinks, cq, ck, 40, 3000, 0, a.scale, out=out,  # noqa: E731
                                         num_splits=6, workspace=ws)
    last = _replays(run, q, lambda i: _bf16_from(1021 + i, tuple(q.shape)), out)
    kf, vf = (inputs.bf16_bits_to_f32(x) for x in (a.k, a.v))
    ro, _ = prefill_append_ref(last.float().cpu().numpy(), kf, vf, a.sinks, a.cu_seqlens_q, a.cu_seqlens_k, 0,
                               a.scale)
    assert_close_out(to_f64(out), ro, "graph split chunk S=6")
