"""The C-ABI library loads, exports every function include/sinkattn.h
declares, and rejects bad arguments on the host (no GPU call is made: every
case here fails validation before anything is launched)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sinkattn.h")
LIB = os.path.join(ROOT, "attention_gqa_flash_amd", "libsinkattn.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"SINKATTN_API\s+[\w\s\*]+?\b(sinkattn_\w+)\s*\(", text)))


def _lib():
    from attention_gqa_flash_amd import binding
    return binding.library()


def test_header_declares_the_entry_points():
    assert _declared() == sorted([
        "sinkattn_decode_paged", "sinkattn_decode_paged_fp8", "sinkattn_decode_paged_multi", "sinkattn_decode_splitkv", "sinkattn_decode_splitkv_fp8",
        "sinkattn_decode_splitkv_multi", "sinkattn_decode_splitkv_multi_fp8", "sinkattn_decode_splitkv_noalloc",
        "sinkattn_decode_paged_multi_fp8",
        "sinkattn_decode_workspace_bytes", "sinkattn_oproj_bias", "sinkattn_oproj_workspace_bytes",
        "sinkattn_rope_qkv_append",
        "sinkattn_last_error", "sinkattn_merge_lse", "sinkattn_prefill_append", "sinkattn_prefill_append_paged",
        "sinkattn_prefill_append_splitkv", "sinkattn_prefill_append_paged_splitkv",
        "sinkattn_prefill_varlen",
        "sinkattn_version"])


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(LIB)
    for name in _declared():
        assert hasattr(lib, name), name


def test_version_and_workspace_size():
    lib = _lib()
    assert b"sinkattn" in lib.sinkattn_version()
    assert lib.sinkattn_decode_workspace_bytes(64, 64, 64, 1) == 0
    rows = 16 * 64 * 64
    expect = (rows * 64 * 4 + 255) // 256 * 256 + (rows * 4 + 255) // 256 * 256
    assert lib.sinkattn_decode_workspace_bytes(64, 64, 64, 16) == expect
    assert lib.sinkattn_decode_workspace_bytes(-1, 64, 64, 4) == 0


FAKE = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below fails validation


def _prefill(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, sinks=None, cu=FAKE, batch=1, max_seqlen=16, total=16, hq=8, hkv=2,
             d=64, window=0, scale=0.125, o=FAKE, lse=None)
    a.update(kw)
    return lib.sinkattn_prefill_varlen(a["q"], a["k"], a["v"], a["sinks"], a["cu"], a["batch"], a["max_seqlen"],
                                       a["total"], a["hq"], a["hkv"], a["d"], a["window"], a["scale"], a["o"],
                                       a["lse"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(d=128), 2),
    (dict(hq=6, hkv=4), 1),
    (dict(hkv=0), 1),
    (dict(scale=0.0), 1),
    (dict(scale=float("nan")), 1),
    (dict(scale=-0.125), 1),
    (dict(batch=-1), 1),
    (dict(q=None), 1),
    (dict(cu=None), 1),
    (dict(o=ctypes.c_void_p((1 << 20) + 2)), 1),
    (dict(max_seqlen=32, total=16), 1),
    (dict(max_seqlen=40_000_000, total=40_000_000), 2),
    # one sequence's K/V rows past 2^31 bytes (32-bit row offsets)
    (dict(max_seqlen=1 << 20, total=1 << 20, hq=128, hkv=128), 2),
    # 64 KV heads x 2^25 query tiles: more than 2^24 - 1 workgroups
    (dict(max_seqlen=1000, total=1 << 30, hq=64, hkv=64), 2),
])
def test_prefill_rejects(kw, status):
    lib = _lib()
    assert _prefill(lib, **kw) == status
    assert lib.sinkattn_last_error()


def test_prefill_empty_is_ok_without_launch():
    lib = _lib()
    assert _prefill(lib, batch=0) == 0
    assert _prefill(lib, total=0, max_seqlen=0) == 0


FAKE2 = ctypes.c_void_p(2 << 20)  # a second offsets array, likewise never read


def _append(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, sinks=None, cuq=FAKE, cuk=FAKE2, batch=2, mq=16, mk=64, tq=20, tk=100,
             hq=8, hkv=2, d=64, window=0, scale=0.125, o=FAKE, lse=None)
    a.update(kw)
    return lib.sinkattn_prefill_append(a["q"], a["k"], a["v"], a["sinks"], a["cuq"], a["cuk"], a["batch"], a["mq"],
                                       a["mk"], a["tq"], a["tk"], a["hq"], a["hkv"], a["d"], a["window"],
                                       a["scale"], a["o"], a["lse"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(d=128), 2),
    (dict(hq=6, hkv=4), 1),
    (dict(scale=0.0), 1),
    (dict(batch=-1), 1),
    (dict(mk=-1), 1),
    (dict(cuk=None), 1),
    (dict(k=None), 1),
    (dict(v=ctypes.c_void_p((1 << 20) + 4)), 1),
    (dict(mq=32, tq=16), 1),                     # max_seqlen_q above total_q
    (dict(mk=200, tk=100), 1),                   # max_seqlen_k above total_k
    (dict(mk=0, tk=0), 1),                       # queries without keys
    (dict(cuk=FAKE, mk=16, tk=100), 1),          # one offsets array, different maxima or totals
    # one sequence's K/V rows past 2^31 bytes (32-bit row offsets)
    (dict(mk=1 << 20, tk=1 << 20, hq=128, hkv=128), 2),
])
def test_append_rejects(kw, status):
    lib = _lib()
    assert _append(lib, **kw) == status
    assert lib.sinkattn_last_error()


def test_append_empty_is_ok_without_launch():
    lib = _lib()
    assert _append(lib, batch=0) == 0
    assert _append(lib, tq=0, mq=0) == 0


def _append_split(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, sinks=None, cuq=FAKE, cuk=FAKE2, batch=2, mq=16, mk=64, tq=20, tk=100,
             hq=8, hkv=2, d=64, window=0, scale=0.125, splits=4, ws=None, ws_bytes=0, o=FAKE, lse=None)
    a.update(kw)
    return lib.sinkattn_prefill_append_splitkv(a["q"], a["k"], a["v"], a["sinks"], a["cuq"], a["cuk"], a["batch"],
                                               a["mq"], a["mk"], a["tq"], a["tk"], a["hq"], a["hkv"], a["d"],
                                               a["window"], a["scale"], a["splits"], a["ws"], a["ws_bytes"], a["o"],
                                               a["lse"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(splits=0), 1),
    (dict(splits=1025), 2),
    (dict(), 3),                                  # no workspace
    (dict(ws=FAKE, ws_bytes=100), 3),
    (dict(ws=ctypes.c_void_p((1 << 20) + 16), ws_bytes=1 << 30), 1),  # misaligned workspace
    (dict(d=128), 2),
    (dict(mk=0, tk=0), 1),
    (dict(cuk=FAKE, mk=16, tk=100), 1),          # one offsets array, different maxima or totals
    (dict(batch=-1), 1),
])
def test_append_split_rejects(kw, status):
    lib = _lib()
    assert _append_split(lib, **kw) == status
    assert lib.sinkattn_last_error()


def test_append_split_empty_is_ok_without_launch():
    lib = _lib()
    assert _append_split(lib, batch=0) == 0
    assert _append_split(lib, tq=0, mq=0) == 0


def test_append_split_workspace_size():
    lib = _lib()
    need = lib.sinkattn_decode_workspace_bytes(20, 8, 64, 4)
    rows = 4 * 20 * 8
    assert need == -(-rows * 64 * 4 // 256) * 256 + -(-rows * 4 // 256) * 256


def _decode(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, cu=FAKE, batch=4, max_seqlen=100, sinks=None, hq=64, hkv=8, d=64,
             window=0, scale=0.125, splits=1, ws=None, ws_bytes=0, o=FAKE, lse=None)
    a.update(kw)
    return lib.sinkattn_decode_splitkv(a["q"], a["k"], a["v"], a["cu"], a["batch"], a["max_seqlen"], a["sinks"],
                                       a["hq"], a["hkv"], a["d"], a["window"], a["scale"], a["splits"], a["ws"],
                                       a["ws_bytes"], a["o"], a["lse"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), 2),
    (dict(hq=64, hkv=1), 2),          # group of 64 > 32
    (dict(splits=0), 1),
    (dict(splits=4), 3),              # no workspace
    (dict(splits=4, ws=FAKE, ws_bytes=100), 3),
    (dict(splits=4, ws=ctypes.c_void_p((1 << 20) + 16), ws_bytes=1 << 30), 1),  # misaligned workspace
    (dict(max_seqlen=0), 1),
    (dict(k=None), 1),
    (dict(scale=float("inf")), 1),
])
def test_decode_rejects(kw, status):
    lib = _lib()
    assert _decode(lib, **kw) == status
    assert lib.sinkattn_last_error()


def _decode_fp8(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, ks=0.0625, vs=0.0625, cu=FAKE, batch=4, max_seqlen=100, sinks=None, hq=64,
             hkv=8, d=64, window=0, scale=0.125, splits=1, ws=None, ws_bytes=0, o=FAKE, lse=None)
    a.update(kw)
    return lib.sinkattn_decode_splitkv_fp8(a["q"], a["k"], a["v"], a["ks"], a["vs"], a["cu"], a["batch"],
                                           a["max_seqlen"], a["sinks"], a["hq"], a["hkv"], a["d"], a["window"],
                                           a["scale"], a["splits"], a["ws"], a["ws_bytes"], a["o"], a["lse"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(ks=0.0), 1),
    (dict(vs=-1.0), 1),
    (dict(ks=float("nan")), 1),
    (dict(vs=float("inf")), 1),
    (dict(d=128), 2),
    (dict(splits=4), 3),              # no workspace
    (dict(v=None), 1),
    (dict(k=ctypes.c_void_p((1 << 20) + 8)), 1),  # misaligned cache
])
def test_decode_fp8_rejects(kw, status):
    lib = _lib()
    assert _decode_fp8(lib, **kw) == status
    assert lib.sinkattn_last_error()


def test_decode_fp8_empty_batch_is_ok_without_launch():
    assert _decode_fp8(_lib(), batch=0) == 0


@pytest.mark.parametrize("args,status", [
    ((FAKE, FAKE, 0, 4, 8, 64), 1),
    ((FAKE, FAKE, 2, 4, 8, 32), 2),
    ((None, FAKE, 2, 4, 8, 64), 1),
    ((FAKE, FAKE, 2, 4, 0, 64), 1),
])
def test_merge_rejects(args, status):
    lib = _lib()
    assert lib.sinkattn_merge_lse(*args, FAKE, None, None) == status


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from attention_gqa_flash_amd import binding
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "_LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(binding.SinkAttnError):
        binding.library()


def _decode_multi(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, cuq=FAKE, cuk=FAKE2, batch=4, mq=4, mk=100, tq=16, sinks=None, hq=64, hkv=8,
             d=64, window=0, scale=0.125, splits=1, ws=None, ws_bytes=0, o=FAKE, lse=None)
    a.update(kw)
    return lib.sinkattn_decode_splitkv_multi(a["q"], a["k"], a["v"], a["cuq"], a["cuk"], a["batch"], a["mq"],
                                             a["mk"], a["tq"], a["sinks"], a["hq"], a["hkv"], a["d"], a["window"],
                                             a["scale"], a["splits"], a["ws"], a["ws_bytes"], a["o"], a["lse"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(mq=9), 2),                  # 9 tokens x 8 heads > 64 columns
    (dict(hq=64, hkv=2, mq=3), 2),    # a group of 32 leaves room for two tokens only
    (dict(cuq=None), 1),
    (dict(hq=8, hkv=8, mq=20, tq=16), 1),  # max_seqlen_q above total_q
    (dict(mq=-1), 1),
    (dict(splits=4), 3),              # no workspace
    (dict(splits=4, ws=FAKE, ws_bytes=4 * 16 * 64 * 65 * 4 - 1), 3),  # sized for the batch, not total_q
    (dict(mk=0), 1),
    (dict(d=128), 2),
])
def test_decode_multi_rejects(kw, status):
    lib = _lib()
    assert _decode_multi(lib, **kw) == status
    assert lib.sinkattn_last_error()


def test_decode_multi_empty_is_ok_without_launch():
    lib = _lib()
    assert _decode_multi(lib, batch=0) == 0
    assert _decode_multi(lib, batch=0, cuq=None) == 0
    assert _decode_multi(lib, tq=0, mq=0) == 0


def _decode_paged(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, lens=FAKE2, batch=4, mp=8, ps=16, npg=40, mk=100, sinks=None, hq=64,
             hkv=8, d=64, window=0, scale=0.125, splits=1, ws=None, ws_bytes=0, o=FAKE, lse=None)
    a.update(kw)
    return lib.sinkattn_decode_paged(a["q"], a["k"], a["v"], a["bt"], a["lens"], a["batch"], a["mp"], a["ps"],
                                     a["npg"], a["mk"], a["sinks"], a["hq"], a["hkv"], a["d"], a["window"],
                                     a["scale"], a["splits"], a["ws"], a["ws_bytes"], a["o"], a["lse"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(ps=8), 2),                  # below 16
    (dict(ps=24), 2),                 # not a power of two
    (dict(mp=0), 1),
    (dict(npg=0), 1),
    (dict(mp=6), 1),                  # 6 x 16 < max_seqlen_k
    (dict(bt=None), 1),
    (dict(lens=None), 1),
    (dict(npg=1 << 27, ps=32), 2),    # pool past 2^31 tokens
    (dict(splits=4), 3),              # no workspace
    (dict(d=128), 2),
    (dict(k=ctypes.c_void_p((1 << 20) + 2)), 1),
])
def test_decode_paged_rejects(kw, status):
    lib = _lib()
    assert _decode_paged(lib, **kw) == status
    assert lib.sinkattn_last_error()


def test_decode_paged_empty_is_ok_without_launch():
    lib = _lib()
    assert _decode_paged(lib, batch=0) == 0
    assert _decode_paged(lib, batch=0, bt=None, lens=None) == 0


def _decode_paged_fp8(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, ks=0.5, vs=0.5, bt=FAKE, lens=FAKE2, batch=4, mp=8, ps=16, npg=40, mk=100,
             sinks=None, hq=64, hkv=8, d=64, window=0, scale=0.125, splits=1, ws=None, ws_bytes=0, o=FAKE, lse=None)
    a.update(kw)
    return lib.sinkattn_decode_paged_fp8(a["q"], a["k"], a["v"], a["ks"], a["vs"], a["bt"], a["lens"], a["batch"],
                                         a["mp"], a["ps"], a["npg"], a["mk"], a["sinks"], a["hq"], a["hkv"], a["d"],
                                         a["window"], a["scale"], a["splits"], a["ws"], a["ws_bytes"], a["o"],
                                         a["lse"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(ps=24), 2),                 # page size not a power of two
    (dict(mp=6), 1),                  # 6 x 16 < max_seqlen_k
    (dict(lens=None), 1),
    (dict(ks=0.0), 1),
    (dict(vs=float("inf")), 1),
    (dict(ks=float("nan")), 1),
    (dict(splits=4), 3),              # no workspace
    (dict(v=ctypes.c_void_p((1 << 20) + 8)), 1),
])
def test_decode_paged_fp8_rejects(kw, status):
    lib = _lib()
    assert _decode_paged_fp8(lib, **kw) == status
    assert lib.sinkattn_last_error()


def test_decode_paged_fp8_empty_is_ok_without_launch():
    lib = _lib()
    assert _decode_paged_fp8(lib, batch=0) == 0


def _decode_paged_multi(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, lens=FAKE2, cuq=FAKE2, batch=4, mp=8, ps=16, npg=40, mq=4, mk=100,
             tq=16, sinks=None, hq=64, hkv=8, d=64, window=0, scale=0.125, splits=1, ws=None, ws_bytes=0, o=FAKE,
             lse=None)
    a.update(kw)
    return lib.sinkattn_decode_paged_multi(a["q"], a["k"], a["v"], a["bt"], a["lens"], a["cuq"], a["batch"],
                                           a["mp"], a["ps"], a["npg"], a["mq"], a["mk"], a["tq"], a["sinks"],
                                           a["hq"], a["hkv"], a["d"], a["window"], a["scale"], a["splits"], a["ws"],
                                           a["ws_bytes"], a["o"], a["lse"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(ps=24), 2),                 # page size not a power of two
    (dict(mp=6), 1),                  # 6 x 16 < max_seqlen_k
    (dict(bt=None), 1),
    (dict(cuq=None), 1),
    (dict(mq=9), 2),                  # 9 tokens x 8 heads > 64 columns
    (dict(mq=4, tq=3), 1),            # more than total_q
    (dict(splits=4), 3),              # no workspace
    (dict(splits=4, ws=FAKE, ws_bytes=(1 << 20)), 3),  # workspace sized for batch rows, not total_q
    (dict(q=ctypes.c_void_p((1 << 20) + 2)), 1),
])
def test_decode_paged_multi_rejects(kw, status):
    lib = _lib()
    assert _decode_paged_multi(lib, **kw) == status
    assert lib.sinkattn_last_error()


def test_decode_paged_multi_empty_is_ok_without_launch():
    lib = _lib()
    assert _decode_paged_multi(lib, batch=0) == 0
    assert _decode_paged_multi(lib, batch=0, bt=None, lens=None, cuq=None) == 0
    assert _decode_paged_multi(lib, tq=0, mq=0) == 0


def _prefill_paged(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, lens=FAKE2, cuq=FAKE2, batch=4, mp=8, ps=16, npg=40, mq=64, mk=100,
             tq=200, sinks=None, hq=64, hkv=8, d=64, window=0, scale=0.125, o=FAKE, lse=None)
    a.update(kw)
    return lib.sinkattn_prefill_append_paged(a["q"], a["k"], a["v"], a["bt"], a["lens"], a["cuq"], a["batch"],
                                             a["mp"], a["ps"], a["npg"], a["mq"], a["mk"], a["tq"], a["sinks"],
                                             a["hq"], a["hkv"], a["d"], a["window"], a["scale"], a["o"], a["lse"],
                                             None)


@pytest.mark.parametrize("kw,status", [
    (dict(ps=24), 2),                 # page size not a power of two
    (dict(mp=6), 1),                  # 6 x 16 < max_seqlen_k
    (dict(bt=None), 1),
    (dict(cuq=None), 1),
    (dict(mq=300), 1),                # more than total_q
    (dict(mk=0), 1),                  # queries need keys
    (dict(d=128), 2),
    (dict(o=ctypes.c_void_p((1 << 20) + 2)), 1),
])
def test_prefill_append_paged_rejects(kw, status):
    lib = _lib()
    assert _prefill_paged(lib, **kw) == status
    assert lib.sinkattn_last_error()


def test_prefill_append_paged_empty_is_ok_without_launch():
    lib = _lib()
    assert _prefill_paged(lib, batch=0) == 0
    assert _prefill_paged(lib, tq=0, mq=0) == 0


def _rope(lib, **kw):
    a = dict(qkv=FAKE, pos=FAKE2, slots=FAKE2, t=16, hq=64, hkv=8, d=64, theta=150000.0, s=32.0, L=4096, bf=32.0,
             bs=1.0, q=FAKE, kc=FAKE, vc=FAKE, rows=100)
    a.update(kw)
    return lib.sinkattn_rope_qkv_append(a["qkv"], a["pos"], a["slots"], a["t"], a["hq"], a["hkv"], a["d"],
                                        ctypes.c_double(a["theta"]), ctypes.c_double(a["s"]), a["L"],
                                        ctypes.c_double(a["bf"]), ctypes.c_double(a["bs"]), a.get("trunc", 0), a["q"],
                                        a["kc"], a["vc"], a["rows"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(d=128), 2),
    (dict(t=-1), 1),
    (dict(hkv=0), 1),
    (dict(theta=1.0), 1),
    (dict(theta=float("inf")), 1),
    (dict(s=0.0), 1),
    (dict(s=float("nan")), 1),
    (dict(L=0), 1),                   # YaRN without an original context
    (dict(bf=1.0, bs=1.0), 1),        # empty ramp
    (dict(bf=32.0, bs=0.0), 1),       # a turn count of 0 has no pair index
    (dict(bf=32.0, bs=-1.0, trunc=1), 1),
    (dict(qkv=None), 1),
    (dict(slots=None), 1),
    (dict(kc=ctypes.c_void_p((1 << 20) + 8)), 1),
])
def test_rope_rejects(kw, status):
    lib = _lib()
    assert _rope(lib, **kw) == status
    assert lib.sinkattn_last_error()


def test_rope_empty_and_plain_rope_arguments():
    lib = _lib()
    assert _rope(lib, t=0) == 0
    assert _rope(lib, t=0, s=1.0, L=0, bf=0.0, bs=0.0) == 0   # no YaRN: its parameters are not read


@pytest.mark.parametrize("args,status", [
    ((FAKE, FAKE, None, 64, 4000, 2880, FAKE), 2),    # in_features not a multiple of 128
    ((FAKE, FAKE, None, 64, 4096, 2890, FAKE), 2),    # out_features not a multiple of 32
    ((FAKE, FAKE, None, -1, 4096, 2880, FAKE), 1),
    ((FAKE, FAKE, None, 64, 0, 2880, FAKE), 1),
    ((None, FAKE, None, 64, 4096, 2880, FAKE), 1),
    ((FAKE, ctypes.c_void_p((1 << 20) + 2), None, 64, 4096, 2880, FAKE), 1),
    ((FAKE, FAKE, None, 65536 * 64, 4096, 2880, FAKE), 2),
    ((FAKE, FAKE, None, 64, 4096, 2880, FAKE), 3),    # split K needs a workspace
])
def test_oproj_rejects(args, status):
    lib = _lib()
    assert lib.sinkattn_oproj_bias(*args, None, 0, None) == status
    assert lib.sinkattn_last_error()
    assert lib.sinkattn_oproj_bias(FAKE, FAKE, None, 0, 4096, 2880, FAKE, None, 0, None) == 0


def test_oproj_workspace_size():
    lib = _lib()
    # 64 rows: 45 tiles of 64 features, K split 4 ways (180 workgroups); 8192 rows: no split
    assert lib.sinkattn_oproj_workspace_bytes(64, 4096, 2880) == 4 * 64 * 2880 * 4
    assert lib.sinkattn_oproj_workspace_bytes(8192, 4096, 2880) == 0
    assert lib.sinkattn_oproj_workspace_bytes(0, 4096, 2880) == 0


def _noalloc(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, cu=FAKE2, b=64, mk=8192, sinks=None, hq=64, hkv=8, d=64, w=0, scale=0.125, s=16,
             o=FAKE, lse=None)
    a.update(kw)
    return lib.sinkattn_decode_splitkv_noalloc(a["q"], a["k"], a["v"], a["cu"], a["b"], a["mk"], a["sinks"], a["hq"],
                                               a["hkv"], a["d"], a["w"], ctypes.c_float(a["scale"]), a["s"], a["o"],
                                               a["lse"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(s=32), 3),                  # 64 x 64 heads x 32 splits: 34.1 MB of partials, above the 32 MiB scratch
    (dict(b=4096, s=2), 3),
    (dict(d=128), 2),
    (dict(hq=60), 1),
    (dict(s=0), 1),
    (dict(scale=0.0), 1),
    (dict(q=None), 1),
])
def test_noalloc_decode_rejects_before_any_launch(kw, status):
    """The allocation-free decode validates its arguments and its scratch
    limit on the host (no device is touched on these paths)."""
    lib = _lib()
    assert _noalloc(lib, **kw) == status
    msg = lib.sinkattn_last_error()
    assert msg
    if status == 3:
        assert b"static scratch" in msg


def test_noalloc_scratch_limit_matches_workspace_sizes():
    """31 splits of the 64 x 64-head decode fit the 32 MiB scratch, 32 do not."""
    lib = _lib()
    limit = 32 << 20
    assert lib.sinkattn_decode_workspace_bytes(64, 64, 64, 31) <= limit < lib.sinkattn_decode_workspace_bytes(64, 64, 64, 32)
    assert _noalloc(lib, b=0) == 0
