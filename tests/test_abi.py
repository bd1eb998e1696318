"""C ABI checks that need no GPU: the library loads, exports every entry
point the header declares, and rejects bad arguments before any HIP call."""
import ctypes
import json
import os
import re

import pytest

import zero_shot_rope_bifocal_amd as jl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "jetlong.h")


def _lib():
    if not os.path.exists(jl.library_path()):
        pytest.skip("libjetlong.so not built (run __graft_entry__.build())")
    return jl.lib()


def test_header_symbols_exported():
    L = _lib()
    names = re.findall(r"\b(jl_[a-z_0-9]+)\s*\(", open(HEADER).read())
    assert len(set(names)) >= 11
    for n in set(names):
        assert hasattr(L, n), f"{n} declared in jetlong.h but not exported"


def test_group_size_matches_golden():
    _lib()
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "group_size.json")))
    for c in g["group_size"]:
        assert jl.group_size(c["L"], c["w_pretrained"]) == c["G"]
    with pytest.raises(jl.JetLongError):
        jl.group_size(5, 0)
    with pytest.raises(jl.JetLongError):
        jl.group_size(-1, 4)


def _prefill(L, **kw):
    a = dict(q=1, k=1, v=1, o=1, lse=None, dtype=jl.JL_BF16, cu_q=1, cu_k=None, B=1, total_q=64,
             total_k=64, max_q=64, max_k=64, Hq=8, Hkv=2, d=128, wp=32, w0=4, theta=1e4, scale=0.0,
             ws=256, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)  # noqa: E731
    return L.jl_bifocal_prefill(vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["o"]), vp(a["lse"]), a["dtype"],
                                vp(a["cu_q"]), vp(a["cu_k"]), a["B"], a["total_q"], a["total_k"],
                                a["max_q"], a["max_k"], a["Hq"], a["Hkv"], a["d"], a["wp"], a["w0"],
                                a["theta"], a["scale"], vp(a["ws"]), a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), -2), (dict(d=96), -2), (dict(Hq=6, Hkv=4), -1), (dict(Hkv=0), -1),
    (dict(wp=0), -1), (dict(w0=-1), -1), (dict(theta=0.0), -1), (dict(theta=float("nan")), -1),
    (dict(scale=-1.0), -1), (dict(q=None), -1), (dict(cu_q=None), -1), (dict(total_q=65), -1),
    (dict(max_q=65), -1), (dict(ws=None), -3), (dict(ws_bytes=16), -3), (dict(ws=257), -3),
    (dict(B=-1), -1), (dict(total_k=80), -1),
])
def test_prefill_rejects_before_any_launch(kw, code):
    L = _lib()
    assert _prefill(L, **kw) == code
    assert L.jl_last_error().decode() != ""


def test_prefill_bf16_key_span_limit():
    # bf16 tiles are addressed with 31-bit byte offsets per KV head:
    # (roundup64(total_k) + 64 B) * d * 2 <= 2^31 - 1
    L = _lib()
    big = dict(total_k=1 << 23, max_k=64, cu_k=1)
    assert _prefill(L, **big) == -2
    assert "2^31" in L.jl_last_error().decode()
    # just inside the limit the call gets past the check (and stops at the missing workspace)
    assert _prefill(L, total_k=(1 << 23) - 128, max_k=64, cu_k=1, ws=None) == -3
    # fp32 does not use these tiles
    assert _prefill(L, dtype=jl.JL_F32, ws=None, **big) == -3
    # head_dim 64 halves the bytes per key
    assert _prefill(L, d=64, ws=None, **big) == -3


def test_prefill_empty_batch_is_ok():
    L = _lib()
    assert _prefill(L, B=0, q=None, k=None, v=None, o=None, cu_q=None, ws=None) == 0
    assert _prefill(L, total_q=0, total_k=0, q=None, ws=None) == 0


def _decode(L, **kw):
    a = dict(q=256, kc=256, vc=256, sb=1 << 20, ss=1024, sh=128, o=1, lse=None, dtype=jl.JL_BF16,
             seq_L=1, B=2, max_L=64, Hq=8, Hkv=2, d=128, wp=32, w0=4, theta=1e4, scale=0.0, ws=256,
             ws_bytes=1 << 40)
    a.update(kw)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)  # noqa: E731
    return L.jl_bifocal_decode(vp(a["q"]), vp(a["kc"]), vp(a["vc"]), a["sb"], a["ss"], a["sh"], vp(a["o"]),
                               vp(a["lse"]), a["dtype"], vp(a["seq_L"]), a["B"], a["max_L"], a["Hq"],
                               a["Hkv"], a["d"], a["wp"], a["w0"], a["theta"], a["scale"], vp(a["ws"]),
                               a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=3), -2), (dict(d=32), -2), (dict(Hq=64, Hkv=2), -2), (dict(Hq=9), -1),
    (dict(seq_L=None), -1), (dict(max_L=0), -1), (dict(ss=64), -1), (dict(sh=100), -1),
    (dict(kc=258), -1), (dict(ws=None), -3), (dict(ws_bytes=1), -3), (dict(wp=0), -1),
])
def test_decode_rejects_before_any_launch(kw, code):
    L = _lib()
    assert _decode(L, **kw) == code


def test_workspace_sizes():
    _lib()
    a = jl.prefill_workspace_size(jl.JL_BF16, 1, 131072, 131072, 32, 8, 128)
    # cos/sin table + two rotated key copies + transposed values (padded rows)
    assert a >= 131072 * 64 * 8 + 3 * 8 * 131072 * 128 * 2
    assert jl.prefill_workspace_size(jl.JL_F32, 1, 2048, 2048, 2, 2, 64) >= 2048 * 32 * 8
    assert jl.prefill_workspace_size(9, 1, 1, 1, 1, 1, 64) == 0
    assert jl.decode_workspace_size(jl.JL_BF16, 16, 131072, 32, 8, 128) > 131072 * 64 * 8


def test_tile_shape():
    _lib()
    assert jl.prefill_tile_shape(jl.JL_BF16, 32, 8, 128) == (64, 64)
    assert jl.prefill_tile_shape(jl.JL_BF16, 8, 8, 128) == (256, 64)
    assert jl.prefill_tile_shape(jl.JL_F32, 2, 2, 64) == (64, 32)


def test_status_strings():
    L = _lib()
    for c in (0, -1, -2, -3, -4):
        assert L.jl_status_string(c)
    assert jl.version().count(".") == 2


def test_unknown_flags_rejected():
    """The *_ex entry points reject flag bits they do not know before any HIP
    call (null pointers would otherwise be the first complaint)."""
    L = _lib()
    rc = L.jl_bifocal_decode_ex(None, None, None, 0, 0, 0, None, None, 1, None, 1, 1, 1, 1, 128, 1, 0, 1e4,
                                0.0, None, 0, None, 2)
    assert rc == -1 and b"flag" in L.jl_last_error()
    rc = L.jl_bifocal_prefill_prepare_ex(None, None, 1, None, 1, 1, 1, 1, 128, 1, 1e4, None, 0, None, 8)
    assert rc == -1 and b"flag" in L.jl_last_error()


def test_prefill_ie_workspace_and_rejections():
    """The merged route needs the prefill workspace plus three fp32 O rows and
    three LSE rows; it rejects an undersized workspace, bad sizes and unknown
    flags before any HIP call."""
    L = _lib()
    base = jl.prefill_workspace_size(jl.JL_BF16, 1, 4096, 4096, 32, 8, 128)
    ie = jl.prefill_ie_workspace_size(jl.JL_BF16, 1, 4096, 4096, 4096, 32, 8, 128)
    assert ie >= base + 3 * 4096 * 32 * 128 * 4 + 3 * 32 * 4096 * 4
    assert jl.prefill_ie_workspace_size(jl.JL_F32, 1, 100, 100, 100, 2, 2, 64) >= 3 * 100 * 2 * 64 * 4
    assert jl.prefill_ie_workspace_size(5, 1, 1, 1, 1, 1, 1, 64) == 0
    vp = ctypes.c_void_p
    small = jl.prefill_workspace_size(jl.JL_BF16, 1, 64, 64, 8, 2, 128)
    assert small < jl.prefill_ie_workspace_size(jl.JL_BF16, 1, 64, 64, 64, 8, 2, 128)
    args = [vp(1), vp(1), vp(1), vp(1), None, jl.JL_BF16, vp(1), None, 1, 64, 64, 64, 64, 8, 2, 128, 32, 4, 1e4,
            0.0, vp(256), small, None]
    assert L.jl_bifocal_prefill_ie(*args, 0) == -3          # the plain prefill workspace is too small
    assert b"needed" in L.jl_last_error()
    bad = list(args)
    bad[15] = 96
    assert L.jl_bifocal_prefill_ie(*bad, 0) == -2
    assert L.jl_bifocal_prefill_ie(*args, 4) == -1 and b"flag" in L.jl_last_error()


def _decode_table(L, **kw):
    a = dict(q=256, kc=256, vc=256, sb=1 << 20, ss=1024, sh=128, o=1, lse=None, dtype=jl.JL_BF16,
             seq_L=1, B=2, max_L=64, Hq=8, Hkv=2, d=128, wp=32, w0=4, scale=0.0, tab=256, tab_bytes=1 << 40,
             tab_rows=64, ws=256, ws_bytes=1 << 40, flags=0)
    a.update(kw)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)  # noqa: E731
    return L.jl_bifocal_decode_with_table(vp(a["q"]), vp(a["kc"]), vp(a["vc"]), a["sb"], a["ss"], a["sh"],
                                          vp(a["o"]), vp(a["lse"]), a["dtype"], vp(a["seq_L"]), a["B"],
                                          a["max_L"], a["Hq"], a["Hkv"], a["d"], a["wp"], a["w0"], a["scale"],
                                          vp(a["tab"]), a["tab_bytes"], a["tab_rows"], vp(a["ws"]),
                                          a["ws_bytes"], None, a["flags"])


@pytest.mark.parametrize("kw,code", [
    (dict(tab=None), -1), (dict(tab_rows=63), -1), (dict(tab_bytes=100), -1), (dict(tab=257), -1),
    (dict(ws=None), -3), (dict(ws_bytes=8), -3), (dict(flags=2), -1), (dict(d=96), -2), (dict(Hq=9), -1),
])
def test_decode_with_table_rejects_before_any_launch(kw, code):
    L = _lib()
    assert _decode_table(L, **kw) == code
    assert L.jl_last_error().decode() != ""


def test_rope_table_and_key_rows_reject_bad_args():
    L = _lib()
    vp = ctypes.c_void_p
    assert jl.rope_table_size(131072, 128) == 131072 * 64 * 8 + 131072 * 128 * 2
    assert jl.rope_table_size(10, 96) == 0
    assert L.jl_bifocal_rope_table(100, 96, 1e4, vp(256), 1 << 30, None) == -2
    assert L.jl_bifocal_rope_table(100, 128, 0.0, vp(256), 1 << 30, None) == -1
    assert L.jl_bifocal_rope_table(100, 128, 1e4, None, 1 << 30, None) == -1
    assert L.jl_bifocal_rope_table(100, 128, 1e4, vp(256), 16, None) == -1
    assert L.jl_bifocal_rope_table(0, 128, 1e4, None, 0, None) == 0
    assert L.jl_bifocal_decode_key_rows(vp(1), 1, 10, 0, 4, 1, 0, vp(1), None) == -1
    assert L.jl_bifocal_decode_key_rows(vp(1), 1, 10, 2, 0, 1, 0, vp(1), None) == -1
    assert L.jl_bifocal_decode_key_rows(None, 1, 10, 2, 4, 1, 0, vp(1), None) == -1
    assert L.jl_bifocal_decode_key_rows(vp(1), 1, 10, 2, 4, 1, 4, vp(1), None) == -1
    assert L.jl_bifocal_decode_key_rows(None, 0, 10, 2, 4, 1, 0, None, None) == 0
    # partial states only: far below the decode workspace that also holds the table rows
    assert 0 < jl.decode_with_table_workspace_size(jl.JL_BF16, 16, 131072, 32, 8, 128) < \
        jl.decode_workspace_size(jl.JL_BF16, 16, 131072, 32, 8, 128) - 131072 * 64 * 8
