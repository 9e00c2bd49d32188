"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/mla_lowbit.h declares, and rejects bad arguments with
the documented status before anything is enqueued."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def m():
    import bit_mla_kv_amd as m
    return m


def declared_functions():
    hdr = open(os.path.join(ROOT, "include", "mla_lowbit.h")).read()
    hdr = re.sub(r"/\*.*?\*/", "", hdr, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_lowbit_\w+)\s*\(", hdr)))


def test_exports_every_declared_symbol(m):
    names = declared_functions()
    assert len(names) >= 6
    for n in names:
        assert hasattr(m.lib, n), n
    assert set(names) == set(m.EXPORTS)


def test_page_bytes(m):
    assert m.page_bytes(m.make_layout(4)) == 64 * (256 + 32 + 36) == 20736
    assert m.page_bytes(m.make_layout(2)) == 64 * (128 + 32 + 36) == 12544
    bad = m.make_layout(3)
    assert m.page_bytes(bad) == 0
    assert "bits" in m.lib.mla_lowbit_last_error().decode()
    v = m.make_layout(4)
    v.abi_version = 2
    assert m.page_bytes(v) == 0


def _cache(m, **kw):
    c = m.CacheDesc(m.make_layout(4), 0x10000, 8, 0x20000, 0x30000, 2, 0x40000, 4)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_append_validation(m):
    L = m.lib
    A = L.mla_lowbit_quantize_append
    assert A(None, 0x1000, 0x1000, 0x1000, 0x1000, 1, None) == m.ERR_INVALID_ARG
    c = _cache(m)
    assert A(ctypes.byref(c), 0x1000, 0x1000, 0x1000, 0x1000, 0, None) == m.OK      # no-op
    assert A(ctypes.byref(c), 0x1000, 0x1000, 0x1000, 0x1000, -1, None) == m.ERR_INVALID_ARG
    assert A(ctypes.byref(c), 0x1001, 0x1000, 0x1000, 0x1000, 4, None) == m.ERR_INVALID_ARG  # misaligned
    assert A(ctypes.byref(c), 0x1000, None, 0x1000, 0x1000, 4, None) == m.ERR_INVALID_ARG
    c2 = _cache(m, pages=0x10010)                                                        # pool not 256-B aligned
    assert A(ctypes.byref(c2), 0x1000, 0x1000, 0x1000, 0x1000, 4, None) == m.ERR_INVALID_ARG
    c3 = _cache(m)
    c3.layout.d_c = 256
    assert A(ctypes.byref(c3), 0x1000, 0x1000, 0x1000, 0x1000, 4, None) == m.ERR_UNSUPPORTED
    c4 = _cache(m)
    c4.layout.n_recent = 0
    assert A(ctypes.byref(c4), 0x1000, 0x1000, 0x1000, 0x1000, 4, None) == m.ERR_UNSUPPORTED
    assert "n_recent" in L.mla_lowbit_last_error().decode()
    c4.layout.n_recent = (1 << 24) + 1
    assert A(ctypes.byref(c4), 0x1000, 0x1000, 0x1000, 0x1000, 4, None) == m.ERR_UNSUPPORTED
    c4.layout.n_recent = 1 << 20  # a long all-bf16 window is a supported layout
    assert m.page_bytes(c4.layout) == 20736


def test_decode_validation(m):
    L = m.lib
    Dd = L.mla_lowbit_decode
    c = _cache(m)
    ws = m.decode_workspace_bytes(c.layout, 2, 16, 4096)
    assert ws > 0
    args = lambda **k: dict(dict(q=0x1000, slot=0x2000, lens=0x3000, batch=2, heads=16, maxlen=4096, scale=0.07,
                                 out=0x4000, lse=0x5000, ws=0x100000, wsb=ws), **k)

    def call(cache=c, **k):
        a = args(**k)
        return Dd(ctypes.byref(cache) if cache is not None else None, a["q"], a["slot"], a["lens"], a["batch"],
                  a["heads"], a["maxlen"], a["scale"], a["out"], a["lse"], a["ws"], a["wsb"], None)

    assert call(cache=None) == m.ERR_INVALID_ARG
    assert call(heads=24) == m.ERR_UNSUPPORTED
    assert call(heads=8) == m.ERR_UNSUPPORTED
    assert call(heads=0) == m.ERR_UNSUPPORTED
    # 96 heads (six 16-head groups) are supported: the check gets as far as the workspace size
    assert call(heads=96) == m.ERR_WORKSPACE
    assert call(wsb=ws - 1) == m.ERR_WORKSPACE
    assert "workspace" in L.mla_lowbit_last_error().decode()
    assert call(ws=0x100010) == m.ERR_INVALID_ARG          # misaligned workspace
    assert call(q=0x1002) == m.ERR_INVALID_ARG
    assert call(out=None) == m.ERR_INVALID_ARG
    assert call(scale=float("nan")) == m.ERR_INVALID_ARG
    assert call(batch=-1) == m.ERR_INVALID_ARG
    assert call(batch=0) == m.OK                            # nothing to do
    c2 = _cache(m)
    c2.layout.bits_r = 2
    assert call(cache=c2) == m.ERR_UNSUPPORTED


def test_decode_multi_validation(m):
    L = m.lib
    c = _cache(m)  # n_recent = 128
    ws = m.decode_workspace_bytes(c.layout, 2, 4 * 16, 4096)
    assert ws > 0

    def call(q_len, heads=16, wsb=ws):
        return L.mla_lowbit_decode_multi(ctypes.byref(c), 0x1000, 0x2000, 0x3000, 2, q_len, heads, 4096, 0.07,
                                         0x4000, 0x5000, 0x100000, wsb, None)

    assert call(0) == m.ERR_UNSUPPORTED
    assert "q_len" in L.mla_lowbit_last_error().decode()
    assert call(130) == m.ERR_UNSUPPORTED                 # beyond n_recent + 1
    assert call(4, heads=8) == m.ERR_UNSUPPORTED          # 32 rows, but 8 heads a query
    assert call(4, heads=24) == m.ERR_UNSUPPORTED
    assert call(4, wsb=ws - 1) == m.ERR_WORKSPACE         # the workspace covers q_len * heads rows
    assert call(129, wsb=0) == m.ERR_WORKSPACE            # n_recent + 1 queries are allowed


def test_workspace_monotone(m):
    lay = m.make_layout(4)
    for h in (16, 32, 48, 64, 96, 128, 256):
        a = m.decode_workspace_bytes(lay, 4, h, 1024)
        b = m.decode_workspace_bytes(lay, 4, h, 131072)
        assert 0 < a <= b
    for h in (0, 8, 40):
        assert m.decode_workspace_bytes(lay, 4, h, 1024) == 0


def test_status_strings(m):
    for s in range(5):
        assert m.lib.mla_lowbit_status_string(s)
    assert m.lib.mla_lowbit_status_string(99) == b"unknown status"
