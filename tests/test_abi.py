"""C ABI checks that need no GPU: the library loads, exports what include/fa.h
declares, and rejects every invalid call before any HIP call.

Only invalid calls are made here: fake device addresses never pass validation,
so nothing is ever launched.
"""
import ctypes
import os
import re

import pytest

from exact_tiled_attention_21_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000          # 16-byte aligned, never dereferenced
MIS = 0x10008           # 8-byte aligned only


def declared_functions():
    text = open(os.path.join(ROOT, "include", "fa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in range(12):
        s = lib.fa_status_str(code).decode()
        assert s and s != "unknown status"
    assert lib.fa_status_str(99).decode() == "unknown status"


def fwd(lib, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, Nq=8, Nk=8, Hq=2, Hkv=1, d=64,
        causal=0, scale=0.125, dtype=0):
    return lib.fa_fwd(q, k, v, o, lse, B, Nq, Nk, Hq, Hkv, d, causal, scale, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(o=None), 1),
    (dict(B=0), 2), (dict(Nq=0), 2), (dict(Nk=-1), 2), (dict(Hq=0), 2), (dict(Hkv=0), 2),
    (dict(B=1 << 20, Nq=1 << 20, Hq=64, d=256), 2),
    (dict(Hq=1 << 15, Hkv=1 << 15, d=256), 2), (dict(Hq=1 << 17, Hkv=1, d=64), 2),
    (dict(B=1 << 10, Nq=1 << 17, Hq=16, Hkv=16, d=32), 2),   # 2^24 workgroups of 256 threads
    (dict(Hq=3, Hkv=2), 3),
    (dict(d=48), 4), (dict(d=16), 4), (dict(d=512), 4), (dict(d=0), 4),
    (dict(dtype=2), 5), (dict(dtype=-1), 5),
    (dict(scale=float("inf")), 10), (dict(scale=float("nan")), 10),
    (dict(q=MIS), 9), (dict(o=MIS), 9), (dict(lse=FAKE + 2), 9),
])
def test_fwd_rejects_invalid_arguments(lib, kw, status):
    assert fwd(lib, **kw) == status


def test_fwd_checks_nullptr_before_shape(lib):
    assert fwd(lib, q=None, B=0) == 1


def test_workspace_size(lib):
    ws = lib.fa_decode_workspace_bytes
    # [4S][B][Hq][Nq][d] fp32 partial outputs, then [4S][B][Hq][Nq] fp32 LSEs, each padded to 256 B
    rows = 4 * 16 * 8 * 32 * 1
    assert ws(8, 1, 32, 128, 16) == rows * 128 * 4 + ((rows * 4 + 255) // 256) * 256
    assert ws(8, 1, 32, 128, 0) == 0
    assert ws(8, 1, 32, 100, 4) == 0
    assert ws(0, 1, 32, 128, 4) == 0
    assert ws(1, 1, 1, 32, _lib.FA_MAX_SPLITS + 1) == 0


def dec(lib, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=2, Nq=1, Nk=64, Hq=4, Hkv=2, d=128, S=4,
        causal=0, scale=0.1, dtype=1, ws=FAKE, wsb=None):
    if wsb is None:
        wsb = lib.fa_decode_workspace_bytes(B, Nq, Hq, d, S) if S >= 1 else 0
    return lib.fa_decode_splitkv(q, k, v, o, lse, B, Nq, Nk, Hq, Hkv, d, S, causal, scale, dtype,
                                 ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(ws=None), 1), (dict(o=None), 1),
    (dict(Nk=0), 2), (dict(Hq=5, Hkv=2), 3), (dict(d=80), 4), (dict(dtype=7), 5),
    (dict(S=0), 6), (dict(S=_lib.FA_MAX_SPLITS + 1), 6),
    (dict(wsb=16), 7), (dict(ws=MIS), 9), (dict(k=MIS), 9), (dict(scale=float("-inf")), 10),
    (dict(Nk=1 << 20, Hkv=8, Hq=8, d=256), 2), (dict(Nk=1, Hq=1 << 15, Hkv=1 << 15, d=256), 2),
    (dict(B=1 << 20, Hq=512, Hkv=512, d=32, S=1), 2),   # combine grid of 2^24 workgroups
])
def test_decode_rejects_invalid_arguments(lib, kw, status):
    assert dec(lib, **kw) == status


def dec_noalloc(lib, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=2, Nq=1, Nk=64, Hq=4, Hkv=2, d=128, S=4,
                causal=0, scale=0.1, dtype=1):
    return lib.fa_decode_splitkv_noalloc(q, k, v, o, lse, B, Nq, Nk, Hq, Hkv, d, S, causal, scale, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(o=None), 1),
    (dict(Nk=0), 2), (dict(Hq=5, Hkv=2), 3), (dict(d=80), 4), (dict(dtype=7), 5),
    (dict(S=0), 6), (dict(S=_lib.FA_MAX_SPLITS + 1), 6),
    (dict(k=MIS), 9), (dict(scale=float("nan")), 10),
    (dict(Nk=1 << 20, Hkv=8, Hq=8, d=256), 2),
    # partials of 16 x 8 x 32 x 64 rows of 256 floats: 256 MiB, beyond the fixed scratch
    (dict(B=8, Nq=64, Hq=32, Hkv=32, d=256, S=16), 11),
])
def test_decode_noalloc_rejects_invalid_arguments(lib, kw, status):
    """The entry point that allocates nothing validates like fa_decode_splitkv and
    refuses a call whose partials exceed the fixed scratch, before any HIP call."""
    assert dec_noalloc(lib, **kw) == status


def test_python_layer_fails_loudly_without_library(tmp_path):
    with pytest.raises(FileNotFoundError):
        _lib.load(str(tmp_path / "libfa.so"))


def test_no_oracle_on_product_path():
    pkg = os.path.join(ROOT, "exact_tiled_attention_21_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), f
                assert "attention_f64" not in text, f


def dec_paged(lib, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, sl=FAKE, o=FAKE, lse=FAKE, B=2, Nq=1, Hq=4, Hkv=2,
              d=128, num_pages=8, page_size=64, max_pages=4, S=4, causal=0, scale=0.1, dtype=1,
              ws=FAKE, wsb=None):
    if wsb is None:
        wsb = lib.fa_decode_workspace_bytes(B, Nq, Hq, d, S) if S >= 1 else 0
    return lib.fa_decode_splitkv_paged(q, k, v, bt, sl, o, lse, B, Nq, Hq, Hkv, d, num_pages,
                                       page_size, max_pages, S, causal, scale, dtype, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(bt=None), 1), (dict(sl=None), 1), (dict(q=None), 1), (dict(ws=None), 1),
    (dict(page_size=48), 2), (dict(page_size=16), 2), (dict(page_size=0), 2), (dict(num_pages=0), 2),
    (dict(max_pages=0), 2), (dict(page_size=1 << 20, max_pages=1 << 12), 2),
    (dict(Hq=5), 3), (dict(d=80), 4), (dict(dtype=3), 5), (dict(S=0), 6), (dict(wsb=8), 7),
    (dict(bt=FAKE + 2), 9), (dict(sl=FAKE + 1), 9), (dict(k=MIS), 9),
    (dict(scale=float("nan")), 10),
])
def test_paged_decode_rejects_invalid_arguments(lib, kw, status):
    assert dec_paged(lib, **kw) == status


def fwd_varlen(lib, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, cq=FAKE, ck=FAKE, B=2, max_q=8, tq=16, tk=16,
               Hq=2, Hkv=1, d=64, causal=0, scale=0.125, dtype=0):
    return lib.fa_fwd_varlen(q, k, v, o, lse, cq, ck, B, max_q, tq, tk, Hq, Hkv, d, causal, scale, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(cq=None), 1), (dict(ck=None), 1), (dict(q=None), 1),
    (dict(B=0), 2), (dict(max_q=0), 2), (dict(tq=0), 2), (dict(tk=0), 2),
    (dict(Hq=3, Hkv=2), 3), (dict(d=40), 4), (dict(dtype=9), 5),
    (dict(cq=FAKE + 2), 9), (dict(ck=FAKE + 1), 9), (dict(o=MIS), 9), (dict(scale=float("inf")), 10),
])
def test_fwd_varlen_rejects_invalid_arguments(lib, kw, status):
    assert fwd_varlen(lib, **kw) == status


@pytest.mark.parametrize("wl,wr,status", [(-2, 0, 2), (0, -2, 2), (-1, -1, 1)])
def test_fwd_window_rejects_invalid_windows(lib, wl, wr, status):
    q = None if status == 1 else FAKE   # a valid window reaches the pointer check
    assert lib.fa_fwd_window(q, FAKE, FAKE, FAKE, FAKE, 1, 8, 8, 2, 1, 64, wl, wr, 0, 0.125, 0, None) == status


def test_bwd_workspace_size(lib):
    ws = lib.fa_bwd_workspace_bytes
    # two float32 arrays [B][Hq][Nq rounded up to 32], each padded to 256 bytes
    assert ws(2, 100, 3) == 2 * (((2 * 3 * 128 * 4) + 255) // 256 * 256)
    assert ws(1, 1, 1) == 2 * 256
    assert ws(0, 8, 1) == 0 and ws(1, 0, 1) == 0 and ws(1, 8, 0) == 0


def bwd(lib, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, do=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, B=1, Nq=8, Nk=8,
        Hq=2, Hkv=1, d=64, causal=0, scale=0.125, dtype=1, ws=FAKE, wsb=None):
    if wsb is None:
        wsb = lib.fa_bwd_workspace_bytes(B, Nq, Hq) if min(B, Nq, Hq) >= 1 else 0
    return lib.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, B, Nq, Nk, Hq, Hkv, d, causal, scale, dtype, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(o=None), 1), (dict(lse=None), 1), (dict(do=None), 1), (dict(dq=None), 1),
    (dict(dk=None), 1), (dict(dv=None), 1), (dict(ws=None), 1),
    (dict(B=0), 2), (dict(Nk=0), 2), (dict(Hq=1 << 15, Hkv=1 << 15, d=256), 2),
    (dict(B=1 << 12, Nq=1 << 11, Hq=16, Hkv=16), 2),   # statistics kernel grid of 2^24 workgroups
    (dict(Hq=3, Hkv=2), 3), (dict(d=80), 4), (dict(dtype=4), 5),
    (dict(wsb=16), 7), (dict(do=MIS), 9), (dict(dq=MIS), 9), (dict(dk=MIS), 9), (dict(dv=MIS), 9),
    (dict(ws=MIS), 9), (dict(lse=FAKE + 2), 9), (dict(scale=float("nan")), 10),
])
def test_bwd_rejects_invalid_arguments(lib, kw, status):
    assert bwd(lib, **kw) == status


@pytest.mark.parametrize("wl,wr,status", [(-2, 0, 2), (0, -2, 2), (-1, -1, 1)])
def test_bwd_window_rejects_invalid_windows(lib, wl, wr, status):
    q = None if status == 1 else FAKE   # a valid window reaches the pointer check
    wsb = lib.fa_bwd_workspace_bytes(1, 8, 2)
    assert lib.fa_bwd_window(q, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 8, 2, 1, 64, wl, wr, 0,
                             0.125, 1, FAKE, wsb, None) == status


def bwd_varlen(lib, q=FAKE, cq=FAKE, ck=FAKE, B=2, mq=8, mk=8, tq=16, tk=16, Hq=2, Hkv=1, d=64, ws=FAKE,
               wsb=None, do=FAKE):
    if wsb is None:
        wsb = lib.fa_bwd_workspace_bytes(max(B, 1), max(mq, 1), Hq)
    return lib.fa_bwd_varlen(q, FAKE, FAKE, FAKE, FAKE, do, FAKE, FAKE, FAKE, cq, ck, B, mq, mk, tq, tk, Hq, Hkv,
                             d, 0, 0.125, 1, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(cq=None), 1), (dict(ck=None), 1), (dict(q=None), 1), (dict(do=None), 1), (dict(ws=None), 1),
    (dict(B=0), 2), (dict(mq=0), 2), (dict(mk=0), 2), (dict(tq=0), 2), (dict(Hq=3, Hkv=2), 3), (dict(d=40), 4),
    (dict(cq=FAKE + 2), 9), (dict(ck=FAKE + 1), 9), (dict(wsb=8), 7),
])
def test_bwd_varlen_rejects_invalid_arguments(lib, kw, status):
    assert bwd_varlen(lib, **kw) == status
