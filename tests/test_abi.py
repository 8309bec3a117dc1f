"""The C-ABI library loads, exports every declared symbol and rejects bad arguments.

CPU only: every call below fails validation on the host and returns before any HIP
call (the pointers are fake, aligned, non-null integers that are never
dereferenced). No call here ever reaches a kernel launch.
"""
import ctypes
import math
import os
import re

import pytest

from kv_cache_fa_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvfa.h")

INVALID, UNSUPPORTED = _lib.FA_ERR_INVALID, _lib.FA_ERR_UNSUPPORTED
P = 1 << 20          # a fake, 16-byte aligned device address (never dereferenced)


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"^(?:int|size_t|const char\*)\s+(\w+)\(", text, flags=re.M)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libkvfa.so not built (run __graft_entry__.build())")
    return _lib.lib()


def test_header_declares_the_expected_entry_points():
    assert set(declared_functions()) == {
        "fa_fwd", "fa_fwd_fp32", "fa_decode_paged", "fa_decode_paged_workspace_size",
        "fa_decode_paged_split_tokens", "fa_fwd_paged", "fa_kv_append", "fa_fwd_window", "fa_fwd_two_pass", "fa_decode_paged_fp8", "fa_bwd", "fa_bwd_workspace_size", "fa_status_string",
        "fa_decode_paged_noalloc"}


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, name


def test_status_strings(lib):
    for st in (0, -1, -2, -3, -4, 7):
        assert _lib.fa_status_string(st)
    assert _lib.fa_status_string(-4).startswith("FA_ERR_SCRATCH")
    assert _lib.fa_status_string(-1).startswith("FA_ERR_INVALID")


def _fwd(lib, fn="fa_fwd", q=P, k=P, v=P, o=P, lse=P, B=1, H=8, Hkv=8, Nq=64, Nk=64, d=128,
         causal=1, scale=0.125):
    return getattr(lib, fn)(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, causal, scale, None)


def test_two_pass_requires_lse(lib):
    assert lib.fa_fwd_two_pass(P, P, P, P, None, 1, 8, 8, 64, 64, 128, 1, 0.125, None) == INVALID
    assert lib.fa_fwd_two_pass(P, P, P, P, P, 1, 8, 8, 64, 64, 96, 1, 0.125, None) == UNSUPPORTED


@pytest.mark.parametrize("fn", ["fa_fwd", "fa_fwd_fp32", "fa_fwd_two_pass"])
@pytest.mark.parametrize("kw,want", [
    (dict(q=None), INVALID), (dict(o=None), INVALID), (dict(k=P + 8), INVALID),
    (dict(lse=P + 2), INVALID),
    (dict(B=0), INVALID), (dict(H=0), INVALID), (dict(Nq=0), INVALID), (dict(Nk=-3), INVALID),
    (dict(H=8, Hkv=3), INVALID), (dict(Hkv=0), INVALID),
    (dict(causal=1, Nq=65, Nk=64), INVALID),
    (dict(scale=0.0), INVALID), (dict(scale=-1.0), INVALID), (dict(scale=math.inf), INVALID),
    (dict(scale=math.nan), INVALID),
    (dict(d=96), UNSUPPORTED), (dict(d=256), UNSUPPORTED), (dict(d=32), UNSUPPORTED),
    (dict(Nk=1 << 23, causal=0), UNSUPPORTED),
])
def test_prefill_validation(lib, fn, kw, want):
    assert _fwd(lib, fn, **kw) == want


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), INVALID), (dict(k=P + 8), INVALID), (dict(Nq=65, Nk=64), INVALID),
    (dict(wl=-2), INVALID), (dict(wr=-5), INVALID), (dict(H=8, Hkv=3), INVALID),
    (dict(scale=0.0), INVALID), (dict(d=96), UNSUPPORTED),
])
def test_window_validation(lib, kw, want):
    a = dict(q=P, k=P, v=P, o=P, lse=None, B=1, H=8, Hkv=8, Nq=64, Nk=64, d=128, wl=16, wr=0,
             scale=0.125)
    a.update(kw)
    assert lib.fa_fwd_window(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Hkv"],
                             a["Nq"], a["Nk"], a["d"], a["wl"], a["wr"], a["scale"], None) == want


def _dec(lib, q=P, kc=P, vc=P, pt=P, sl=P, page_size=16, o=P, lse=None, S=4, H=32, Hkv=8,
         d=128, num_pages=100, max_pages=8, max_seq_len=128, scale=0.09, ws=P, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.fa_decode_paged_workspace_size(S, H, d, max_seq_len, page_size) \
            if page_size == 16 and d in (64, 128) else 1 << 30
    return lib.fa_decode_paged(q, kc, vc, pt, sl, page_size, o, lse, S, H, Hkv, d, num_pages,
                               max_pages, max_seq_len, scale, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), INVALID), (dict(pt=None), INVALID), (dict(sl=None), INVALID),
    (dict(ws=None), INVALID), (dict(kc=P + 4), INVALID), (dict(pt=P + 2), INVALID),
    (dict(S=0), INVALID), (dict(num_pages=0), INVALID), (dict(max_pages=0), INVALID),
    (dict(max_seq_len=0), INVALID), (dict(H=32, Hkv=5), INVALID),
    (dict(max_pages=7, max_seq_len=128), INVALID),
    (dict(scale=0.0), INVALID), (dict(scale=math.nan), INVALID),
    (dict(ws_bytes=16), INVALID),
    (dict(page_size=32, max_pages=4), UNSUPPORTED), (dict(d=80), UNSUPPORTED),
    (dict(H=40, Hkv=2), UNSUPPORTED),   # group of 20 query heads
    (dict(S=65536), UNSUPPORTED),        # one combine row per sequence
    # 8 sequences x 2031586 pages: one page more than 248 x 65535 work-group rows cover
    (dict(S=8, max_seq_len=16 * 2031586, max_pages=2031586), UNSUPPORTED),
])
def test_decode_validation(lib, kw, want):
    assert _dec(lib, **kw) == want


def _fwd_paged(lib, q=P, kc=P, vc=P, pt=P, sl=P, page_size=16, o=P, lse=None, B=2, H=16,
               Hkv=4, Nq=100, d=128, num_pages=64, max_pages=16, max_seq_len=256, causal=1,
               scale=0.09):
    return lib.fa_fwd_paged(q, kc, vc, pt, sl, page_size, o, lse, B, H, Hkv, Nq, d, num_pages,
                            max_pages, max_seq_len, causal, scale, None)


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), INVALID), (dict(kc=None), INVALID), (dict(pt=None), INVALID),
    (dict(sl=None), INVALID), (dict(o=None), INVALID), (dict(vc=P + 8), INVALID),
    (dict(sl=P + 2), INVALID), (dict(lse=P + 1), INVALID),
    (dict(B=0), INVALID), (dict(Nq=0), INVALID), (dict(num_pages=0), INVALID),
    (dict(max_pages=0), INVALID), (dict(H=16, Hkv=3), INVALID),
    (dict(Nq=300, max_seq_len=256), INVALID),            # queries longer than any sequence
    (dict(max_pages=15, max_seq_len=256), INVALID),      # table too short
    (dict(scale=0.0), INVALID), (dict(scale=math.inf), INVALID),
    (dict(page_size=8, max_pages=32), UNSUPPORTED), (dict(d=96), UNSUPPORTED),
])
def test_fwd_paged_validation(lib, kw, want):
    assert _fwd_paged(lib, **kw) == want


def _append(lib, kn=P, vn=P, kc=P, vc=P, pt=P, sp=P, page_size=16, S=4, n_new=8, Hkv=8,
            d=128, num_pages=64, max_pages=16):
    return lib.fa_kv_append(kn, vn, kc, vc, pt, sp, page_size, S, n_new, Hkv, d, num_pages,
                            max_pages, None)


@pytest.mark.parametrize("kw,want", [
    (dict(kn=None), INVALID), (dict(vc=None), INVALID), (dict(pt=None), INVALID),
    (dict(sp=None), INVALID), (dict(kn=P + 4), INVALID), (dict(sp=P + 2), INVALID),
    (dict(S=0), INVALID), (dict(n_new=0), INVALID), (dict(Hkv=0), INVALID),
    (dict(num_pages=0), INVALID), (dict(max_pages=0), INVALID),
    (dict(page_size=32), UNSUPPORTED), (dict(d=80), UNSUPPORTED),
])
def test_kv_append_validation(lib, kw, want):
    assert _append(lib, **kw) == want


def test_decode_fp8_validation(lib):
    ws = lib.fa_decode_paged_workspace_size(4, 32, 128, 128, 16)

    def call(ks=P, vs=P, **kw):
        a = dict(q=P, kc=P, vc=P, pt=P, sl=P, page_size=16, o=P, lse=None, S=4, H=32, Hkv=8,
                 d=128, num_pages=100, max_pages=8, max_seq_len=128, scale=0.09)
        a.update(kw)
        return lib.fa_decode_paged_fp8(a["q"], a["kc"], a["vc"], ks, vs, a["pt"], a["sl"],
                                       a["page_size"], a["o"], a["lse"], a["S"], a["H"],
                                       a["Hkv"], a["d"], a["num_pages"], a["max_pages"],
                                       a["max_seq_len"], a["scale"], P, ws, None)
    assert call(ks=None) == INVALID
    assert call(vs=None) == INVALID
    assert call(ks=P + 2) == INVALID
    assert call(S=0) == INVALID
    assert call(d=96) == UNSUPPORTED
    assert call(H=32, Hkv=5) == INVALID


def test_decode_cache_type_travels_with_scales(lib):
    """The cache's element type is tied to its scale arrays: fa_decode_paged (bf16 cache)
    takes none, fa_decode_paged_fp8 (e4m3 cache) needs both, and a call with only one of
    them is rejected before anything is enqueued."""
    assert len(_lib.SIGNATURES["fa_decode_paged"][1]) == 19
    assert len(_lib.SIGNATURES["fa_decode_paged_fp8"][1]) == 21
    ws = lib.fa_decode_paged_workspace_size(4, 32, 128, 128, 16)
    for ks, vs in ((None, P), (P, None), (None, None)):
        assert lib.fa_decode_paged_fp8(P, P, P, ks, vs, P, P, 16, P, None, 4, 32, 8, 128, 100,
                                       8, 128, 0.09, P, ws, None) == INVALID


def test_decode_noalloc_host_checks(lib):
    """The no-allocation decode checks its arguments like fa_decode_paged and refuses a
    workspace need beyond its static array, all before any HIP call."""
    def call(S=4, H=32, Hkv=8, d=128, max_pages=8, max_seq_len=128, q=P, pt=P, scale=0.09):
        return lib.fa_decode_paged_noalloc(q, P, P, pt, P, 16, P, None, S, H, Hkv, d, 100,
                                           max_pages, max_seq_len, scale, None)
    assert call(q=None) == INVALID
    assert call(pt=P + 2) == INVALID
    assert call(H=32, Hkv=5) == INVALID
    assert call(scale=0.0) == INVALID
    assert call(d=96) == UNSUPPORTED
    S, L = 256, 8192
    assert lib.fa_decode_paged_workspace_size(S, 32, 128, L, 16) > _lib.FA_NOALLOC_SCRATCH_BYTES
    assert call(S=S, max_pages=L // 16, max_seq_len=L) == _lib.FA_ERR_SCRATCH
    # the 64-sequence, 8192-token decode workload fits
    assert lib.fa_decode_paged_workspace_size(64, 32, 128, 8192, 16) <= \
        _lib.FA_NOALLOC_SCRATCH_BYTES


def test_bwd_validation(lib):
    ws = lib.fa_bwd_workspace_size(1, 8, 64)
    assert ws == 8 * 64 * 4
    assert lib.fa_bwd_workspace_size(0, 8, 64) == 0

    def call(**kw):
        a = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, B=1, H=8, Hkv=8, Nq=64,
                 Nk=64, d=128, causal=1, scale=0.125, ws=P, ws_bytes=ws)
        a.update(kw)
        return lib.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"],
                          a["dv"], a["B"], a["H"], a["Hkv"], a["Nq"], a["Nk"], a["d"],
                          a["causal"], a["scale"], a["ws"], a["ws_bytes"], None)
    for kw in (dict(lse=None), dict(do=None), dict(dq=None), dict(dk=P + 8), dict(ws=None),
               dict(ws_bytes=16), dict(Nq=65, Nk=64), dict(H=8, Hkv=3), dict(scale=0.0)):
        assert call(**kw) == INVALID, kw
    assert call(d=96) == UNSUPPORTED


def test_workspace_size(lib):
    f = lib.fa_decode_paged_workspace_size
    assert f(64, 32, 128, 8192, 16) > 0
    assert f(0, 32, 128, 8192, 16) == 0
    assert f(64, 32, 100, 8192, 16) == 0
    assert f(64, 32, 128, 8192, 8) == 0
    assert f(64, 0, 128, 8192, 16) == 0
    # fewest cached tokens a work-group's range holds: 4 pages, or 1/32 of the longest
    # possible sequence, at most 248 pages (62 per wave)
    T = lib.fa_decode_paged_split_tokens(64, 8192, 16)
    assert T == 16 * 16
    slots = -(-8192 // T) + 1  # segments a sequence can be cut into
    # partial results, per sequence its slot count, then the plan: 4 totals and 2 ints per
    # work-group row (at most max(1536, work-groups the longest cache needs, sequences))
    rows = max(1536, -(-(64 * 512) // 248), 64)
    assert f(64, 32, 128, 8192, 16) == (64 * 32 * slots * (128 + 1) * 4 + 64 * 4
                                           + (4 + 2 * rows) * 4)
    assert lib.fa_decode_paged_split_tokens(1, 100, 16) == 4 * 16
    assert lib.fa_decode_paged_split_tokens(1, 131072, 16) == 248 * 16
    assert lib.fa_decode_paged_split_tokens(1, 1 << 30, 16) == 248 * 16


def test_binding_refuses_host_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        _lib.fa_fwd(x, x, x, x, causal=False, scale=0.125)
