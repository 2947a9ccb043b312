"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, and every invalid-argument path returns its status code before any
HIP call (so no call here can reach a kernel launch)."""

import ctypes
import os
import re

import pytest

from paged_kv_cache_03_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedkv.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH),
                                reason="libpagedkv.so not built")

A16 = 0x10000        # 16- and 256-byte aligned fake device address (never dereferenced)
A4 = 0x10004         # only 4-byte aligned
MIS = 0x10002        # not even 4-byte aligned


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = header_functions()
    assert len(names) >= 9
    for name in names:
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, f"{name} has no ctypes signature"
    assert set(_lib.SIGNATURES) == set(names)


def test_status_strings(lib):
    for code in range(8):
        assert lib.pkv_status_string(code)
    assert lib.pkv_status_string(99) == b"unknown status"
    assert lib.pkv_abi_version() == _lib.ABI_VERSION


def decode(lib, **kw):
    args = dict(q=A16, k=A16, v=A16, tables=A16, maxb=128, ctx=A16, maxctx=2048, B=4, H=32,
                D=128, bs=16, nb=1024, scale=0.088, out=A16, ws=A16, wsb=1 << 30, part=0,
                flags=0)
    args.update(kw)
    return lib.pkv_pa_decode_ex(args["q"], args["k"], args["v"], args["tables"], args["maxb"],
                                args["ctx"], args["maxctx"], args["B"], args["H"], args["D"],
                                args["bs"], args["nb"], args["scale"], args["out"], args["ws"],
                                args["wsb"], args["part"], args["flags"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(bs=8), _lib.ERR_UNSUPPORTED),
    (dict(D=96), _lib.ERR_BAD_SHAPE),
    (dict(H=0), _lib.ERR_BAD_SHAPE),
    (dict(B=-1), _lib.ERR_BAD_SHAPE),
    (dict(maxctx=-5), _lib.ERR_BAD_SHAPE),
    (dict(maxb=127), _lib.ERR_BAD_SHAPE),          # 127*16 < 2048
    (dict(nb=0), _lib.ERR_BAD_SHAPE),
    (dict(part=24), _lib.ERR_BAD_SHAPE),
    (dict(part=1024), _lib.ERR_BAD_SHAPE),
    (dict(flags=2), _lib.ERR_BAD_SHAPE),           # unknown flag bit
    (dict(q=None), _lib.ERR_NULL_PTR),
    (dict(k=None), _lib.ERR_NULL_PTR),
    (dict(tables=None), _lib.ERR_NULL_PTR),
    (dict(out=None), _lib.ERR_NULL_PTR),
    (dict(q=A4), _lib.ERR_MISALIGNED),
    (dict(v=A4), _lib.ERR_MISALIGNED),
    (dict(ctx=MIS), _lib.ERR_MISALIGNED),
    (dict(ws=None), _lib.ERR_NULL_PTR),
    (dict(ws=A16 + 16), _lib.ERR_MISALIGNED),
    (dict(wsb=64), _lib.ERR_WORKSPACE_TOO_SMALL),
])
def test_decode_rejects_bad_arguments(lib, kw, code):
    assert decode(lib, **kw) == code


def test_decode_empty_batch_is_a_no_op(lib):
    assert decode(lib, B=0, q=None, k=None, v=None, tables=None, ctx=None, out=None) == _lib.OK


def test_plain_decode_entry_checks_too(lib):
    assert lib.pkv_pa_decode(A16, A16, A16, A16, 128, A16, 2048, 4, 32, 128, 8, 1024, 0.1, A16,
                             A16, 1 << 30, None) == _lib.ERR_UNSUPPORTED


def decode_append(lib, **kw):
    args = dict(q=A16, kn=A16, vn=A16, k=A16, v=A16, tables=A16, maxb=128, ctx=A16, maxctx=2048,
                B=4, H=32, D=128, bs=16, nb=1024, scale=0.088, out=A16, ws=A16, wsb=1 << 30,
                flags=0)
    args.update(kw)
    return lib.pkv_pa_decode_append(args["q"], args["kn"], args["vn"], args["k"], args["v"],
                                    args["tables"], args["maxb"], args["ctx"], args["maxctx"],
                                    args["B"], args["H"], args["D"], args["bs"], args["nb"],
                                    args["scale"], args["out"], args["ws"], args["wsb"],
                                    args["flags"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(bs=8), _lib.ERR_UNSUPPORTED),
    (dict(D=96), _lib.ERR_BAD_SHAPE),
    (dict(maxb=127), _lib.ERR_BAD_SHAPE),
    (dict(flags=2), _lib.ERR_BAD_SHAPE),
    (dict(kn=None), _lib.ERR_NULL_PTR),
    (dict(vn=None), _lib.ERR_NULL_PTR),
    (dict(kn=None, B=0), _lib.ERR_NULL_PTR),       # the new rows are always required
    (dict(q=None), _lib.ERR_NULL_PTR),
    (dict(kn=A4), _lib.ERR_MISALIGNED),
    (dict(vn=A4), _lib.ERR_MISALIGNED),
    (dict(ws=None), _lib.ERR_NULL_PTR),
    (dict(wsb=64), _lib.ERR_WORKSPACE_TOO_SMALL),
    (dict(B=5000, maxctx=1 << 16, maxb=4096), _lib.ERR_UNSUPPORTED),   # flat staging too big
])
def test_decode_append_rejects_bad_arguments(lib, kw, code):
    assert decode_append(lib, **kw) == code


def test_decode_append_empty_batch_is_a_no_op(lib):
    assert decode_append(lib, B=0, q=None, k=None, v=None, tables=None, ctx=None,
                         out=None) == _lib.OK


def test_workspace_size(lib):
    B, H, D, ctx = 200, 32, 128, 2048
    # default plan: the flat strategy, whose partial pieces do not grow with
    # the context (at most two per workgroup range and head)
    assert lib.pkv_pa_decode_default_partition(B, H, D, ctx) == 0
    flat = lib.pkv_pa_decode_workspace_size(B, H, D, ctx)
    assert 0 < flat < (16 << 20)
    assert lib.pkv_pa_decode_workspace_size(B, H, D, 1024) == flat
    # ... and only the per-sequence offsets (one int32 each) grow with the batch
    assert flat - lib.pkv_pa_decode_workspace_size(10, H, D, ctx) == (B - 10) * 4
    # explicit partitions: one (m, l, acc[D]) slot per (sequence, head, partition)
    part = 256
    np_ = -(-ctx // part)
    rows = B * H * np_
    ml = -(-rows * 8 // 256) * 256
    assert lib.pkv_pa_decode_workspace_size_ex(B, H, D, ctx, part) == ml + rows * D * 4
    # a context that fits one partition needs no workspace
    assert lib.pkv_pa_decode_workspace_size_ex(B, H, D, 256, 256) == 0
    assert lib.pkv_pa_decode_workspace_size_ex(B, H, D, 257, 256) > 0
    assert lib.pkv_pa_decode_workspace_size_ex(B, H, D, 100, 24) == 0     # invalid partition
    assert lib.pkv_pa_decode_workspace_size(B, H, 96, 100) == 0           # invalid D
    # very large batches fall back to partitions, split finer when short
    big = lib.pkv_pa_decode_default_partition(8192, H, D, ctx)
    assert big % 16 == 0 and 16 <= big <= 512
    assert lib.pkv_pa_decode_workspace_size(8192, H, D, ctx) == \
        lib.pkv_pa_decode_workspace_size_ex(8192, H, D, ctx, big)


def append(lib, **kw):
    args = dict(k=A16, v=A16, slots=A16, T=8, kp=A16, vp=A16, nb=64, H=32, D=128, bs=16)
    args.update(kw)
    return lib.pkv_kv_append(args["k"], args["v"], args["slots"], args["T"], args["kp"],
                             args["vp"], args["nb"], args["H"], args["D"], args["bs"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(bs=32), _lib.ERR_UNSUPPORTED),
    (dict(D=80), _lib.ERR_BAD_SHAPE),
    (dict(T=-1), _lib.ERR_BAD_SHAPE),
    (dict(nb=0), _lib.ERR_BAD_SHAPE),
    (dict(slots=None), _lib.ERR_NULL_PTR),
    (dict(kp=None), _lib.ERR_NULL_PTR),
    (dict(k=A4), _lib.ERR_MISALIGNED),
    (dict(vp=A4), _lib.ERR_MISALIGNED),
    (dict(slots=MIS), _lib.ERR_MISALIGNED),
])
def test_append_rejects_bad_arguments(lib, kw, code):
    assert append(lib, **kw) == code


def test_append_nothing_is_a_no_op(lib):
    assert append(lib, T=0, k=None, v=None, slots=None) == _lib.OK


def cow(lib, pools_k, pools_v, layers=2, pairs=A16, n=3, nb=64, bb=131072):
    K = (ctypes.c_void_p * max(1, len(pools_k)))(*pools_k)
    V = (ctypes.c_void_p * max(1, len(pools_v)))(*pools_v)
    return lib.pkv_cow_copy_blocks(K, V, layers, pairs, n, nb, bb, None)


def test_cow_rejects_bad_arguments(lib):
    ok = [A16, A16 + 4096]
    assert cow(lib, ok, ok, bb=100) == _lib.ERR_BAD_SHAPE
    assert cow(lib, ok, ok, layers=0) == _lib.ERR_BAD_SHAPE
    assert cow(lib, ok, ok, nb=0) == _lib.ERR_BAD_SHAPE
    assert cow(lib, ok, ok, n=-1) == _lib.ERR_BAD_SHAPE
    assert cow(lib, ok, ok, pairs=None) == _lib.ERR_NULL_PTR
    assert cow(lib, [A16, None], ok) == _lib.ERR_NULL_PTR
    assert cow(lib, ok, [A16, A4]) == _lib.ERR_MISALIGNED
    assert cow(lib, ok, ok, pairs=MIS) == _lib.ERR_MISALIGNED
    assert cow(lib, ok, ok, n=0, pairs=None) == _lib.OK
    assert lib.pkv_cow_copy_blocks(None, None, 2, A16, 3, 64, 131072, None) == _lib.ERR_NULL_PTR


def test_probe_rejects_bad_arguments(lib):
    assert lib.pkv_hbm_read_probe(A16, 0, A16, 64, None) == _lib.ERR_BAD_SHAPE
    assert lib.pkv_hbm_read_probe(A16, 24, A16, 64, None) == _lib.ERR_BAD_SHAPE
    assert lib.pkv_hbm_read_probe(A16, 32, A16, 0, None) == _lib.ERR_BAD_SHAPE
    assert lib.pkv_hbm_read_probe(None, 32, A16, 64, None) == _lib.ERR_NULL_PTR
    assert lib.pkv_hbm_read_probe(A4, 32, A16, 64, None) == _lib.ERR_MISALIGNED
    c = lib.pkv_hbm_copy_probe
    assert c(A16, A16, 0, 64, None) == _lib.ERR_BAD_SHAPE
    assert c(A16, A16, 24, 64, None) == _lib.ERR_BAD_SHAPE
    assert c(A16, A16, 32, 0, None) == _lib.ERR_BAD_SHAPE
    assert c(None, A16, 32, 64, None) == _lib.ERR_NULL_PTR
    assert c(A16, None, 32, 64, None) == _lib.ERR_NULL_PTR
    assert c(A16, A4, 32, 64, None) == _lib.ERR_MISALIGNED
    g = lib.pkv_hbm_gather_probe
    assert g(A16, 0, A16, 4096, A16, 64, None) == _lib.ERR_BAD_SHAPE
    assert g(A16, 8192, A16, 3072, A16, 64, None) == _lib.ERR_BAD_SHAPE    # not a power of two
    assert g(A16, 8192, A16, 512, A16, 64, None) == _lib.ERR_BAD_SHAPE     # below 1 KiB
    assert g(A16, 8192, A16, 2 << 20, A16, 64, None) == _lib.ERR_BAD_SHAPE  # above 1 MiB
    assert g(A16, 6144, A16, 4096, A16, 64, None) == _lib.ERR_BAD_SHAPE    # not a whole chunk
    assert g(A16, 8192, A16, 4096, A16, 0, None) == _lib.ERR_BAD_SHAPE
    assert g(A16, 8192, None, 4096, A16, 64, None) == _lib.ERR_NULL_PTR
    assert g(A4, 8192, A16, 4096, A16, 64, None) == _lib.ERR_MISALIGNED
    s = lib.pkv_lds_read_probe
    assert s(A16, A16, 0, 4, 1, 0, None) == _lib.ERR_BAD_SHAPE
    assert s(A16, A16, 8, 0, 1, 0, None) == _lib.ERR_BAD_SHAPE
    assert s(A16, A16, 8, 17, 1, 0, None) == _lib.ERR_BAD_SHAPE
    assert s(A16, A16, 8, 4, 0, 0, None) == _lib.ERR_BAD_SHAPE
    assert s(A16, A16, 8, 4, 1, 2, None) == _lib.ERR_BAD_SHAPE
    assert s(None, A16, 8, 4, 1, 0, None) == _lib.ERR_NULL_PTR
    assert s(A16, None, 8, 4, 1, 0, None) == _lib.ERR_NULL_PTR
    assert s(A4, A16, 8, 4, 1, 0, None) == _lib.ERR_MISALIGNED


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(_lib.LibraryMissing):
        _lib.load_library(str(tmp_path / "libpagedkv.so"))


def test_grouped_rejects_bad_arguments(lib):
    g = lib.pkv_pa_decode_grouped

    def call(**kw):
        a = dict(q=A16, k=A16, v=A16, tables=A16, mb=128, lens=A16, max_ctx=2048, offs=A16,
                 shared=A16, G=3, gs=16, B=8, H=32, D=128, bs=16, NB=64, scale=0.1, out=A16,
                 ws=A16, ws_bytes=1 << 40, flags=0)
        a.update(kw)
        return g(a["q"], a["k"], a["v"], a["tables"], a["mb"], a["lens"], a["max_ctx"], a["offs"],
                 a["shared"], a["G"], a["gs"], a["B"], a["H"], a["D"], a["bs"], a["NB"],
                 a["scale"], a["out"], a["ws"], a["ws_bytes"], a["flags"], None)

    assert call(bs=32) == _lib.ERR_UNSUPPORTED
    assert call(flags=2) == _lib.ERR_BAD_SHAPE
    assert call(gs=0) == _lib.ERR_BAD_SHAPE
    assert call(gs=17) == _lib.ERR_BAD_SHAPE
    assert call(G=-1) == _lib.ERR_BAD_SHAPE
    assert call(G=1 << 20) == _lib.ERR_BAD_SHAPE            # prefix table does not fit LDS
    assert call(D=96) == _lib.ERR_BAD_SHAPE
    assert call(mb=100) == _lib.ERR_BAD_SHAPE               # table narrower than the context
    assert call(B=0, q=None) == _lib.OK                      # empty batch: nothing to do
    assert call(q=None) == _lib.ERR_NULL_PTR
    assert call(offs=None) == _lib.ERR_NULL_PTR
    assert call(shared=None) == _lib.ERR_NULL_PTR
    assert call(ws=None) == _lib.ERR_NULL_PTR
    assert call(out=A4) == _lib.ERR_MISALIGNED
    assert call(ws=A16 + 16) == _lib.ERR_MISALIGNED
    need = lib.pkv_pa_decode_grouped_workspace_size(8, 32, 128, 2048, 3, 16)
    assert need > 0
    assert call(ws_bytes=need - 1) == _lib.ERR_WORKSPACE_TOO_SMALL


def test_grouped_workspace_size():
    lib = _lib.load_library()
    ws = lib.pkv_pa_decode_grouped_workspace_size
    assert ws(0, 32, 128, 2048, 0, 16) == 0
    assert ws(8, 32, 128, 2048, 3, 0) == 0 and ws(8, 32, 128, 2048, -1, 16) == 0
    # grows with every dimension it depends on: the batch (per-sequence
    # map), members (partials per range), groups (offsets), and the context
    # only once the ranges' LDS staging forces more ranges; the partials
    # scale with heads x ranges, and the ranges per head group shrink as the
    # head groups grow (the grid stays at its target)
    base = ws(200, 32, 128, 2048, 50, 4)
    for bigger in (ws(400, 32, 128, 2048, 50, 4), ws(200, 32, 128, 2048, 50, 8),
                   ws(200, 32, 128, 2048, 150, 4), ws(4000, 32, 128, 1 << 16, 50, 4)):
        assert bigger > base
    assert ws(200, 64, 128, 2048, 50, 4) == base
    assert ws(200, 32, 128, 4096, 50, 4) == base
    assert ws(200, 32, 64, 2048, 50, 4) < base
    # the context lengths and group offsets are staged on chip next to at
    # least one position of range staging: B + num_groups is at most 11,259
    assert ws(8, 32, 128, 2048, 11251, 16) > 0
    assert ws(8, 32, 128, 2048, 11252, 16) == 0
    assert ws(5000, 32, 128, 2048, 6259, 16) > 0
    assert ws(5000, 32, 128, 2048, 6260, 16) == 0


def test_prefill_rejects_bad_arguments(lib):
    f = lib.pkv_pa_prefill

    def call(**kw):
        a = dict(q=A16, k=A16, v=A16, tables=A16, mb=128, lens=A16, max_ctx=2048, qs=A16, T=512,
                 B=8, H=32, D=128, bs=16, NB=64, scale=0.1, out=A16, flags=0)
        a.update(kw)
        return f(a["q"], a["k"], a["v"], a["tables"], a["mb"], a["lens"], a["max_ctx"], a["qs"],
                 a["T"], a["B"], a["H"], a["D"], a["bs"], a["NB"], a["scale"], a["out"],
                 a["flags"], None)

    assert call(bs=8) == _lib.ERR_UNSUPPORTED
    assert call(flags=1) == _lib.ERR_BAD_SHAPE
    # heads per item: codes 1..4 (1, 2, 4, 8 heads) in bits 8..15; an
    # accepted code passes the flag check (the null q then fails)
    for code in (1, 2, 3, 4):
        assert call(flags=code << 8, q=None) == _lib.ERR_NULL_PTR
    assert call(flags=5 << 8) == _lib.ERR_BAD_SHAPE
    assert call(flags=(1 << 8) | 1) == _lib.ERR_BAD_SHAPE
    assert call(flags=1 << 16) == _lib.ERR_BAD_SHAPE
    assert call(T=-1) == _lib.ERR_BAD_SHAPE
    assert call(D=80) == _lib.ERR_BAD_SHAPE
    assert call(mb=64) == _lib.ERR_BAD_SHAPE                 # table narrower than the context
    assert call(B=9000) == _lib.ERR_BAD_SHAPE                # staging would not fit in LDS
    assert call(T=0, q=None) == _lib.OK and call(B=0, q=None) == _lib.OK
    assert call(qs=None) == _lib.ERR_NULL_PTR
    assert call(out=None) == _lib.ERR_NULL_PTR
    assert call(q=A4) == _lib.ERR_MISALIGNED
    assert call(qs=A16 + 2) == _lib.ERR_MISALIGNED


def test_prefill_append_rejects_bad_arguments(lib):
    f = lib.pkv_pa_prefill_append

    def call(**kw):
        a = dict(q=A16, kn=A16, vn=A16, k=A16, v=A16, tables=A16, mb=128, lens=A16, max_ctx=2048,
                 qs=A16, T=512, B=8, H=32, D=128, bs=16, NB=64, scale=0.1, out=A16, flags=0)
        a.update(kw)
        return f(a["q"], a["kn"], a["vn"], a["k"], a["v"], a["tables"], a["mb"], a["lens"],
                 a["max_ctx"], a["qs"], a["T"], a["B"], a["H"], a["D"], a["bs"], a["NB"],
                 a["scale"], a["out"], a["flags"], None)

    # the checks of pkv_pa_prefill, then the new rows'
    assert call(bs=8) == _lib.ERR_UNSUPPORTED
    assert call(flags=1) == _lib.ERR_BAD_SHAPE
    assert call(D=80) == _lib.ERR_BAD_SHAPE
    assert call(mb=64) == _lib.ERR_BAD_SHAPE
    assert call(T=0, kn=None) == _lib.OK and call(B=0, vn=None) == _lib.OK
    assert call(kn=None) == _lib.ERR_NULL_PTR
    assert call(vn=None) == _lib.ERR_NULL_PTR
    assert call(k=None) == _lib.ERR_NULL_PTR
    assert call(kn=A4) == _lib.ERR_MISALIGNED
    assert call(vn=A16 + 8) == _lib.ERR_MISALIGNED


def test_contig_decode_rejects_bad_arguments(lib):
    f = lib.pkv_contig_decode

    def call(**kw):
        a = dict(q=A16, k=A16, v=A16, L=2048, lens=A16, cap=A16, max_ctx=2048, B=8, H=32, D=128,
                 scale=0.1, out=A16, ws=A16, ws_bytes=1 << 40, flags=0)
        a.update(kw)
        return f(a["q"], a["k"], a["v"], a["L"], a["lens"], a["cap"], a["max_ctx"], a["B"],
                 a["H"], a["D"], a["scale"], a["out"], a["ws"], a["ws_bytes"], a["flags"], None)

    assert call(flags=1) == _lib.ERR_BAD_SHAPE
    assert call(L=1000) == _lib.ERR_BAD_SHAPE              # not a multiple of 16
    assert call(L=1024) == _lib.ERR_BAD_SHAPE              # shorter than the longest context
    assert call(D=32) == _lib.ERR_BAD_SHAPE
    assert call(B=0, q=None) == _lib.OK
    assert call(k=None) == _lib.ERR_NULL_PTR
    assert call(ws=None) == _lib.ERR_NULL_PTR
    assert call(cap=MIS) == _lib.ERR_MISALIGNED
    need = lib.pkv_contig_decode_workspace_size(8, 32, 128, 2048)
    assert need > 0 and call(ws_bytes=need - 1) == _lib.ERR_WORKSPACE_TOO_SMALL


def test_vkv_rejects_bad_arguments(lib):
    h = ctypes.c_void_p()
    create = lib.pkv_vkv_create
    assert create(8, 2048, 1, 32, 128, 2 << 20, None) == _lib.ERR_NULL_PTR
    assert create(8, 2000, 1, 32, 128, 2 << 20, ctypes.byref(h)) == _lib.ERR_BAD_SHAPE
    assert create(8, 2048, 1, 32, 96, 2 << 20, ctypes.byref(h)) == _lib.ERR_BAD_SHAPE
    assert create(8, 2048, 0, 32, 128, 2 << 20, ctypes.byref(h)) == _lib.ERR_BAD_SHAPE
    assert create(8, 2048, 1, 32, 128, 0, ctypes.byref(h)) == _lib.ERR_BAD_SHAPE
    assert create(8, 2048, 1, 32, 128, 3 << 20, ctypes.byref(h)) == _lib.ERR_BAD_SHAPE  # no divisor
    assert not h.value
    assert lib.pkv_vkv_grow(None, 0, 16) == _lib.ERR_NULL_PTR
    assert lib.pkv_vkv_release(None, 0) == _lib.ERR_NULL_PTR
    assert lib.pkv_vkv_destroy(None) == _lib.OK
    k, v = ctypes.c_void_p(), ctypes.c_void_p()
    assert lib.pkv_vkv_buffers(None, 0, ctypes.byref(k), ctypes.byref(v)) == _lib.ERR_NULL_PTR
    assert lib.pkv_vkv_capacity(None) is None
    info = _lib.VkvInfo()
    assert lib.pkv_vkv_stats(None, ctypes.byref(info)) == _lib.ERR_NULL_PTR
    assert lib.pkv_vkv_append(None, 0, A16, A16, A16, A16, 4, None) == _lib.ERR_NULL_PTR


def test_noalloc_rejects_shapes_beyond_its_scratch(lib):
    """The allocation-free decode step checks its fixed scratch size before
    any HIP call: 4,096 heads need 8,192 partial rows of 128 floats, more
    than PKV_NOALLOC_SCRATCH_BYTES; other errors as for the workspace call."""
    assert lib.pkv_pa_decode_workspace_size(1, 4096, 128, 16) > _lib.NOALLOC_SCRATCH_BYTES
    assert lib.pkv_pa_decode_workspace_size(200, 32, 128, 2048) <= _lib.NOALLOC_SCRATCH_BYTES

    def call(**kw):
        a = dict(q=A16, kn=A16, vn=A16, k=A16, v=A16, tables=A16, maxb=128, ctx=A16,
                 maxctx=2048, B=4, H=32, D=128, bs=16, nb=1024, out=A16, flags=0)
        a.update(kw)
        return lib.pkv_pa_decode_append_noalloc(
            a["q"], a["kn"], a["vn"], a["k"], a["v"], a["tables"], a["maxb"], a["ctx"],
            a["maxctx"], a["B"], a["H"], a["D"], a["bs"], a["nb"], 0.088, a["out"], a["flags"],
            None)

    assert call(B=1, H=4096, maxctx=16, maxb=1) == _lib.ERR_SCRATCH_TOO_SMALL
    assert call(kn=None) == _lib.ERR_NULL_PTR
    assert call(out=None) == _lib.ERR_NULL_PTR
    assert call(bs=32) == _lib.ERR_UNSUPPORTED
    assert call(D=96) == _lib.ERR_BAD_SHAPE
    assert call(q=MIS) == _lib.ERR_MISALIGNED
    assert call(flags=4) == _lib.ERR_BAD_SHAPE
    assert call(B=0) == _lib.OK
