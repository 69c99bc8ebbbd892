"""The C-ABI library without a GPU: it loads, exports what include/fa2.h
declares, and rejects bad arguments on the host before any HIP call.

Every fa2_fwd call here fails validation by construction (the pointers are
never dereferenced), so these tests are also safe on a GPU machine."""
import os
import re

import pytest

from flashattention_forward_tile_amd import _build, fa2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa2.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa2_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_build.LIB):
        _build.build()
    return fa2.lib()


def test_header_declares_the_entry_points():
    assert declared_functions() == ["fa2_fwd", "fa2_fwd_ext", "fa2_fwd_kv_fp8",
                                    "fa2_fwd_kv_int8", "fa2_fwd_kv_split", "fa2_fwd_split",
                                    "fa2_fwd_split_noalloc", "fa2_fwd_split_workspace",
                                    "fa2_strerror", "fa2_tile_config"]


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_race_check_build_exports_the_same_symbols():
    """The race-check build the GPU tests compare against loads on the host
    and exports every declared entry point."""
    if not os.path.exists(_build.LIB_SYNC):
        _build.build_sync()
    handle = fa2.load(_build.LIB_SYNC)
    for name in declared_functions():
        assert hasattr(handle, name), name


def test_strerror_covers_every_status(lib):
    texts = set()
    for code in range(0, -12, -1):
        s = fa2.strerror(code)
        assert s and s != "unknown status", code
        texts.add(s)
    assert len(texts) == 12
    assert fa2.strerror(17) == "unknown status"


def test_tile_config(lib):
    for d in (64, 128, 256):
        bq, bk, nw = fa2.tile_config(d, fa2.BF16)
        # 32 query rows per wave (16 on 16x16x32 MFMA at d = 256)
        assert bq == (16 if d == 256 else 32) * nw and bk % 32 == 0 and nw >= 1
    with pytest.raises(fa2.FA2Error) as e:
        fa2.tile_config(96)
    assert e.value.code == fa2.ERR_HEADDIM
    with pytest.raises(fa2.FA2Error) as e:
        fa2.tile_config(128, 7)
    assert e.value.code == fa2.ERR_DTYPE


A = 0x100000      # fake, 16-byte aligned, never dereferenced
GOOD = dict(B=2, H=3, N=100, d=128, scale=0.1, dtype=fa2.BF16)


def call(q=A, k=A + 0x1000000, v=A + 0x2000000, o=A + 0x3000000,
         lse=A + 0x4000000, **kw):
    p = dict(GOOD)
    p.update(kw)
    return fa2.fwd_raw(q, k, v, o, lse, p["B"], p["H"], p["N"], p["d"],
                       p["scale"], p["dtype"], 0)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), fa2.ERR_NULL), (dict(k=0), fa2.ERR_NULL), (dict(v=0), fa2.ERR_NULL),
    (dict(o=0), fa2.ERR_NULL), (dict(lse=0), fa2.ERR_NULL),
    (dict(B=-1), fa2.ERR_SHAPE), (dict(H=-2), fa2.ERR_SHAPE), (dict(N=-5), fa2.ERR_SHAPE),
    (dict(N=1 << 31), fa2.ERR_SHAPE), (dict(B=1 << 40, H=1 << 30), fa2.ERR_SHAPE),
    # 2^26 heads of 32 half-height (128-row) query tiles: one past the 1-D grid
    (dict(B=1 << 22, H=16, N=4096), fa2.ERR_SHAPE),
    # a shape that takes the persistent launch still reports the null pointer
    (dict(B=4, H=16, N=4096, q=0), fa2.ERR_NULL),
    (dict(d=96), fa2.ERR_HEADDIM), (dict(d=0), fa2.ERR_HEADDIM), (dict(d=512), fa2.ERR_HEADDIM),
    (dict(dtype=2), fa2.ERR_DTYPE), (dict(dtype=-1), fa2.ERR_DTYPE),
    (dict(scale=float("nan")), fa2.ERR_SCALE), (dict(scale=float("inf")), fa2.ERR_SCALE),
    # finite in fp32, but scale * log2(e) is not
    (dict(scale=3e38), fa2.ERR_SCALE), (dict(scale=-2.5e38), fa2.ERR_SCALE),
    (dict(q=A + 2), fa2.ERR_ALIGN), (dict(o=A + 0x3000008), fa2.ERR_ALIGN),
    (dict(lse=A + 0x4000002), fa2.ERR_ALIGN),
    (dict(o=A), fa2.ERR_ALIAS), (dict(o=A + 0x1000000 + 4096), fa2.ERR_ALIAS),
    (dict(lse=A + 0x2000000 + 64), fa2.ERR_ALIAS), (dict(lse=A + 0x3000000), fa2.ERR_ALIAS),
])
def test_host_validation(lib, kw, code):
    assert call(**kw) == code


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(N=0)])
def test_empty_problem_is_a_no_op(lib, kw):
    assert call(q=0, k=0, v=0, o=0, lse=0, **kw) == fa2.OK


def test_no_silent_fallback(monkeypatch):
    monkeypatch.setattr(_build, "LIB", "/nonexistent/libfa2.so")
    monkeypatch.setattr(fa2, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        fa2.lib()


EXT = dict(B=2, Hq=4, Hkv=2, Nq=100, Nk=70, d=128, scale=0.1, causal=1, dtype=fa2.BF16)


def call_ext(q=A, k=A + 0x1000000, v=A + 0x2000000, o=A + 0x3000000,
             lse=A + 0x4000000, **kw):
    p = dict(EXT)
    p.update(kw)
    return fa2.fwd_ext_raw(q, k, v, o, lse, p["B"], p["Hq"], p["Hkv"], p["Nq"], p["Nk"],
                           p["d"], p["scale"], p["causal"], p["dtype"], 0)


@pytest.mark.parametrize("kw,code", [
    (dict(causal=2), fa2.ERR_OPTION), (dict(causal=-1), fa2.ERR_OPTION),
    (dict(Hkv=3), fa2.ERR_SHAPE), (dict(Hkv=0), fa2.ERR_SHAPE), (dict(Hkv=-1), fa2.ERR_SHAPE),
    (dict(Nk=-1), fa2.ERR_SHAPE), (dict(Nq=-1), fa2.ERR_SHAPE),
    (dict(Nk=1 << 31), fa2.ERR_SHAPE), (dict(q=0), fa2.ERR_NULL), (dict(k=0), fa2.ERR_NULL),
    # each query head fits 32-bit offsets, but a K/V head's 64 query heads do not
    (dict(Hq=64, Hkv=1, Nq=1 << 18, d=128), fa2.ERR_SHAPE),
    (dict(d=32), fa2.ERR_HEADDIM), (dict(k=A + 0x1000004), fa2.ERR_ALIGN),
    (dict(o=A + 0x2000000 + 512), fa2.ERR_ALIAS), (dict(scale=float("nan")), fa2.ERR_SCALE),
])
def test_ext_host_validation(lib, kw, code):
    assert call_ext(**kw) == code


@pytest.mark.parametrize("kw", [dict(B=0), dict(Hq=0, Hkv=0), dict(Nq=0)])
def test_ext_empty_output_is_a_no_op(lib, kw):
    assert call_ext(q=0, k=0, v=0, o=0, lse=0, **kw) == fa2.OK


# fa2_fwd_kv_int8: q, kq, ks, vq, vs, o, lse (fake pointers, never dereferenced)
I8 = dict(B=2, Hq=4, Hkv=2, Nq=100, Nk=70, d=128, scale=0.1, causal=0, dtype=fa2.BF16)
I8_PTRS = dict(q=A, kq=A + 0x1000000, ks=A + 0x2000000, vq=A + 0x3000000, vs=A + 0x4000000,
               o=A + 0x5000000, lse=A + 0x6000000)


def call_int8(raw=None, **kw):
    p = dict(I8)
    p.update(I8_PTRS)
    p.update(kw)
    raw = raw or fa2.fwd_kv_int8_raw
    return raw(p["q"], p["kq"], p["ks"], p["vq"], p["vs"], p["o"], p["lse"],
               p["B"], p["Hq"], p["Hkv"], p["Nq"], p["Nk"], p["d"], p["scale"],
               p["causal"], p["dtype"], 0)


@pytest.mark.parametrize("kw,code", [
    (dict(d=96), fa2.ERR_HEADDIM), (dict(d=512), fa2.ERR_HEADDIM), (dict(dtype=3), fa2.ERR_DTYPE),
    (dict(causal=2), fa2.ERR_OPTION), (dict(Hkv=3), fa2.ERR_SHAPE), (dict(Nk=-1), fa2.ERR_SHAPE),
    (dict(q=0), fa2.ERR_NULL), (dict(kq=0), fa2.ERR_NULL), (dict(ks=0), fa2.ERR_NULL),
    (dict(vs=0), fa2.ERR_NULL), (dict(ks=0, Nk=0), fa2.ERR_NULL),
    (dict(ks=A + 0x2000004), fa2.ERR_ALIGN), (dict(vq=A + 0x3000008), fa2.ERR_ALIGN),
    (dict(o=A + 0x2000000 + 256), fa2.ERR_ALIAS),   # o over ks
    (dict(lse=A + 0x4000000), fa2.ERR_ALIAS),       # lse over vs
    (dict(scale=float("inf")), fa2.ERR_SCALE),
])
def test_int8_host_validation(lib, kw, code):
    assert call_int8(**kw) == code
    # the FP8 cache shares the INT8 cache's validation
    assert call_int8(raw=fa2.fwd_kv_fp8_raw, **kw) == code


@pytest.mark.parametrize("kw", [dict(B=0), dict(Hq=0, Hkv=0), dict(Nq=0)])
def test_int8_empty_output_is_a_no_op(lib, kw):
    assert call_int8(q=0, kq=0, ks=0, vq=0, vs=0, o=0, lse=0, **kw) == fa2.OK
    assert call_int8(raw=fa2.fwd_kv_fp8_raw, q=0, kq=0, ks=0, vq=0, vs=0, o=0, lse=0, **kw) == fa2.OK


# fa2_fwd_split: as fa2_fwd_ext plus splits, workspace, workspace_bytes
SPLIT = dict(EXT, splits=4)
WS = A + 0x7000000


def call_split(ws=WS, ws_bytes=1 << 24, **kw):
    p = dict(SPLIT)
    ptrs = dict(q=A, k=A + 0x1000000, v=A + 0x2000000, o=A + 0x3000000, lse=A + 0x4000000)
    for name in list(kw):
        if name in ptrs:
            ptrs[name] = kw.pop(name)
    p.update(kw)
    return fa2.fwd_split_raw(ptrs["q"], ptrs["k"], ptrs["v"], ptrs["o"], ptrs["lse"], p["B"],
                             p["Hq"], p["Hkv"], p["Nq"], p["Nk"], p["d"], p["scale"],
                             p["causal"], p["dtype"], p["splits"], ws, ws_bytes, 0)


def split_bytes():
    p = SPLIT
    return fa2.split_workspace_bytes(p["B"], p["Hq"], p["Hkv"], p["Nq"], p["Nk"], p["d"],
                                     p["causal"], p["dtype"], p["splits"])


def test_split_workspace_size(lib):
    # splits * rows of all heads * (d + 1) fp32 values
    assert split_bytes() == 4 * (2 * 4 * 100) * 129 * 4
    assert fa2.split_workspace_bytes(2, 4, 2, 100, 70, 128, True, fa2.BF16, 1) == 0
    assert fa2.split_workspace_bytes(0, 4, 2, 100, 70, 128, True, fa2.BF16, 9) == 0
    for kw, code in [(dict(splits=129), fa2.ERR_OPTION), (dict(splits=-1), fa2.ERR_OPTION),
                     (dict(d=96), fa2.ERR_HEADDIM), (dict(Hkv=3), fa2.ERR_SHAPE),
                     (dict(dtype=2), fa2.ERR_DTYPE), (dict(causal=2), fa2.ERR_OPTION),
                     (dict(cache=3), fa2.ERR_OPTION), (dict(cache=1, d=96), fa2.ERR_HEADDIM)]:
        a = dict(B=2, Hq=4, Hkv=2, Nq=100, Nk=70, d=128, causal=1, dtype=fa2.BF16, splits=4)
        a.update(kw)
        assert lib.fa2_fwd_split_workspace(a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["d"],
                                           a["causal"], a["dtype"], a.get("cache", 0),
                                           a["splits"]) == code, kw
    with pytest.raises(fa2.FA2Error) as e:
        fa2.split_workspace_bytes(2, 4, 2, 100, 70, 96)
    assert e.value.code == fa2.ERR_HEADDIM


@pytest.mark.parametrize("kw,code", [
    (dict(splits=129), fa2.ERR_OPTION), (dict(splits=-3), fa2.ERR_OPTION),
    (dict(ws=0), fa2.ERR_WORKSPACE), (dict(ws_bytes=4 * 800 * 129 * 4 - 1), fa2.ERR_WORKSPACE),
    (dict(ws=WS + 8), fa2.ERR_ALIGN),
    (dict(ws=A + 0x3000000 + 256), fa2.ERR_ALIAS),    # workspace over o
    (dict(ws=A + 0x1000000), fa2.ERR_ALIAS),          # workspace over k
    (dict(ws=A + 0x4000000 - 64), fa2.ERR_ALIAS),     # workspace over lse
    (dict(q=0), fa2.ERR_NULL), (dict(d=32), fa2.ERR_HEADDIM), (dict(causal=3), fa2.ERR_OPTION),
    (dict(scale=float("nan")), fa2.ERR_SCALE), (dict(Hkv=3), fa2.ERR_SHAPE),
])
def test_split_host_validation(lib, kw, code):
    assert call_split(**kw) == code


@pytest.mark.parametrize("kw", [dict(B=0), dict(Hq=0, Hkv=0), dict(Nq=0)])
def test_split_empty_output_is_a_no_op(lib, kw):
    assert call_split(q=0, k=0, v=0, o=0, lse=0, ws=0, ws_bytes=0, **kw) == fa2.OK


def call_kv_split(cache=fa2.CACHE_FP8, splits=4, ws=WS, ws_bytes=1 << 24, **kw):
    p = dict(I8)
    p.update(I8_PTRS)
    p.update(kw)
    return fa2.fwd_kv_split_raw(p["q"], p["kq"], p["ks"], p["vq"], p["vs"], p["o"], p["lse"],
                                p["B"], p["Hq"], p["Hkv"], p["Nq"], p["Nk"], p["d"], p["scale"],
                                p["causal"], p["dtype"], cache, splits, ws, ws_bytes, 0)


@pytest.mark.parametrize("kw,code", [
    (dict(cache=0), fa2.ERR_OPTION), (dict(cache=3), fa2.ERR_OPTION),
    (dict(splits=200), fa2.ERR_OPTION), (dict(d=32), fa2.ERR_HEADDIM),
    (dict(ks=0), fa2.ERR_NULL), (dict(ws=0), fa2.ERR_WORKSPACE),
    (dict(ws_bytes=100), fa2.ERR_WORKSPACE), (dict(ws=WS + 4), fa2.ERR_ALIGN),
    (dict(ws=A + 0x4000000), fa2.ERR_ALIAS),           # workspace over vs
    (dict(cache=fa2.CACHE_INT8, vs=A + 0x4000008), fa2.ERR_ALIGN),
])
def test_kv_split_host_validation(lib, kw, code):
    assert call_kv_split(**kw) == code
