"""Race check (needs an MI355X): the production library against its
race-check build, bit for bit.

libfa2_sync.so is the same kernel source built with FA2_SYNC_CHECK: every
iteration waits for all of its HBM -> LDS loads and synchronises the
workgroup right where they are issued, instead of letting them land during
the next iteration as the key/value ring does.  The arithmetic and its order
are the same, so any difference in O or LSE would mean the production
pipeline read a tile before it landed or overwrote one still in use.  Each
case covers one kernel family: persistent, one item per workgroup, causal,
short keys, each head dimension, grouped heads, the INT8 and FP8 caches, and
key splits.
"""
import math

import pytest
import torch

from flashattention_forward_tile_amd import _build, fa2
from flashattention_forward_tile_amd.workloads import (WORKLOADS, make_inputs,
                                                       make_inputs_kv_fp8, make_inputs_kv_int8,
                                                       workload_inputs)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
_sync = None


def sync_lib():
    global _sync
    if _sync is None:
        _sync = fa2.load(_build.LIB_SYNC)
    return _sync


def announce(*what):
    print("CASE", *what, flush=True)


def run_both(q, k, v, Hkv, scale, causal):
    """(o, lse) from the production and the race-check library."""
    B, Hq, Nq, d = q.shape
    Nk = k.shape[2]
    outs = []
    for handle in (fa2.lib(), sync_lib()):
        o = torch.full_like(q, float("nan"))
        lse = torch.full((B, Hq, Nq), float("nan"), device=DEV)
        code = handle.fa2_fwd_ext(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                  lse.data_ptr(), B, Hq, Hkv, Nq, Nk, d, float(scale),
                                  int(causal), fa2._DTYPE[q.dtype], 0)
        assert code == 0, fa2.strerror(code)
        torch.cuda.synchronize()
        outs.append((o.cpu(), lse.cpu()))
    return outs


def assert_same(outs, tag):
    (o1, l1), (o2, l2) = outs
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), tag
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), tag


@pytest.mark.parametrize("name", ["headline", "causal", "sweep_n512", "gqa", "gqa_chunk",
                                  "kv_cache", "stress"])
def test_workloads_match_race_check_build(name):
    w = WORKLOADS[name]
    announce(w)
    q, k, v = (t.to(DEV) for t in workload_inputs(w, seed=1))
    assert_same(run_both(q, k, v, w.kv_heads, w.scale, w.causal), name)


@pytest.mark.parametrize("d,H", [(64, 8), (256, 4)])
@pytest.mark.parametrize("causal", [False, True])
def test_head_dims_match_race_check_build(d, H, causal):
    announce("d", d, "causal", causal)
    q, k, v = (t.to(DEV) for t in make_inputs(2, H, 2000, d, "bf16", "normal", 3))
    assert_same(run_both(q, k, v, H, 1.0 / math.sqrt(d), causal), "d=%d" % d)


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,dtype,scale", [
    (2, 64, 64, 1000, 1130, "bf16", None),     # persistent, ragged tiles
    (4, 32, 8, 1100, 2048, "fp16", -0.15),     # persistent, grouped heads, negative scale
    (2, 128, 16, 520, 1152, "bf16", 0.0),      # persistent, zero scale
    (16, 16, 16, 512, 500, "fp16", None),      # persistent, short keys (causal: four waves)
    (2, 4, 2, 300, 777, "bf16", None),         # one item per workgroup, Nq != Nk
])
def test_shapes_match_race_check_build(B, Hq, Hkv, Nq, Nk, dtype, scale):
    announce("shape", B, Hq, Hkv, Nq, Nk, dtype, scale)
    q, k, v = (t.to(DEV) for t in make_inputs(B, Hq, Nq, 128, dtype, "normal", 5, Hkv, Nk))
    s = 1.0 / math.sqrt(128) if scale is None else scale
    for causal in (False, True):
        assert_same(run_both(q, k, v, Hkv, s, causal), "causal=%d" % causal)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("fmt", ["int8", "fp8"])
def test_quantized_cache_matches_race_check_build(fmt, causal):
    announce(fmt, causal)
    make = make_inputs_kv_int8 if fmt == "int8" else make_inputs_kv_fp8
    q, kq, ks, vq, vs = (t.to(DEV) for t in make(2, 16, 4, 1500, 3000, 128, "bf16", 7))
    outs = []
    for handle in (fa2.lib(), sync_lib()):
        o = torch.full_like(q, float("nan"))
        lse = torch.full(q.shape[:3], float("nan"), device=DEV)
        call = handle.fa2_fwd_kv_int8 if fmt == "int8" else handle.fa2_fwd_kv_fp8
        code = call(q.data_ptr(), kq.data_ptr(), ks.data_ptr(), vq.data_ptr(), vs.data_ptr(),
                    o.data_ptr(), lse.data_ptr(), 2, 16, 4, 1500, 3000, 128,
                    1.0 / math.sqrt(128), int(causal), fa2.BF16, 0)
        assert code == 0, fa2.strerror(code)
        torch.cuda.synchronize()
        outs.append((o.cpu(), lse.cpu()))
    assert_same(outs, "%s causal=%d" % (fmt, causal))


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_key_splits_match_race_check_build(d, causal):
    announce("split", d, causal)
    B, Hq, Hkv, Nq, Nk, splits = 2, 8, 2, 3, 6000, 7
    q, k, v = (t.to(DEV) for t in make_inputs(B, Hq, Nq, d, "fp16", "normal", 8, Hkv, Nk))
    nbytes = fa2.split_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, causal, fa2.FP16, splits)
    outs = []
    for handle in (fa2.lib(), sync_lib()):
        ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
        o = torch.full_like(q, float("nan"))
        lse = torch.full((B, Hq, Nq), float("nan"), device=DEV)
        code = handle.fa2_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                    lse.data_ptr(), B, Hq, Hkv, Nq, Nk, d, 1.0 / math.sqrt(d),
                                    int(causal), fa2.FP16, splits, ws.data_ptr(), nbytes, 0)
        assert code == 0, fa2.strerror(code)
        torch.cuda.synchronize()
        outs.append((o.cpu(), lse.cpu()))
    assert_same(outs, "split d=%d causal=%d" % (d, causal))


@pytest.mark.parametrize("cache", [fa2.CACHE_INT8, fa2.CACHE_FP8])
def test_quantized_key_splits_match_race_check_build(cache):
    announce("split cache", cache)
    B, Hq, Hkv, Nq, Nk, splits = 2, 8, 2, 3, 6000, 7
    make = make_inputs_kv_int8 if cache == fa2.CACHE_INT8 else make_inputs_kv_fp8
    q, kq, ks, vq, vs = (t.to(DEV) for t in make(B, Hq, Hkv, Nq, Nk, 128, "bf16", 9))
    nbytes = fa2.split_workspace_bytes(B, Hq, Hkv, Nq, Nk, 128, True, fa2.BF16, splits, cache)
    outs = []
    for handle in (fa2.lib(), sync_lib()):
        ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
        o = torch.full_like(q, float("nan"))
        lse = torch.full((B, Hq, Nq), float("nan"), device=DEV)
        code = handle.fa2_fwd_kv_split(q.data_ptr(), kq.data_ptr(), ks.data_ptr(), vq.data_ptr(),
                                       vs.data_ptr(), o.data_ptr(), lse.data_ptr(), B, Hq, Hkv,
                                       Nq, Nk, 128, 1.0 / math.sqrt(128), 1, fa2.BF16, cache,
                                       splits, ws.data_ptr(), nbytes, 0)
        assert code == 0, fa2.strerror(code)
        torch.cuda.synchronize()
        outs.append((o.cpu(), lse.cpu()))
    assert_same(outs, "split cache %d" % cache)
