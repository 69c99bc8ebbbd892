"""GPU parity of fa2_fwd_split (key splits with a merge) against the fp64
oracle (needs an MI355X).

The split path (fa2_fwd_split; fa2_fwd_kv_split over INT8 and FP8 caches)
computes the same attention as the unsplit calls through a different
reduction order (partial softmaxes over key ranges, merged by
their logsumexps), so it is compared with the oracle at the 16-bit path's
tolerances, and with fa2_fwd_ext only loosely.  Outputs start as NaN, so an
unwritten row cannot pass; split counts cover the library's own choice, a
few explicit counts, and more splits than key tiles (empty parts)."""
import math

import numpy as np
import pytest
import torch

import oracle
from flashattention_forward_tile_amd import fa2
from flashattention_forward_tile_amd.workloads import (bits, make_inputs, make_inputs_kv_fp8,
                                                       make_inputs_kv_int8)
from parity import assert_parity

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def announce(*what):
    print("CASE", *what, flush=True)


def run_split(q, k, v, scale, causal, splits, workspace=None):
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o = torch.full_like(qd, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
    fa2.fwd_split(qd, kd, vd, scale=scale, causal=causal, splits=splits, workspace=workspace,
                  out=o, lse=lse)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def check(q, k, v, dtype, scale, causal, splits, tag):
    o, lse = run_split(q, k, v, scale, causal, splits)
    o_ref, lse_ref = oracle.attention(bits(q), bits(k), bits(v), dtype, scale, causal=causal)
    og, lg = o.double().numpy(), lse.double().numpy()
    seen = np.isfinite(lse_ref)
    assert np.all(og[~seen] == 0.0) and np.all(lg[~seen] == -np.inf), tag
    assert_parity(og[seen], lg[seen], o_ref[seen], lse_ref[seen], tag, lse_abs=1e-3)
    return o, lse


@pytest.mark.parametrize("splits", [0, 2, 5, 16])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_decode_rows(d, dtype, causal, splits):
    """One query row per head, four query heads per K/V head, a long ragged
    key sequence (not a multiple of any tile)."""
    announce("split decode", d, dtype, causal, splits)
    q, k, v = make_inputs(2, 8, 1, d, dtype, seed=d + splits, Hkv=2, Nk=5000)
    check(q, k, v, dtype, 1.0 / math.sqrt(d), causal, splits,
          "split decode d=%d %s causal=%d splits=%d" % (d, dtype, causal, splits))


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,splits", [
    (1, 4, 1, 37, 3000, 0), (2, 8, 2, 64, 4096, 3), (1, 2, 2, 130, 2049, 7),
    (1, 4, 4, 200, 100, 8),      # more splits than key tiles: empty parts
    (1, 2, 1, 300, 200, 4),      # causal: rows before Nq - Nk see no key
    (3, 6, 3, 5, 33, 2), (1, 1, 1, 1, 1, 2), (1, 4, 2, 1, 70000, 128),
    (128, 4, 2, 1, 2048, 0)])    # items fill the GPU: the library's floor of two parts
@pytest.mark.parametrize("causal", [False, True])
def test_chunks(B, Hq, Hkv, Nq, Nk, splits, causal):
    announce("split chunk", B, Hq, Hkv, Nq, Nk, splits, causal)
    q, k, v = make_inputs(B, Hq, Nq, 128, "bf16", seed=Nq + Nk, Hkv=Hkv, Nk=Nk)
    check(q, k, v, "bf16", 1.0 / math.sqrt(128), causal, splits,
          "split B=%d Hq=%d Hkv=%d Nq=%d Nk=%d splits=%d causal=%d" % (
              B, Hq, Hkv, Nq, Nk, splits, causal))


@pytest.mark.parametrize("scale", [0.0, -0.3, 2.5])
def test_scales(scale):
    announce("split scale", scale)
    q, k, v = make_inputs(1, 8, 3, 128, "fp16", seed=9, Hkv=2, Nk=3000)
    check(q, k, v, "fp16", scale, True, 6, "split scale=%g" % scale)


def test_no_keys():
    announce("split Nk=0")
    q, _, _ = make_inputs(1, 4, 3, 128, "bf16", seed=2)
    empty = torch.empty((1, 2, 0, 128), dtype=torch.bfloat16)
    for causal in (False, True):
        o, lse = run_split(q, empty, empty.clone(), None, causal, 4)
        assert torch.all(o == 0) and torch.all(lse == -float("inf"))


def test_matches_unsplit_and_is_deterministic():
    """Against fa2_fwd_ext on the same inputs: the same result up to the
    reordered rounding; two split calls: bit for bit."""
    announce("split vs unsplit")
    q, k, v = make_inputs(2, 16, 4, 128, "bf16", seed=5, Hkv=4, Nk=20000)
    o1, l1 = run_split(q, k, v, None, True, 0)
    o2, l2 = run_split(q, k, v, None, True, 0)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o3, l3 = fa2.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True)
    torch.cuda.synchronize()
    assert (o1.float() - o3.cpu().float()).abs().max().item() <= 2e-2
    assert (l1 - l3.cpu()).abs().max().item() <= 1e-3


def test_workspace_reused_with_smaller_calls():
    """One workspace for a large call, then a smaller one: every result is
    the oracle's (the workspace holds nothing between calls)."""
    announce("split workspace reuse")
    ws = torch.empty(fa2.split_workspace_bytes(2, 8, 2, 16, 9000, 128, False, fa2.BF16, 12),
                     dtype=torch.uint8, device=DEV)
    for (B, Nq, Nk, splits) in ((2, 16, 9000, 12), (1, 3, 700, 3)):
        q, k, v = make_inputs(B, 8, Nq, 128, "bf16", seed=Nk, Hkv=2, Nk=Nk)
        o, lse = run_split(q, k, v, None, False, splits, workspace=ws)
        o_ref, lse_ref = oracle.attention(bits(q), bits(k), bits(v), "bf16",
                                          1.0 / math.sqrt(128))
        assert_parity(o.double().numpy(), lse.double().numpy(), o_ref, lse_ref,
                      "split reuse Nk=%d" % Nk)


def test_chosen_split_count_uses_the_compute_units():
    """splits = 0 on a long decode: the workspace query reports the bytes of
    the count the library picks (one workgroup per compute unit)."""
    announce("split choice")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n = fa2.split_workspace_bytes(4, 32, 8, 1, 32768, 128, True, fa2.BF16, 0)
    per_split = 4 * 32 * 1 * (128 + 1) * 4
    assert n % per_split == 0
    items = 4 * 8 * 1  # one 128-row query tile per K/V head
    assert n // per_split == min(-(-cus // items), 32768 // 32 // 8, 128)
    # quantized caches: two workgroups per compute unit
    for cache in (fa2.CACHE_INT8, fa2.CACHE_FP8):
        n = fa2.split_workspace_bytes(4, 32, 8, 1, 32768, 128, True, fa2.BF16, 0, cache)
        assert n // per_split == min(-(-2 * cus // items), 32768 // 32 // 8, 128)
    # Items of a few rows each that already fill the GPU: at least two parts
    # from 64 key tiles on, none below that or for rows filling most of a tile.
    for B, Nk in ((64, 4096), (2 * cus, 2048)):
        for cache in (0, fa2.CACHE_INT8, fa2.CACHE_FP8):
            n = fa2.split_workspace_bytes(B, 32, 8, 1, Nk, 128, True, fa2.BF16, 0, cache)
            parts = n // (B * 32 * 1 * (128 + 1) * 4)
            assert parts == max(2, -(-(2 if cache else 1) * cus // (B * 8))), (B, Nk, cache, parts)
    assert fa2.split_workspace_bytes(2 * cus, 32, 8, 1, 1024, 128, True, fa2.BF16, 0) == 0
    assert fa2.split_workspace_bytes(2 * cus, 32, 8, 32, 4096, 128, True, fa2.BF16, 0) == 0


QUANTIZED = {"int8": (fa2.CACHE_INT8, make_inputs_kv_int8, "attention_kv_int8"),
             "fp8": (fa2.CACHE_FP8, make_inputs_kv_fp8, "attention_kv_fp8")}


@pytest.mark.parametrize("splits", [0, 3, 16])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("fmt", ["int8", "fp8"])
def test_quantized_cache_decode(fmt, d, dtype, causal, splits):
    """Decode rows over an INT8 / FP8 cache with key splits, against the
    oracle's quantized functions (each part quantizes the query row as the
    unsplit call does) and against the unsplit call."""
    announce("split", fmt, d, dtype, causal, splits)
    cache, make, attn = QUANTIZED[fmt]
    q, kq, ks, vq, vs = make(2, 8, 2, 2, 5000, d, dtype, seed=splits + 17 + d)
    q[0, 0, 1] = 0  # a zero row: codes 0, sq 0
    dev = [t.to(DEV) for t in (q, kq, ks, vq, vs)]
    o = torch.full_like(dev[0], float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
    fa2.fwd_kv_split(*dev, cache, causal=causal, splits=splits, out=o, lse=lse)
    unsplit = fa2.fwd_kv_int8 if fmt == "int8" else fa2.fwd_kv_fp8
    o1, l1 = unsplit(*dev, causal=causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = getattr(oracle, attn)(bits(q), kq.numpy(), ks.numpy(), vq.numpy(),
                                           vs.numpy(), dtype, 1.0 / math.sqrt(d),
                                           causal=causal)
    tag = "split %s d=%d %s causal=%d splits=%d" % (fmt, d, dtype, causal, splits)
    assert_parity(o.cpu().double().numpy(), lse.cpu().double().numpy(), o_ref, lse_ref, tag,
                  lse_abs=1e-3)
    assert (o.float() - o1.float()).abs().max().item() <= 2e-2, tag
    assert (lse - l1).abs().max().item() <= 1e-3, tag


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("fmt", ["bf16", "fp16", "int8", "fp8"])
def test_unsplit_calls_on_few_rows(fmt, d, causal):
    """Calls without splits whose items hold at most 128 query rows (here 4
    query heads on each K/V head, one row each) run on the key-split
    kernels as one part writing O itself (16-bit inputs once the K/V heads
    number at least the compute units, as here; quantized caches always):
    against the oracle, and bit for bit the same through fa2_fwd_split with
    splits = 1."""
    announce("one part", fmt, d, causal)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wide = fmt in ("bf16", "fp16")
    B, Hq, Hkv, Nq, Nk = (cus // 2 + 1, 8, 2, 1, 1500) if wide else (3, 8, 2, 1, 3000)
    scale = 1.0 / math.sqrt(d)
    if wide:
        q, k, v = make_inputs(B, Hq, Nq, d, fmt, seed=d + causal, Hkv=Hkv, Nk=Nk)
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
        o, lse = fa2.fwd(qd, kd, vd, causal=causal)
        o1 = torch.full_like(qd, float("nan"))
        l1 = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
        fa2.fwd_split(qd, kd, vd, causal=causal, splits=1, out=o1, lse=l1)
        o_ref, lse_ref = oracle.attention(bits(q), bits(k), bits(v), fmt, scale, causal=causal)
    else:
        cache, make, attn = QUANTIZED[fmt]
        q, kq, ks, vq, vs = make(B, Hq, Hkv, Nq, Nk, d, "bf16", seed=d + causal)
        dev = [t.to(DEV) for t in (q, kq, ks, vq, vs)]
        unsplit = fa2.fwd_kv_int8 if fmt == "int8" else fa2.fwd_kv_fp8
        o, lse = unsplit(*dev, causal=causal)
        o1 = torch.full_like(dev[0], float("nan"))
        l1 = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
        fa2.fwd_kv_split(*dev, cache, causal=causal, splits=1, out=o1, lse=l1)
        o_ref, lse_ref = getattr(oracle, attn)(bits(q), kq.numpy(), ks.numpy(), vq.numpy(),
                                               vs.numpy(), "bf16", scale, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o, o1) and torch.equal(lse, l1)
    assert_parity(o.cpu().double().numpy(), lse.cpu().double().numpy(), o_ref, lse_ref,
                  "one part %s d=%d causal=%d" % (fmt, d, causal), lse_abs=1e-3)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("fmt", ["bf16", "int8", "fp8"])
def test_one_part_matches_the_other_kernels_bit_for_bit(fmt, d):
    """The one-part route computes each row exactly as the kernels it
    replaces: the first batch entries of a call large enough to take one
    route equal, bit for bit, a call of just those entries, which takes the
    other (16-bit: one query row per head, routed only once B*Hkv reaches
    the compute units; 8-bit caches at d = 64 and 128: 200 rows per K/V
    head, routed only while the 256-row grid is smaller than the compute
    units)."""
    if fmt != "bf16" and d == 256:
        pytest.skip("the 8-bit caches keep one shape at d = 256")
    announce("one part vs other kernels", fmt, d)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    B, Hq, Hkv, Nk = cus // 2 + 1, 8, 2, 1500
    Nq = 1 if fmt == "bf16" else 50
    if fmt == "bf16":
        q, k, v = (t.to(DEV) for t in make_inputs(B, Hq, Nq, d, "bf16", seed=d, Hkv=Hkv, Nk=Nk))
        o, lse = fa2.fwd(q, k, v, causal=True)
        o3, l3 = fa2.fwd(q[:3].contiguous(), k[:3].contiguous(), v[:3].contiguous(), causal=True)
    else:
        cache, make, _ = QUANTIZED[fmt]
        dev = [t.to(DEV) for t in make(B, Hq, Hkv, Nq, Nk, d, "bf16", seed=d)]
        unsplit = fa2.fwd_kv_int8 if fmt == "int8" else fa2.fwd_kv_fp8
        o, lse = unsplit(*dev, causal=True)
        o3, l3 = unsplit(*[t[:3].contiguous() for t in dev], causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o[:3], o3) and torch.equal(lse[:3], l3)
