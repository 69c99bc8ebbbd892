"""GPU parity of the persistent-workgroup launches (needs an MI355X).

d = 128 calls with enough (K/V head, query tile) items whose key-tile counts
4 divides (at least 8) run one workgroup per compute unit, each walking
several items with its key/value ring carried from one item into the next;
with the causal mask a workgroup walks pairs of query tiles i and T-1-i of
one K/V head.  Each case here checks that launch against the oracle on sampled rows,
and bit for bit against launches of one K/V head group at a time, which are
too small for persistent workgroups and run one item per workgroup: a row's
arithmetic does not depend on how the items are spread over workgroups.  The
same check covers the non-persistent full-height launch (256-row workgroups),
whose per-group launches, with fewer items than compute units, use 128-row
workgroups.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from flashattention_forward_tile_amd import fa2
from flashattention_forward_tile_amd.workloads import bits
from parity import assert_parity

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
_TD = {"bf16": torch.bfloat16, "fp16": torch.float16}
BLOCK_Q = 256   # query rows per d = 128 workgroup
BLOCK_K = 32    # keys per tile


def announce(*what):
    print("CASE", *what, flush=True)


def rand(shape, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(_TD[dtype])


def persistent(B, Hq, Hkv, Nq, Nk):
    """Whether the call's shape takes the persistent launch on this device."""
    groups = B * Hkv * math.ceil(Hq // Hkv * Nq / BLOCK_Q)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tiles = math.ceil(Nk / BLOCK_K)
    return (tiles >= 8 and tiles % 4 == 0 and groups % 8 == 0
            and cus % 8 == 0 and groups >= 2 * cus)


# (B, Hq, Hkv, Nq, Nk, dtype): 512 items (two per workgroup), 576 (two or
# three), ragged query tiles and a ragged last key tile, grouped heads; short
# key sequences down to the fewest key tiles the persistent loop takes (8).
CASES = [
    (2, 64, 64, 1000, 1130, "bf16"),
    (4, 32, 8, 1100, 2048, "fp16"),
    (2, 128, 16, 520, 1152, "bf16"),
    (16, 16, 16, 512, 500, "fp16"),
    (4, 64, 16, 600, 256, "bf16"),
]


def persistent_causal(B, Hq, Hkv, Nq, Nk):
    """Whether a causal call takes the persistent launch (pairs of query tiles
    of one K/V head per workgroup): no query tile straddles two query heads,
    every tile's key count fills whole ring rotations, and the tiles of each
    K/V head pair up."""
    rows = Hq // Hkv * Nq
    items = B * Hkv * rows // BLOCK_Q
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return (Nq % BLOCK_Q == 0 and Nk % (4 * BLOCK_K) == 0 and Nk >= Nq
            and (rows // BLOCK_Q) % 2 == 0 and items % 16 == 0
            and cus % 8 == 0 and items >= 2 * cus)


# Causal shapes for the persistent launch: the causal headline (1024 items,
# four per workgroup), Nk > Nq with grouped heads, the shortest items (8 and
# 16 key tiles), and grouped heads whose packed query tiles pair across query
# heads (24 tiles per K/V head).
CAUSAL_CASES = [
    (4, 16, 16, 4096, 4096, "bf16"),
    (4, 32, 8, 1024, 1536, "fp16"),
    (16, 16, 16, 512, 512, "bf16"),
    (4, 64, 8, 768, 768, "fp16"),
]


def persistent_d64(B, Hq, Hkv, Nq, Nk):
    """Whether a non-causal d = 64 call takes the persistent launch (256-row
    items, 64-key tiles)."""
    items = B * Hkv * math.ceil(Hq // Hkv * Nq / BLOCK_Q)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tiles = math.ceil(Nk / 64)
    return (tiles >= 8 and tiles % 4 == 0 and items % 8 == 0
            and cus % 8 == 0 and items >= 2 * cus)


# d = 64 shapes for the persistent launch: the d = 64 workload (B4 H16 N4096),
# ragged query tiles and a ragged last key tile with grouped heads, the
# shortest key sequence it takes (8 tiles of 64 keys).
D64_CASES = [
    (4, 16, 16, 4096, 4096, "bf16"),
    (2, 64, 16, 1100, 2000, "fp16"),
    (8, 64, 64, 512, 512, "bf16"),
]


def full_height(B, Hq, Hkv, Nq, Nk):
    """Whether a non-causal call takes one full-height (256-row) workgroup per
    item: not persistent, and at least as many items as compute units."""
    groups = B * Hkv * math.ceil(Hq // Hkv * Nq / BLOCK_Q)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return Nk > 1024 and not persistent(B, Hq, Hkv, Nq, Nk) and groups >= cus


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,dtype", CASES)
@pytest.mark.parametrize("scale_kind", ["default", "negative", "zero"])
def test_persistent_equals_per_group_launches(B, Hq, Hkv, Nq, Nk, dtype, scale_kind):
    announce("persistent", B, Hq, Hkv, Nq, Nk, dtype, scale_kind)
    if not persistent(B, Hq, Hkv, Nq, Nk):
        pytest.skip("shape does not take the persistent launch on this device")
    check_against_groups(B, Hq, Hkv, Nq, Nk, dtype, scale_kind)


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,dtype", CAUSAL_CASES)
@pytest.mark.parametrize("scale_kind", ["default", "negative"])
def test_persistent_causal_equals_per_group_launches(B, Hq, Hkv, Nq, Nk, dtype, scale_kind):
    """Causal calls on persistent workgroups (pairs of query tiles i and T-1-i
    of one K/V head, the ring carried from one item into the next) give bit
    for bit what launches of one K/V head group at a time give (one item per
    workgroup), and match the oracle on sampled rows."""
    announce("persistent causal", B, Hq, Hkv, Nq, Nk, dtype, scale_kind)
    if not persistent_causal(B, Hq, Hkv, Nq, Nk):
        pytest.skip("shape does not take the persistent launch on this device")
    check_against_groups(B, Hq, Hkv, Nq, Nk, dtype, scale_kind, causal=True)


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,dtype", D64_CASES)
@pytest.mark.parametrize("scale_kind", ["default", "negative"])
def test_persistent_d64_equals_per_group_launches(B, Hq, Hkv, Nq, Nk, dtype, scale_kind):
    """d = 64 on persistent eight-wave workgroups gives bit for bit what
    launches of one K/V head group at a time give (four-wave workgroups, one
    item each), and matches the oracle on sampled rows."""
    announce("persistent d64", B, Hq, Hkv, Nq, Nk, dtype, scale_kind)
    if not persistent_d64(B, Hq, Hkv, Nq, Nk):
        pytest.skip("shape does not take the persistent launch on this device")
    check_against_groups(B, Hq, Hkv, Nq, Nk, dtype, scale_kind, d=64)


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,dtype", [(2, 128, 128, 1100, 1100, "bf16"),
                                                  (1, 64, 16, 2000, 2050, "fp16")])
def test_full_height_equals_per_group_launches(B, Hq, Hkv, Nq, Nk, dtype):
    """Key-tile counts that 4 does not divide keep one full-height workgroup
    per item; the per-group launches of the same rows use half-height ones."""
    announce("full height", B, Hq, Hkv, Nq, Nk, dtype)
    if not full_height(B, Hq, Hkv, Nq, Nk):
        pytest.skip("shape does not take full-height workgroups on this device")
    check_against_groups(B, Hq, Hkv, Nq, Nk, dtype, "default")


def check_against_groups(B, Hq, Hkv, Nq, Nk, dtype, scale_kind, causal=False, d=128):
    scale = {"default": 1.0 / math.sqrt(d), "negative": -0.15, "zero": 0.0}[scale_kind]
    seed = B * 1000 + Hq + Nk
    q = rand((B, Hq, Nq, d), dtype, seed).to(DEV)
    k = rand((B, Hkv, Nk, d), dtype, seed + 1).to(DEV)
    v = rand((B, Hkv, Nk, d), dtype, seed + 2).to(DEV)
    o, lse = fa2.fwd(q, k, v, scale=scale, causal=causal)
    torch.cuda.synchronize()
    G = Hq // Hkv
    for b in range(B):
        for g in range(Hkv):
            qs = q[b:b + 1, g * G:(g + 1) * G].contiguous()
            o1, l1 = fa2.fwd(qs, k[b:b + 1, g:g + 1].contiguous(), v[b:b + 1, g:g + 1].contiguous(),
                             scale=scale, causal=causal)
            torch.cuda.synchronize()
            assert torch.equal(o[b:b + 1, g * G:(g + 1) * G], o1), (b, g)
            assert torch.equal(lse[b:b + 1, g * G:(g + 1) * G], l1), (b, g)
    # sampled rows against the oracle: every item position of a workgroup is
    # represented (first and last rows of query tiles across all groups)
    rng = np.random.default_rng(seed)
    flat = B * Hq * Nq
    rows = np.unique(np.concatenate([
        rng.integers(0, flat, size=48),
        np.arange(0, flat, Nq * 7 + 255)[:48],
        [0, flat - 1]]).astype(np.int64))
    o_ref, lse_ref = oracle.attention(bits(q.cpu()), bits(k.cpu()), bits(v.cpu()), dtype, scale,
                                      rows=rows, nthreads=8, causal=causal)
    og = o.cpu().double().numpy().reshape(-1, d)[rows]
    lg = lse.cpu().double().numpy().reshape(-1)[rows]
    assert_parity(og, lg, o_ref, lse_ref,
                  "launch %s" % ((B, Hq, Hkv, Nq, Nk, dtype, scale, causal),), lse_abs=1e-3)


def test_persistent_headline_deterministic():
    """The B=4, H=16, N=4096 bf16 call (persistent on a 256-CU device) twice
    on fresh outputs: the same bits, every output written."""
    announce("persistent headline deterministic")
    if not persistent(4, 16, 16, 4096, 4096):
        pytest.skip("shape does not take the persistent launch on this device")
    q = rand((4, 16, 4096, 128), "bf16", 3).to(DEV)
    k = rand((4, 16, 4096, 128), "bf16", 4).to(DEV)
    v = rand((4, 16, 4096, 128), "bf16", 5).to(DEV)
    outs = []
    for fill in (float("nan"), 7.0):
        o = torch.full_like(q, fill)
        lse = torch.full((4, 16, 4096), fill, device=DEV)
        fa2.fwd(q, k, v, out=o, lse=lse)
        torch.cuda.synchronize()
        outs.append((o.cpu(), lse.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert torch.isfinite(outs[0][0]).all() and torch.isfinite(outs[0][1]).all()
