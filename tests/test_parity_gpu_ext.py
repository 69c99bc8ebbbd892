"""GPU parity of fa2_fwd_ext (causal masking, Nq != Nk, grouped K/V heads)
against the fp64 oracle (needs an MI355X)."""
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


def announce(*what):
    print("CASE", *what, flush=True)


def rand(shape, dtype, seed, mult=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * mult).to(_TD[dtype])


def inputs(B, Hq, Hkv, Nq, Nk, d, dtype, seed):
    return (rand((B, Hq, Nq, d), dtype, seed), rand((B, Hkv, Nk, d), dtype, seed + 1),
            rand((B, Hkv, Nk, d), dtype, seed + 2))


def run_gpu(q, k, v, scale, causal):
    o, lse = fa2.fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def f64(t):
    return t.double().numpy()


def check(q, k, v, dtype, scale, causal, tag, rows=None):
    o, lse = run_gpu(q, k, v, scale, causal)
    o_ref, lse_ref = oracle.attention(bits(q), bits(k), bits(v), dtype, scale, rows=rows,
                                      causal=causal)
    d = q.shape[-1]
    og = f64(o) if rows is None else f64(o).reshape(-1, d)[rows]
    lg = f64(lse) if rows is None else f64(lse).reshape(-1)[rows]
    seen = np.isfinite(lse_ref)
    # rows that see no key: exactly O = 0 and lse = -inf
    assert np.all(og[~seen] == 0.0) and np.all(lg[~seen] == -np.inf), tag
    assert_parity(og[seen], lg[seen], o_ref[seen], lse_ref[seen], tag, lse_abs=1e-3)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("N", [1, 7, 64, 255, 256, 1000])
def test_causal_square(N, dtype, d):
    announce("causal", N, dtype, d)
    q, k, v = inputs(1, 2, 2, N, N, d, dtype, seed=N + d)
    check(q, k, v, dtype, 1.0 / math.sqrt(d), True, "causal N=%d %s d=%d" % (N, dtype, d))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Nq,Nk", [(100, 300), (300, 100), (1, 1000), (257, 513), (600, 31)])
def test_unequal_lengths(Nq, Nk, causal):
    announce("lengths", Nq, Nk, causal)
    q, k, v = inputs(2, 2, 2, Nq, Nk, 128, "bf16", seed=Nq * 7 + Nk)
    check(q, k, v, "bf16", 1.0 / math.sqrt(128), causal,
          "Nq=%d Nk=%d causal=%d" % (Nq, Nk, causal))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (8, 1), (6, 3)])
def test_grouped_heads(Hq, Hkv, causal):
    announce("gqa", Hq, Hkv, causal)
    q, k, v = inputs(2, Hq, Hkv, 200, 330, 128, "fp16", seed=Hq * 10 + Hkv)
    check(q, k, v, "fp16", 1.0 / math.sqrt(128), causal,
          "Hq=%d Hkv=%d causal=%d" % (Hq, Hkv, causal))


@pytest.mark.parametrize("scale", [0.0, -0.2, 1.5])
def test_causal_scales(scale):
    announce("causal scale", scale)
    q, k, v = inputs(1, 2, 2, 300, 300, 64, "bf16", seed=77)
    check(q, k, v, "bf16", scale, True, "causal scale=%g" % scale)


def test_no_keys():
    """Nk = 0: every row sees no key (O = 0, lse = -inf), with or without mask."""
    announce("Nk=0")
    q = rand((1, 2, 50, 128), "bf16", 1).to(DEV)
    k = torch.empty((1, 2, 0, 128), dtype=torch.bfloat16, device=DEV)
    for causal in (False, True):
        o, lse = fa2.fwd(q, k, k.clone(), causal=causal)
        torch.cuda.synchronize()
        assert torch.all(o == 0) and torch.all(lse == -float("inf"))


def test_causal_last_row_equals_full_attention():
    """The last causal row sees every key: bit for bit the non-causal row."""
    announce("causal last row")
    q, k, v = inputs(1, 4, 4, 777, 777, 128, "bf16", seed=9)
    oc, lc = run_gpu(q, k, v, 0.09, True)
    of, lf = run_gpu(q, k, v, 0.09, False)
    assert torch.equal(oc[:, :, -1], of[:, :, -1]) and torch.equal(lc[:, :, -1], lf[:, :, -1])


def test_grouped_heads_equal_repeated_heads():
    """Hkv < Hq gives bit for bit what repeating each K/V head gives."""
    announce("gqa repeat")
    q, k, v = inputs(2, 8, 2, 300, 300, 128, "bf16", seed=11)
    for causal in (False, True):
        og, lg = run_gpu(q, k, v, 0.1, causal)
        kr = k.repeat_interleave(4, dim=1).contiguous()
        vr = v.repeat_interleave(4, dim=1).contiguous()
        orr, lr = run_gpu(q, kr, vr, 0.1, causal)
        assert torch.equal(og, orr) and torch.equal(lg, lr)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hq,Hkv,Nq,Nk", [(32, 4, 1, 1000), (32, 4, 5, 300), (16, 2, 64, 4100),
                                          (8, 8, 3, 513), (12, 3, 100, 90), (32, 1, 17, 2048)])
def test_packed_query_heads(Hq, Hkv, Nq, Nk, causal):
    """Short query blocks: the rows of a K/V head's query heads are tiled
    together, so one workgroup mixes heads (and, causal, rows at different
    diagonal offsets; Nq > Nk leaves rows that see no key)."""
    announce("packed", Hq, Hkv, Nq, Nk, causal)
    q, k, v = inputs(2, Hq, Hkv, Nq, Nk, 128, "bf16", seed=Hq + Nq + Nk)
    check(q, k, v, "bf16", 1.0 / math.sqrt(128), causal,
          "packed Hq=%d Hkv=%d Nq=%d Nk=%d causal=%d" % (Hq, Hkv, Nq, Nk, causal))


@pytest.mark.parametrize("Nq,Nk", [(37, 700), (300, 200), (1, 64)])
def test_packed_heads_equal_repeated_heads(Nq, Nk):
    """Packed rows get bit for bit the result they get in their own head's
    tiles (repeated K/V heads, one query head per K/V head)."""
    announce("packed repeat", Nq, Nk)
    q, k, v = inputs(2, 16, 2, Nq, Nk, 64, "fp16", seed=Nq + 3 * Nk)
    for causal in (False, True):
        og, lg = run_gpu(q, k, v, 0.2, causal)
        kr = k.repeat_interleave(8, dim=1).contiguous()
        vr = v.repeat_interleave(8, dim=1).contiguous()
        orr, lr = run_gpu(q, kr, vr, 0.2, causal)
        assert torch.equal(og, orr) and torch.equal(lg, lr), causal


def test_maximum_query_rows():
    """The largest query block fa2_fwd accepts at d = 128 (Nq*d = 2^31 - 2^20
    elements, less a ragged 7 rows), with 256 keys, which takes the persistent
    launch: query byte offsets then reach the top of their unsigned 32-bit
    range both in the per-lane fragment loads and in the staging of later
    items' query tiles.  Q repeats a block of 4096 distinct rows, so every
    output row is compared, element by element, with the oracle's row for its
    block position (a row's result depends only on its query and the keys)."""
    Nq = (1 << 24) - 8192 - 7
    L, Nk, d = 4096, 256, 128
    announce("max query rows", Nq)
    g = torch.Generator().manual_seed(23)
    qb = torch.randn((L, d), generator=g).to(torch.bfloat16)
    k = torch.randn((1, 1, Nk, d), generator=g).to(torch.bfloat16)
    v = torch.randn((1, 1, Nk, d), generator=g).to(torch.bfloat16)
    reps = -(-Nq // L)
    q = qb.to(DEV).repeat(reps, 1)[:Nq].reshape(1, 1, Nq, d).contiguous()
    o = torch.full_like(q, float("nan"))
    lse = torch.full((1, 1, Nq), float("nan"), device=DEV)
    scale = 1.0 / math.sqrt(d)
    fa2.fwd(q, k.to(DEV), v.to(DEV), scale=scale, out=o, lse=lse)
    torch.cuda.synchronize()
    del q
    o_ref, lse_ref = oracle.attention(bits(qb[None, None]), bits(k), bits(v), "bf16", scale)
    o_ref = torch.from_numpy(o_ref[0, 0]).to(DEV)      # [L, d] fp64
    lse_ref = torch.from_numpy(lse_ref[0, 0]).to(DEV)  # [L]
    o_max = o_sum = lse_rel = 0.0
    step = 256 * L  # rows per chunk, a whole number of blocks
    for r0 in range(0, Nq, step):
        r1 = min(Nq, r0 + step)
        n = r1 - r0
        blk = torch.arange(r0, r1, device=DEV) % L
        e = (o[0, 0, r0:r1].double() - o_ref[blk]).abs()
        assert torch.isfinite(e).all(), "rows %d..%d not all written" % (r0, r1)
        o_max = max(o_max, e.max().item())
        o_sum += e.sum().item()
        le = ((lse[0, 0, r0:r1].double() - lse_ref[blk]).abs() / lse_ref[blk].abs()).max().item()
        assert math.isfinite(le), "lse rows %d..%d not all written" % (r0, r1)
        lse_rel = max(lse_rel, le)
        del e, blk
    err = {"o_max_abs": o_max, "o_mean_abs": o_sum / (Nq * d), "lse_max_rel": lse_rel}
    print("max query rows:", err, flush=True)
    assert o_max <= 2e-2 and err["o_mean_abs"] <= 2e-3 and lse_rel <= 1e-3, err


def test_maximum_key_length():
    """The largest key length fa2_fwd_ext accepts at d = 128 (Nk*d = 2^31 -
    2^20 elements, less a ragged 7), so K and V offsets reach the top of their
    32-bit range.  K and V are a block of 2^20 keys repeated 15 times plus a
    distinct tail whose last 100 keys line up with the (identical) query rows,
    so the output hinges on the farthest keys.  Keys that repeat with their
    values contribute 15 times one block's weights: the expected row merges the
    oracle's (O, lse) of the block and of the tail with those weights."""
    Nk = ((1 << 31) - (1 << 20)) // 128 - 7
    L, R = 1 << 20, 15
    T = Nk - R * L
    announce("max key length", Nk)
    g = torch.Generator().manual_seed(21)
    qrow = torch.randn(128, generator=g)
    q = qrow.repeat(1, 1, 64, 1).to(torch.bfloat16)                   # [1, 1, 64, 128]
    kb = torch.randn((L, 128), generator=g).to(torch.bfloat16)
    vb = torch.randn((L, 128), generator=g).to(torch.bfloat16)
    kt = torch.randn((T, 128), generator=g)
    kt[-100:] = 8.0 * qrow + 0.1 * torch.randn((100, 128), generator=g)
    kt = kt.to(torch.bfloat16)
    vt = torch.randn((T, 128), generator=g).to(torch.bfloat16)
    k = torch.empty((1, 1, Nk, 128), dtype=torch.bfloat16, device=DEV)
    v = torch.empty_like(k)
    for r in range(R):
        k[0, 0, r * L:(r + 1) * L] = kb.to(DEV)
        v[0, 0, r * L:(r + 1) * L] = vb.to(DEV)
    k[0, 0, R * L:] = kt.to(DEV)
    v[0, 0, R * L:] = vt.to(DEV)
    scale = 1.0 / math.sqrt(128)
    o, lse = fa2.fwd(q.to(DEV), k, v, scale=scale)
    torch.cuda.synchronize()
    o, lse = o.cpu().double().numpy()[0, 0], lse.cpu().double().numpy()[0, 0]
    del k, v
    rows = [0, 63]
    ob, lb = oracle.attention(bits(q), bits(kb[None, None]), bits(vb[None, None]), "bf16", scale,
                              rows=rows, nthreads=2)
    ot, lt = oracle.attention(bits(q), bits(kt[None, None]), bits(vt[None, None]), "bf16", scale,
                              rows=rows, nthreads=2)
    for n, i in enumerate(rows):
        m = max(lb[n], lt[n])
        wb, wt = R * math.exp(lb[n] - m), math.exp(lt[n] - m)
        o_ref = (wb * ob[n] + wt * ot[n]) / (wb + wt)
        lse_ref = m + math.log(wb + wt)
        assert_parity(o[i][None], np.array([lse[i]]), o_ref[None], np.array([lse_ref]),
                      "max key length row %d" % i, lse_abs=1e-3)
