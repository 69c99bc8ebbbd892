"""Seeded random shapes against the fp64 oracle (needs an MI355X).

The targeted tests pin one feature at a time; these cases draw every option
together (head dimension, dtype, grouped K/V heads, unequal and ragged query
and key lengths, the causal mask, positive, negative and zero scales, an empty
key set, key splits) so that combinations no targeted case lists are still
compared with the oracle in full.  Each case is fixed by its index: the shapes do not change
from run to run.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from flashattention_forward_tile_amd import fa2
from flashattention_forward_tile_amd.workloads import bits, make_inputs_kv_fp8, make_inputs_kv_int8
from parity import assert_parity

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
_TD = {"bf16": torch.bfloat16, "fp16": torch.float16}
CASES = 40


def announce(*what):
    print("CASE", *what, flush=True)


def draw(i):
    """Shape and options of case i (from its own seeded generator)."""
    rng = np.random.default_rng(1000 + i)
    d = int(rng.choice([64, 128, 256]))
    dtype = str(rng.choice(["bf16", "fp16"]))
    B = int(rng.integers(1, 3))
    Hkv = int(rng.integers(1, 4))
    group = int(rng.choice([1, 2, 4]))
    Nq = int(np.exp(rng.uniform(0.0, math.log(700.0))))
    Nk = 0 if i % 13 == 5 else int(np.exp(rng.uniform(0.0, math.log(1400.0))))
    causal = bool(rng.integers(0, 2))
    scale = float(rng.choice([1.0, 1.0, 0.5, 2.0, -1.0, 0.0])) / math.sqrt(d)
    return dict(B=B, Hq=Hkv * group, Hkv=Hkv, Nq=Nq, Nk=Nk, d=d, dtype=dtype,
                causal=causal, scale=scale)


def compare(o, lse, o_ref, lse_ref, tag):
    og, lg = o.double().numpy(), lse.double().numpy()
    seen = np.isfinite(lse_ref)
    # rows that see no key (causal with Nq > Nk, or no keys): O = 0, lse = -inf
    assert np.all(og[~seen] == 0.0) and np.all(lg[~seen] == -np.inf), tag
    if seen.any():
        assert_parity(og[seen], lg[seen], o_ref[seen], lse_ref[seen], tag, lse_abs=1e-3)


@pytest.mark.parametrize("i", range(CASES))
def test_random_shape(i):
    c = draw(i)
    tag = "random %d %s" % (i, c)
    announce(tag)
    g = torch.Generator().manual_seed(2000 + i)
    td = _TD[c["dtype"]]
    q = torch.randn((c["B"], c["Hq"], c["Nq"], c["d"]), generator=g).to(td)
    k = torch.randn((c["B"], c["Hkv"], c["Nk"], c["d"]), generator=g).to(td)
    v = torch.randn((c["B"], c["Hkv"], c["Nk"], c["d"]), generator=g).to(td)
    o, lse = fa2.fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale=c["scale"], causal=c["causal"])
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(bits(q), bits(k), bits(v), c["dtype"], c["scale"],
                                      causal=c["causal"])
    compare(o.cpu(), lse.cpu(), o_ref, lse_ref, tag)


@pytest.mark.parametrize("i", range(12))
def test_random_shape_int8_cache(i):
    c = draw(i)
    c["d"] = 128
    c["Nk"] = max(c["Nk"], 1)
    c["scale"] = c["scale"] * math.sqrt(draw(i)["d"]) / math.sqrt(128)
    tag = "random int8 %d %s" % (i, c)
    announce(tag)
    q, kq, ks, vq, vs = make_inputs_kv_int8(c["B"], c["Hq"], c["Hkv"], c["Nq"], c["Nk"], 128,
                                            c["dtype"], seed=3000 + i)
    o, lse = fa2.fwd_kv_int8(q.to(DEV), kq.to(DEV), ks.to(DEV), vq.to(DEV), vs.to(DEV),
                             scale=c["scale"], causal=c["causal"])
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_kv_int8(bits(q), kq.numpy(), ks.numpy(), vq.numpy(),
                                              vs.numpy(), c["dtype"], c["scale"],
                                              causal=c["causal"])
    compare(o.cpu(), lse.cpu(), o_ref, lse_ref, tag)


@pytest.mark.parametrize("i", range(12))
def test_random_shape_fp8_cache(i):
    c = draw(i + 100)
    c["d"] = 128
    c["Nk"] = max(c["Nk"], 1)
    c["scale"] = c["scale"] * math.sqrt(draw(i + 100)["d"]) / math.sqrt(128)
    tag = "random fp8 %d %s" % (i, c)
    announce(tag)
    q, kq, ks, vq, vs = make_inputs_kv_fp8(c["B"], c["Hq"], c["Hkv"], c["Nq"], c["Nk"], 128,
                                           c["dtype"], seed=4000 + i)
    o, lse = fa2.fwd_kv_fp8(q.to(DEV), kq.to(DEV), ks.to(DEV), vq.to(DEV), vs.to(DEV),
                            scale=c["scale"], causal=c["causal"])
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_kv_fp8(bits(q), kq.numpy(), ks.numpy(), vq.numpy(),
                                             vs.numpy(), c["dtype"], c["scale"],
                                             causal=c["causal"])
    compare(o.cpu(), lse.cpu(), o_ref, lse_ref, tag)


@pytest.mark.parametrize("i", range(16))
def test_random_shape_key_splits(i):
    """The drawn shapes through fa2_fwd_split, with a split count drawn from
    0 (the library's choice) to 40."""
    c = draw(i + 200)
    splits = int(np.random.default_rng(500 + i).integers(0, 41))
    tag = "random split %d %s splits=%d" % (i, c, splits)
    announce(tag)
    g = torch.Generator().manual_seed(5000 + i)
    td = _TD[c["dtype"]]
    q = torch.randn((c["B"], c["Hq"], c["Nq"], c["d"]), generator=g).to(td)
    k = torch.randn((c["B"], c["Hkv"], c["Nk"], c["d"]), generator=g).to(td)
    v = torch.randn((c["B"], c["Hkv"], c["Nk"], c["d"]), generator=g).to(td)
    o, lse = fa2.fwd_split(q.to(DEV), k.to(DEV), v.to(DEV), scale=c["scale"],
                           causal=c["causal"], splits=splits)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(bits(q), bits(k), bits(v), c["dtype"], c["scale"],
                                      causal=c["causal"])
    compare(o.cpu(), lse.cpu(), o_ref, lse_ref, tag)


@pytest.mark.parametrize("i", range(12))
def test_random_shape_quantized_key_splits(i):
    """Drawn shapes (d = 128) over INT8 (even i) or FP8 (odd i) caches
    through fa2_fwd_kv_split, with a split count drawn from 0 to 40."""
    c = draw(i + 300)
    c["d"] = 128
    c["scale"] = c["scale"] * math.sqrt(draw(i + 300)["d"]) / math.sqrt(128)
    splits = int(np.random.default_rng(700 + i).integers(0, 41))
    fmt = "int8" if i % 2 == 0 else "fp8"
    tag = "random split %s %d %s splits=%d" % (fmt, i, c, splits)
    announce(tag)
    make = make_inputs_kv_int8 if fmt == "int8" else make_inputs_kv_fp8
    q, kq, ks, vq, vs = make(c["B"], c["Hq"], c["Hkv"], c["Nq"], max(c["Nk"], 1), 128,
                             c["dtype"], seed=6000 + i)
    if c["Nk"] == 0:
        kq, vq = kq[:, :, :0].contiguous(), vq[:, :, :0].contiguous()
    cache = fa2.CACHE_INT8 if fmt == "int8" else fa2.CACHE_FP8
    o, lse = fa2.fwd_kv_split(q.to(DEV), kq.to(DEV), ks.to(DEV), vq.to(DEV), vs.to(DEV), cache,
                              scale=c["scale"], causal=c["causal"], splits=splits)
    torch.cuda.synchronize()
    attn = oracle.attention_kv_int8 if fmt == "int8" else oracle.attention_kv_fp8
    o_ref, lse_ref = attn(bits(q), kq.numpy(), ks.numpy(), vq.numpy(), vs.numpy(), c["dtype"],
                          c["scale"], causal=c["causal"])
    compare(o.cpu(), lse.cpu(), o_ref, lse_ref, tag)
