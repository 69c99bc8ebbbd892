"""GPU parity of fa2_fwd_kv_int8 (attention over an INT8 key/value cache)
against the fp64 oracle's INT8 function (needs an MI355X).

The query codes are an integer decision both sides take in binary32, so the
kernel and the oracle compute the same quantized attention and differ only by
floating-point rounding: the tolerances are those of the 16-bit path."""
import math

import numpy as np
import pytest
import torch

import oracle
from flashattention_forward_tile_amd import fa2
from flashattention_forward_tile_amd.workloads import bits, make_inputs_kv_int8
from parity import assert_parity

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def announce(*what):
    print("CASE", *what, flush=True)


def run_gpu(q, kq, ks, vq, vs, scale, causal):
    o, lse = fa2.fwd_kv_int8(q.to(DEV), kq.to(DEV), ks.to(DEV), vq.to(DEV), vs.to(DEV),
                             scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def check(inputs, dtype, scale, causal, tag, rows=None):
    q, kq, ks, vq, vs = inputs
    o, lse = run_gpu(q, kq, ks, vq, vs, scale, causal)
    o_ref, lse_ref = oracle.attention_kv_int8(bits(q), kq.numpy(), ks.numpy(), vq.numpy(),
                                              vs.numpy(), dtype, scale, rows=rows, causal=causal)
    d = q.shape[-1]
    og = o.double().numpy() if rows is None else o.double().numpy().reshape(-1, d)[rows]
    lg = lse.double().numpy() if rows is None else lse.double().numpy().reshape(-1)[rows]
    seen = np.isfinite(lse_ref)
    assert np.all(og[~seen] == 0.0) and np.all(lg[~seen] == -np.inf), tag
    assert_parity(og[seen], lg[seen], o_ref[seen], lse_ref[seen], tag, lse_abs=1e-3)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk", [
    (1, 2, 2, 64, 64), (1, 2, 1, 100, 300), (2, 4, 2, 257, 513), (1, 8, 1, 5, 1000),
    (1, 2, 2, 1, 1), (1, 3, 3, 300, 90), (1, 4, 4, 32, 33)])
def test_int8_cache(B, Hq, Hkv, Nq, Nk, d, dtype, causal):
    announce("int8", B, Hq, Hkv, Nq, Nk, d, dtype, causal)
    inputs = make_inputs_kv_int8(B, Hq, Hkv, Nq, Nk, d, dtype, seed=Nq + 7 * Nk + Hq + d)
    check(inputs, dtype, 1.0 / math.sqrt(d), causal,
          "int8 B=%d Hq=%d Hkv=%d Nq=%d Nk=%d d=%d %s causal=%d" % (
              B, Hq, Hkv, Nq, Nk, d, dtype, causal))



@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_int8_cache_full_height(d, causal):
    """Enough K/V heads that the 256-row workgroups fill the compute units
    (smaller calls at d = 64 and 128 take the 128-row one-part kernels):
    ragged query and key counts on the full-height path."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    H = cus + 16
    announce("int8 full height", H, d, causal)
    inputs = make_inputs_kv_int8(1, H, H, 300, 513, d, "bf16", seed=d + causal)
    check(inputs, "bf16", 1.0 / math.sqrt(d), causal,
          "int8 full height H=%d d=%d causal=%d" % (H, d, causal))


@pytest.mark.parametrize("scale", [0.0, -0.2, 1.5])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_int8_scales(d, scale, causal):
    announce("int8 scale", d, scale, causal)
    inputs = make_inputs_kv_int8(1, 4, 2, 200, 333, d, "bf16", seed=3)
    check(inputs, "bf16", scale, causal, "int8 d=%d scale=%g causal=%d" % (d, scale, causal))


def test_int8_zero_query_rows():
    """Rows of zeros quantize to zero codes and sq = 0: uniform attention over
    the dequantized values (also under the causal mask and with tail keys)."""
    announce("int8 zero rows")
    q, kq, ks, vq, vs = make_inputs_kv_int8(1, 2, 1, 70, 130, 128, "bf16", seed=8)
    q[:, :, ::3] = 0
    for causal in (False, True):
        check((q, kq, ks, vq, vs), "bf16", 0.1, causal, "int8 zero rows causal=%d" % causal)


def test_int8_no_keys():
    announce("int8 Nk=0")
    q, _, ks, _, vs = make_inputs_kv_int8(1, 2, 2, 40, 1, 128, "fp16", seed=1)
    empty = torch.empty((1, 2, 0, 128), dtype=torch.int8, device=DEV)
    for causal in (False, True):
        o, lse = fa2.fwd_kv_int8(q.to(DEV), empty, ks.to(DEV), empty.clone(), vs.to(DEV),
                                 causal=causal)
        torch.cuda.synchronize()
        assert torch.all(o == 0) and torch.all(lse == -float("inf"))


def test_int8_deterministic():
    announce("int8 determinism")
    inputs = [t.to(DEV) for t in make_inputs_kv_int8(2, 8, 2, 600, 700, 128, "bf16", seed=4)]
    o1, l1 = fa2.fwd_kv_int8(*inputs, causal=True)
    o2, l2 = fa2.fwd_kv_int8(*inputs, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_int8_query_codes_golden_on_gpu():
    """The kernel's query codes are the hand-derived ones of
    tests/golden/int8_query_codes.json (ties to even, key scales folded in,
    a zero row, a row where binary32 and exact rationals disagree).  Each
    fixture row, padded with zeros to d = 128, meets one-hot keys (key j holds
    code 1 in channel j) and identity values, so the output is the softmax
    over channels of scale * sq * code: a closed form computed here in fp64
    from the fixture, with the scale chosen so that one code unit moves a
    channel's probability by about 5%, far above the 16-bit rounding."""
    import json
    import os

    announce("int8 golden codes on the GPU")
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                        "int8_query_codes.json")
    cases = json.load(open(path))["cases"]
    d = 128
    eye = torch.eye(d, dtype=torch.int8)
    for dtype in ("bf16", "fp16"):
        sel = [c for c in cases if c["dtype"] == dtype]
        if not sel:
            continue
        B = len(sel)
        td = torch.bfloat16 if dtype == "bf16" else torch.float16
        q = torch.zeros((B, 1, 1, d), dtype=torch.float32)
        ks = torch.ones((B, 1, d), dtype=torch.float32)
        for b, c in enumerate(sel):
            n = len(c["q"])
            q[b, 0, 0, :n] = torch.tensor(c["q"], dtype=torch.float32)
            ks[b, 0, :n] = torch.tensor(c["ks"], dtype=torch.float32)
        q = q.to(td)
        for c in sel:  # the fixture's query values are exact in its dtype
            exact = torch.tensor(c["q"], dtype=torch.float32)
            assert torch.equal(exact.to(td).float(), exact), c["name"]
        kq = eye.expand(B, 1, d, d).contiguous()
        vq = eye.expand(B, 1, d, d).contiguous()
        vs = torch.ones((B, 1, d), dtype=torch.float32)
        for b, c in enumerate(sel):
            sq = np.frombuffer(np.uint32(int(c["sq_bits"], 16)).tobytes(), np.float32)[0]
            codes = np.zeros(d)
            codes[:len(c["codes"])] = c["codes"]
            scale = 0.05 / float(sq) if sq > 0 else 0.3
            o, lse = fa2.fwd_kv_int8(q[b:b + 1].to(DEV), kq[b:b + 1].to(DEV), ks[b:b + 1].to(DEV),
                                     vq[b:b + 1].to(DEV), vs[b:b + 1].to(DEV), scale=scale)
            torch.cuda.synchronize()
            s = scale * float(sq) * codes
            p = np.exp(s - s.max())
            o_ref = p / p.sum()
            lse_ref = s.max() + math.log(p.sum())
            og = o.cpu().double().numpy().reshape(-1)
            rel = np.abs(og - o_ref) / o_ref
            assert rel.max() <= 1e-2, (c["name"], float(rel.max()), int(rel.argmax()))
            assert abs(float(lse.cpu()) - lse_ref) <= 1e-4 * max(1.0, abs(lse_ref)), c["name"]
