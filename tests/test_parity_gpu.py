"""GPU parity of the HIP path against the fp64 oracle (needs an MI355X).

Every case prints its name, shape and seed before touching the GPU, so a
failing run names its case.  Inputs come from the seeded generators in
flashattention_forward_tile_amd.workloads; expected values come only from the
oracle or from closed forms computed here in fp64.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from flashattention_forward_tile_amd import fa2
from flashattention_forward_tile_amd.workloads import (WORKLOADS, bits, make_inputs,
                                                       torch_dtype, workload_inputs)
from parity import assert_parity

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
_TD = {"bf16": torch.bfloat16, "fp16": torch.float16}


def announce(*what):
    print("CASE", *what, flush=True)


def run_gpu(q, k, v, scale):
    o, lse = fa2.fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale=scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def f64(t):
    return t.double().numpy()


def check_full(q, k, v, dtype, scale, tag, **kw):
    o, lse = run_gpu(q, k, v, scale)
    o_ref, lse_ref = oracle.attention(bits(q), bits(k), bits(v), dtype, scale)
    return assert_parity(f64(o), f64(lse), o_ref, lse_ref, tag, **kw)


# ---------------------------------------------------------------- edge cases

@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("N", [1, 2, 3, 31, 33, 64, 65, 127, 129, 200, 257, 1000])
def test_ragged_lengths(N, dtype, d):
    announce("ragged", N, dtype, d)
    q, k, v = make_inputs(1, 2, N, d, dtype, "normal", seed=N)
    check_full(q, k, v, dtype, 1.0 / math.sqrt(d), "ragged N=%d %s d=%d" % (N, dtype, d))


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("scale", [0.0, -0.09, 0.5, 1e-3, -1.0, 40.0, -40.0])
def test_scales(scale, dtype):
    """Scales from uniform attention (0) to near one-hot rows (+-40: logits
    with a spread of about 450, lse up to about 2300, so the running max jumps
    by hundreds of log2 units)."""
    announce("scale", scale, dtype)
    q, k, v = make_inputs(2, 2, 300, 128, dtype, "normal", seed=5)
    # lse can sit near 0 for a negative scale; bound it absolutely there too
    check_full(q, k, v, dtype, scale, "scale=%g %s" % (scale, dtype), lse_abs=1e-3)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_stress_distribution_all_head_dims(d):
    announce("stress", d)
    q, k, v = make_inputs(1, 4, 512, d, "bf16", "stress", seed=d)
    check_full(q, k, v, "bf16", 1.0 / math.sqrt(d), "stress d=%d" % d)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_running_max_jumps_late(d, dtype):
    """Keys far into the sequence whose logits jump far above everything
    before them (to about 30 and then 60 in log2 units, so the tile's sum of
    p passes any limit the lazy reference max allows): the rows' reference
    must move, the output already accumulated must be rescaled, and the
    result stays within tolerance.  Full comparison with the oracle."""
    announce("late max jump", d, dtype)
    B, H, N = 1, 2, 1500
    g = torch.Generator().manual_seed(40 + d)
    q = torch.randn((B, H, N, d), generator=g)
    k = torch.randn((B, H, N, d), generator=g)
    v = torch.randn((B, H, N, d), generator=g)
    scale = 1.0 / math.sqrt(d)
    c = scale / math.log(2.0)  # logit in log2 units per unit of q.k
    # key 700 along query row 0 with log2-unit logit 30 for that row; key 1300
    # along row 1 with 60 (other rows see them at about +-30/sqrt(d) and
    # +-60/sqrt(d))
    for h in range(H):
        for key, row, target in ((700, 0, 30.0), (1300, 1, 60.0)):
            qr = q[0, h, row]
            k[0, h, key] = qr * (target / (c * float(qr @ qr)))
    q, k, v = q.to(_TD[dtype]), k.to(_TD[dtype]), v.to(_TD[dtype])
    check_full(q, k, v, dtype, scale, "late max jump d=%d %s" % (d, dtype))


def test_empty_inputs():
    announce("empty")
    for shape in ((0, 2, 64, 128), (1, 0, 64, 128), (1, 2, 0, 128)):
        q = torch.empty(shape, dtype=torch.bfloat16, device=DEV)
        o, lse = fa2.fwd(q, q.clone(), q.clone())
        assert o.shape == shape and lse.shape == shape[:3]


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_constant_values(dtype):
    """All rows of V equal c: O = c.  The weights are rounded to 16 bits for
    the second product while l sums them unrounded, so O may differ from c by
    the weights' rounding, well under one 16-bit ulp of c on average."""
    announce("constant V", dtype)
    B, H, N, d = 2, 2, 777, 128
    q, k, _ = make_inputs(B, H, N, d, dtype, "normal", seed=3)
    c = torch.randn(1, 1, 1, d, generator=torch.Generator().manual_seed(4)).to(_TD[dtype])
    v = c.expand(B, H, N, d).contiguous()
    o, _ = run_gpu(q, k, v, 1.0 / math.sqrt(d))
    rel = np.abs(f64(o) - f64(v)) / np.abs(f64(v))
    ulp = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -11
    assert rel.max() <= 2 * ulp and (o == v).double().mean() >= 0.9


@pytest.mark.parametrize("N", [256, 4096])
def test_uniform_attention(N):
    """Q = 0: O is the column mean of V and lse = ln N."""
    announce("Q=0", N)
    d = 128
    _, k, v = make_inputs(1, 2, N, d, "bf16", "normal", seed=6)
    q = torch.zeros_like(k)
    o, lse = run_gpu(q, k, v, 1.0 / math.sqrt(d))
    mean = f64(v).mean(axis=2, keepdims=True)
    assert np.abs(f64(o) - mean).max() <= 2e-2 * 0.1
    assert np.allclose(f64(lse), math.log(N), rtol=1e-6, atol=0)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_worked_examples_on_gpu(dtype):
    """The hand-derived examples of tests/golden/worked_examples.json (exact
    fractions for O, ln of a fraction for lse), zero-padded to d = 64 (padding
    adds nothing to q.k and gives zero output channels), straight against the
    printed values: no oracle in between.  The bars are the output's own
    rounding (half an ulp of 16-bit O) plus that of P."""
    import json
    import os
    from fractions import Fraction

    announce("worked examples", dtype)
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                        "worked_examples.json")
    td = _TD[dtype]
    for case in json.load(open(path))["cases"]:
        sign = -1.0 if case["scale"].startswith("-") else 1.0
        scale = sign * math.log(2.0 if case["scale"].lstrip("-") == "ln2" else 3.0)
        qa, ka, va = (torch.tensor(case[x], dtype=torch.float32) for x in ("q", "k", "v"))
        N, dd = qa.shape
        pad = lambda t: torch.nn.functional.pad(t, (0, 64 - t.shape[1]))[None, None].to(td)
        o, lse = run_gpu(pad(qa), pad(ka), pad(va), scale)
        o = f64(o)[0, 0]
        o_ref = np.array([[float(Fraction(x)) for x in row] for row in case["O"]])
        lse_ref = np.array([math.log(Fraction(x)) for x in case["lse_ln"]])
        ulp = 2.0 ** (-8 if dtype == "bf16" else -11)
        bar = ulp * np.maximum(np.abs(o_ref), 1.0) + ulp * va.abs().max().item()
        assert np.all(np.abs(o[:, :dd] - o_ref) <= bar), (case["name"], o[:, :dd], o_ref)
        assert np.all(o[:, dd:] == 0.0), case["name"]
        assert np.allclose(f64(lse)[0, 0], lse_ref, rtol=0, atol=1e-5), case["name"]


def test_rank_one_logits_closed_form():
    """Q and K nonzero only in coordinate 0: s_ij = scale * a_i * b_j, so the
    softmax is computable directly in fp64 without the oracle."""
    announce("rank-one logits")
    B, H, N, d = 1, 2, 512, 64
    g = torch.Generator().manual_seed(8)
    a = torch.randn(B, H, N, generator=g).to(torch.bfloat16)
    b = torch.randn(B, H, N, generator=g).to(torch.bfloat16)
    q = torch.zeros(B, H, N, d, dtype=torch.bfloat16)
    k = torch.zeros(B, H, N, d, dtype=torch.bfloat16)
    q[..., 0] = a
    k[..., 0] = b
    v = torch.randn(B, H, N, d, generator=g).to(torch.bfloat16)
    scale = 3.0
    o, lse = run_gpu(q, k, v, scale)
    s = scale * f64(a)[..., :, None] * f64(b)[..., None, :]
    mx = s.max(axis=-1, keepdims=True)
    w = np.exp(s - mx)
    o_ref = (w @ f64(v)) / w.sum(axis=-1, keepdims=True)
    lse_ref = mx[..., 0] + np.log(w.sum(axis=-1))
    assert_parity(f64(o), f64(lse), o_ref, lse_ref, "rank-one", lse_abs=1e-3)


# ---------------------------------------------------------------- invariants

def test_logit_shift_invariance():
    """K -> K + 1 u^T (exact in bf16) leaves O alone and shifts lse by
    scale * <q_i, u>, on the GPU itself."""
    announce("shift")
    B, H, N, d = 1, 2, 1024, 128
    rng = np.random.default_rng(9)
    q, _, v = make_inputs(B, H, N, d, "bf16", "normal", seed=9)
    kk = np.clip(np.round(rng.standard_normal((B, H, N, d)) * 16) / 16, -7.5, 7.5)
    u = np.clip(np.round(rng.standard_normal(d) * 16) / 16, -7.5, 7.5)
    k0 = torch.from_numpy(kk).to(torch.bfloat16)
    k1 = torch.from_numpy(kk + u).to(torch.bfloat16)
    assert torch.equal(k1.double(), torch.from_numpy(kk + u))
    scale = 1.0 / math.sqrt(d)
    o0, l0 = run_gpu(q, k0, v, scale)
    o1, l1 = run_gpu(q, k1, v, scale)
    diff = np.abs(f64(o0) - f64(o1))
    assert diff.max() <= 2e-2 and diff.mean() <= 2e-3
    shift = scale * (f64(q) @ u)
    assert np.allclose(f64(l1) - f64(l0), shift, rtol=0, atol=2e-3 * np.abs(f64(l1)).max())


def test_key_permutation_invariance():
    announce("permutation")
    B, H, N, d = 1, 2, 640, 128
    q, k, v = make_inputs(B, H, N, d, "bf16", "normal", seed=10)
    perm = torch.randperm(N, generator=torch.Generator().manual_seed(11))
    o0, l0 = run_gpu(q, k, v, 0.1)
    o1, l1 = run_gpu(q, k[:, :, perm].contiguous(), v[:, :, perm].contiguous(), 0.1)
    diff = np.abs(f64(o0) - f64(o1))
    assert diff.max() <= 2e-2 and diff.mean() <= 2e-3
    assert np.allclose(f64(l0), f64(l1), rtol=1e-4)
    oq, lq = run_gpu(q[:, :, perm].contiguous(), k, v, 0.1)
    assert torch.equal(oq, o0[:, :, perm]) and torch.equal(lq, l0[:, :, perm])


# ---------------------------------------------------------------- hygiene

def test_deterministic_and_fully_written():
    """Two runs into NaN-prefilled outputs give bit-identical, finite results."""
    w = WORKLOADS["headline"]
    announce("determinism", w)
    q, k, v = (t.to(DEV) for t in workload_inputs(w, seed=1))
    outs = []
    for _ in range(2):
        o = torch.full_like(q, float("nan"))
        lse = torch.full((w.B, w.H, w.N), float("nan"), device=DEV)
        fa2.fwd(q, k, v, scale=w.scale, out=o, lse=lse)
        torch.cuda.synchronize()
        assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
        outs.append((o, lse))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_non_default_stream():
    announce("stream")
    q, k, v = make_inputs(2, 4, 512, 128, "fp16", "normal", seed=12)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    ref_o, ref_l = fa2.fwd(qd, kd, vd)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o, lse = fa2.fwd(qd, kd, vd)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(lse, ref_l)


def test_concurrent_streams():
    """Different calls in flight at once on two streams (a persistent launch,
    a causal grouped-head launch, a d = 64 launch) give bit for bit what each
    gives alone: the library keeps no state between or across calls."""
    announce("concurrent streams")
    cases = [
        (make_inputs(4, 16, 2048, 128, "bf16", "normal", seed=31), False),
        (make_inputs(2, 8, 700, 128, "fp16", "normal", seed=32, Hkv=2, Nk=1500), True),
        (make_inputs(2, 4, 900, 64, "bf16", "normal", seed=33), False),
    ]
    dev = [((q.to(DEV), k.to(DEV), v.to(DEV)), c) for (q, k, v), c in cases]
    alone = []
    for (q, k, v), c in dev:
        alone.append(fa2.fwd(q, k, v, causal=c))
        torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    together = []
    for rep in range(3):
        for i, ((q, k, v), c) in enumerate(dev):
            with torch.cuda.stream(streams[(i + rep) % 2]):
                together.append((i, fa2.fwd(q, k, v, causal=c)))
    torch.cuda.synchronize()
    for i, (o, lse) in together:
        assert torch.equal(o, alone[i][0]) and torch.equal(lse, alone[i][1]), i


def test_device_argument_errors():
    announce("errors")
    q = torch.randn(1, 2, 64, 128, device=DEV).to(torch.bfloat16)
    k, v = q.clone(), q.clone()
    o = torch.empty_like(q)
    lse = torch.empty(1, 2, 64, device=DEV)
    p = lambda t: t.data_ptr()
    # misaligned by one element
    assert fa2.fwd_raw(p(q) + 2, p(k), p(v), p(o), p(lse), 1, 2, 63, 128, 0.1, fa2.BF16) == fa2.ERR_ALIGN
    # output on top of an input
    assert fa2.fwd_raw(p(q), p(k), p(v), p(q), p(lse), 1, 2, 64, 128, 0.1, fa2.BF16) == fa2.ERR_ALIAS
    assert fa2.fwd_raw(p(q), p(k), p(v), p(o), p(lse), 1, 2, 64, 96, 0.1, fa2.BF16) == fa2.ERR_HEADDIM
    with pytest.raises(ValueError):
        fa2.fwd(q, k.to(torch.float16), v)
    with pytest.raises(ValueError):
        fa2.fwd(q.transpose(2, 3), k.transpose(2, 3), v.transpose(2, 3))
    with pytest.raises(ValueError):
        fa2.fwd(q.cpu(), k.cpu(), v.cpu())
