"""Pins of the fp64 oracle: checks against what mathematics fixes, not itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError if
that oracle disagrees with the definition of scaled dot-product attention
(softmax(scale * Q K^T) V, natural-log logsumexp) through:
  * exact fixtures hand-derived from the definition (tests/golden),
  * closed forms (N = 1, N = 2, Q = 0, scale = 0, constant V, V = I),
  * invariants (logit shift, permutations, head independence, linearity),
  * brute force in pure Python (math.fsum) on tiny inputs,
  * library routines (torch fp64 softmax / scaled_dot_product_attention),
  * exact decoding of every 16-bit pattern, and extreme-logit stability.
Causal masking, unequal query/key lengths and grouped key/value heads are
pinned the same ways: truncation to the visible prefix, torch fp64 SDPA with an
explicit bottom-right mask or enable_gqa, repeated key/value heads, brute
force, and the closed forms of the first row and of rows that see no key.
They are plain functions so the same pins also run against deliberately broken
copies of the oracle (test_oracle_mutants.py), which they must reject.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

from flashattention_forward_tile_amd.workloads import bits, from_bits, make_inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
DTYPES = ("bf16", "fp16")
_TD = {"bf16": torch.bfloat16, "fp16": torch.float16}


def _t16(x, dtype):
    """Exact 16-bit tensor from float values (callers pass representable ones)."""
    t = torch.as_tensor(np.asarray(x, dtype=np.float64)).to(_TD[dtype])
    assert torch.equal(t.double(), torch.as_tensor(np.asarray(x, np.float64))), \
        "fixture value not representable in %s" % dtype
    return t


def _f64(t):
    return t.double().numpy()


def _rand16(shape, dtype, seed, mult=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * mult).to(_TD[dtype])


def _run(orc, q, k, v, dtype, scale, **kw):
    return orc.attention(bits(q), bits(k), bits(v), dtype, scale, **kw)


def _visible(i, Nq, Nk):
    """Keys a causal row i sees: 0 .. i + Nk - Nq (bottom-right aligned)."""
    return max(0, min(Nk, i + 1 + Nk - Nq))


# --------------------------------------------------------------------------
# decoding

def pin_decode_every_pattern(orc):
    pats = np.arange(65536, dtype=np.uint16)
    got = orc.decode(pats, "bf16")
    ref = from_bits(pats, "bf16").double().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok]), "bf16 decode"
    got = orc.decode(pats, "fp16")
    ref = pats.view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok]), "fp16 decode"


# --------------------------------------------------------------------------
# exact hand-derived fixtures

def _parse_scale(s):
    sign = -1.0 if s.startswith("-") else 1.0
    body = s.lstrip("-")
    assert body in ("ln2", "ln3")
    return sign * math.log(2.0 if body == "ln2" else 3.0)


def pin_worked_examples(orc):
    with open(os.path.join(GOLDEN, "worked_examples.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        scale = _parse_scale(case["scale"])
        for dtype in DTYPES:
            q = _t16(case["q"], dtype)[None, None]
            k = _t16(case["k"], dtype)[None, None]
            v = _t16(case["v"], dtype)[None, None]
            o, lse = _run(orc, q, k, v, dtype, scale)
            o_ref = np.array([[float(Fraction(x)) for x in row] for row in case["O"]])
            lse_ref = np.array([math.log(Fraction(x)) for x in case["lse_ln"]])
            assert np.allclose(o[0, 0], o_ref, rtol=0, atol=1e-13), case["name"]
            assert np.allclose(lse[0, 0], lse_ref, rtol=0, atol=1e-13), case["name"]


# --------------------------------------------------------------------------
# brute force in pure Python

def _brute_row(qi, K, V, scale):
    """softmax by p_j = exp(s_j - lse), lse by max + log(fsum(exp))."""
    s = [scale * math.fsum(a * b for a, b in zip(qi, kj)) for kj in K]
    mx = max(s)
    lse = mx + math.log(math.fsum(math.exp(x - mx) for x in s))
    p = [math.exp(x - lse) for x in s]
    o = [math.fsum(pj * vj[c] for pj, vj in zip(p, V)) for c in range(len(V[0]))]
    return o, lse


def pin_brute_force_tiny(orc):
    rng = np.random.default_rng(7)
    shapes = [(1, 1, 1, 1), (1, 2, 3, 2), (2, 1, 4, 3), (1, 1, 4, 4), (2, 2, 2, 5)]
    scales = [1.0, 0.37, -0.8, 0.0, 2.5]
    for dtype in DTYPES:
        for shp, scale in zip(shapes, scales):
            # entries on a grid of quarters in [-2, 2]: exact in both dtypes
            q = rng.integers(-8, 9, size=shp) / 4.0
            k = rng.integers(-8, 9, size=shp) / 4.0
            v = rng.integers(-8, 9, size=shp) / 4.0
            o, lse = _run(orc, _t16(q, dtype), _t16(k, dtype), _t16(v, dtype),
                          dtype, scale)
            B, H, N, d = shp
            for b in range(B):
                for h in range(H):
                    for i in range(N):
                        ob, lb = _brute_row(q[b, h, i].tolist(), k[b, h].tolist(),
                                            v[b, h].tolist(), scale)
                        assert np.allclose(o[b, h, i], ob, rtol=0, atol=1e-12), (shp, i)
                        assert abs(lse[b, h, i] - lb) <= 1e-12 * max(1.0, abs(lb)), (shp, i)


# --------------------------------------------------------------------------
# library routines

def pin_torch_fp64(orc):
    import torch.nn.functional as F
    for dtype, (B, H, N, d) in (("bf16", (1, 2, 256, 128)), ("fp16", (2, 1, 128, 64))):
        q, k, v = make_inputs(B, H, N, d, dtype, "normal", seed=11)
        scale = 1.0 / math.sqrt(d)
        o, lse = _run(orc, q, k, v, dtype, scale)
        qd, kd, vd = q.double(), k.double(), v.double()
        logits = scale * (qd @ kd.transpose(-1, -2))
        o_ref = torch.softmax(logits, dim=-1) @ vd
        o_sdpa = F.scaled_dot_product_attention(qd, kd, vd, scale=scale)
        lse_ref = torch.logsumexp(logits, dim=-1)
        assert np.allclose(o, o_ref.numpy(), rtol=0, atol=1e-10)
        assert np.allclose(o, o_sdpa.numpy(), rtol=0, atol=1e-10)
        assert np.allclose(lse, lse_ref.numpy(), rtol=1e-12, atol=0)


# --------------------------------------------------------------------------
# closed forms

def pin_identity_values_are_probabilities(orc):
    """V = I (N <= d): O_i is the probability row; rows sum to 1, P = exp(s - lse)."""
    for dtype in DTYPES:
        N = d = 64
        q = _rand16((1, 1, N, d), dtype, 21)
        k = _rand16((1, 1, N, d), dtype, 22)
        v = torch.eye(N, d).to(_TD[dtype])[None, None]
        scale = 0.3
        o, lse = _run(orc, q, k, v, dtype, scale)
        p = o[0, 0]
        assert np.all(p >= 0)
        assert np.allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
        s = scale * (_f64(q[0, 0]) @ _f64(k[0, 0]).T)
        assert np.allclose(p, np.exp(s - lse[0, 0][:, None]), rtol=1e-12, atol=1e-300)


def pin_constant_values(orc):
    """Every row of V equal to c: O_i = c for every query."""
    for dtype in DTYPES:
        B, H, N, d = 1, 2, 96, 32
        q = _rand16((B, H, N, d), dtype, 31, 2.0)
        k = _rand16((B, H, N, d), dtype, 32)
        c = _rand16((1, 1, 1, d), dtype, 33)
        v = c.expand(B, H, N, d).contiguous()
        o, _ = _run(orc, q, k, v, dtype, 0.5)
        assert np.allclose(o, np.broadcast_to(_f64(c), o.shape), rtol=1e-13, atol=1e-15)


def pin_uniform_attention(orc):
    """Q = 0 or scale = 0: O_i = column mean of V and lse_i = ln N."""
    for dtype in DTYPES:
        B, H, N, d = 1, 2, 256, 16
        k = _rand16((B, H, N, d), dtype, 41)
        v = _rand16((B, H, N, d), dtype, 42)
        mean = _f64(v).mean(axis=2, keepdims=True)
        for q, scale in ((torch.zeros(B, H, N, d, dtype=_TD[dtype]), 0.7),
                         (_rand16((B, H, N, d), dtype, 43), 0.0)):
            o, lse = _run(orc, q, k, v, dtype, scale)
            assert np.allclose(o, np.broadcast_to(mean, o.shape), rtol=0, atol=1e-14)
            # ln 256 = 8 ln 2 = 5.545177444479562
            assert np.allclose(lse, 5.545177444479562, rtol=0, atol=1e-14)


def pin_single_key(orc):
    """N = 1: O = v_0 exactly; lse = the one logit."""
    for dtype in DTYPES:
        q = _rand16((2, 3, 1, 8), dtype, 51)
        k = _rand16((2, 3, 1, 8), dtype, 52)
        v = _rand16((2, 3, 1, 8), dtype, 53)
        o, lse = _run(orc, q, k, v, dtype, 0.9)
        assert np.array_equal(o, _f64(v))
        s = 0.9 * np.einsum("bhnc,bhnc->bhn", _f64(q), _f64(k))
        assert np.allclose(lse, s, rtol=1e-14, atol=1e-15)


def pin_two_keys(orc):
    """N = 2: O_i = sigma(s_i0 - s_i1) v_0 + sigma(s_i1 - s_i0) v_1."""
    for dtype in DTYPES:
        q = _rand16((1, 2, 2, 8), dtype, 61, 2.0)
        k = _rand16((1, 2, 2, 8), dtype, 62)
        v = _rand16((1, 2, 2, 8), dtype, 63)
        scale = 0.75
        o, lse = _run(orc, q, k, v, dtype, scale)
        qd, kd, vd = _f64(q), _f64(k), _f64(v)
        for h in range(2):
            for i in range(2):
                s0 = scale * math.fsum(qd[0, h, i] * kd[0, h, 0])
                s1 = scale * math.fsum(qd[0, h, i] * kd[0, h, 1])
                w0 = 1.0 / (1.0 + math.exp(s1 - s0))
                w1 = 1.0 / (1.0 + math.exp(s0 - s1))
                ref = w0 * vd[0, h, 0] + w1 * vd[0, h, 1]
                assert np.allclose(o[0, h, i], ref, rtol=0, atol=1e-14)
                big = max(s0, s1)
                lref = big + math.log1p(math.exp(min(s0, s1) - big))
                assert abs(lse[0, h, i] - lref) <= 1e-14 * max(1.0, abs(lref))


# --------------------------------------------------------------------------
# invariants

def pin_logit_shift(orc):
    """K -> K + 1 u^T adds scale*<q_i, u> to row i's logits: O unchanged,
    lse shifted by exactly that amount.  K and u sit on a 1/16 grid with
    |K + u| < 16, so K + u is exact in bf16 and fp16."""
    rng = np.random.default_rng(71)
    for dtype in DTYPES:
        B, H, N, d = 1, 2, 128, 32
        q = _rand16((B, H, N, d), dtype, 72)
        kk = np.clip(np.round(rng.standard_normal((B, H, N, d)) * 16) / 16, -7.5, 7.5)
        u = np.clip(np.round(rng.standard_normal((1, 1, 1, d)) * 32) / 16, -7.5, 7.5)
        k0 = _t16(kk, dtype)
        k1 = _t16(kk + u, dtype)
        v = _rand16((B, H, N, d), dtype, 73)
        scale = 0.4
        o0, l0 = _run(orc, q, k0, v, dtype, scale)
        o1, l1 = _run(orc, q, k1, v, dtype, scale)
        assert np.allclose(o0, o1, rtol=0, atol=1e-12)
        shift = scale * (_f64(q) @ u[0, 0, 0])
        assert np.allclose(l1 - l0, shift, rtol=0, atol=1e-11)


def pin_permutations(orc):
    """Permuting K and V rows together leaves O alone; permuting Q rows permutes O."""
    for dtype in DTYPES:
        B, H, N, d = 1, 1, 64, 16
        q = _rand16((B, H, N, d), dtype, 81)
        k = _rand16((B, H, N, d), dtype, 82)
        v = _rand16((B, H, N, d), dtype, 83)
        perm = torch.randperm(N, generator=torch.Generator().manual_seed(84))
        o, lse = _run(orc, q, k, v, dtype, 0.6)
        o_kv, lse_kv = _run(orc, q, k[:, :, perm], v[:, :, perm], dtype, 0.6)
        assert np.allclose(o, o_kv, rtol=0, atol=1e-13)
        assert np.allclose(lse, lse_kv, rtol=1e-14, atol=0)
        o_q, lse_q = _run(orc, q[:, :, perm], k, v, dtype, 0.6)
        assert np.array_equal(o_q, o[:, :, perm.numpy()])
        assert np.array_equal(lse_q, lse[:, :, perm.numpy()])


def pin_value_linearity(orc):
    """O is linear in V: V -> 2V and V -> -V scale O exactly (bit for bit)."""
    for dtype in DTYPES:
        q = _rand16((1, 2, 48, 24), dtype, 91)
        k = _rand16((1, 2, 48, 24), dtype, 92)
        v = _rand16((1, 2, 48, 24), dtype, 93)
        o, lse = _run(orc, q, k, v, dtype, 0.3)
        o2, lse2 = _run(orc, q, k, v * 2, dtype, 0.3)
        on, _ = _run(orc, q, k, -v, dtype, 0.3)
        assert np.array_equal(o2, 2 * o)
        assert np.array_equal(on, -o)
        assert np.array_equal(lse2, lse)


def pin_head_independence(orc):
    """Each (b, h) is attention on its own slice: a batched call equals the
    per-head calls bit for bit, and rows= equals the full result."""
    for dtype in DTYPES:
        B, H, N, d = 2, 3, 40, 8
        q = _rand16((B, H, N, d), dtype, 101)
        k = _rand16((B, H, N, d), dtype, 102)
        v = _rand16((B, H, N, d), dtype, 103)
        o, lse = _run(orc, q, k, v, dtype, 0.5)
        for b in range(B):
            for h in range(H):
                sl = (slice(b, b + 1), slice(h, h + 1))
                oh, lh = _run(orc, q[sl], k[sl], v[sl], dtype, 0.5)
                assert np.array_equal(oh[0, 0], o[b, h])
                assert np.array_equal(lh[0, 0], lse[b, h])
        rows = np.array([5, 0, B * H * N - 1, 77, 123])
        orow, lrow = _run(orc, q, k, v, dtype, 0.5, rows=rows)
        assert np.array_equal(orow, o.reshape(-1, d)[rows])
        assert np.array_equal(lrow, lse.reshape(-1)[rows])


def pin_extreme_logits(orc):
    """Logits of magnitude ~1e3 (exp overflows/underflows in fp64 without the
    max subtraction): a key ahead by a gap >> 40 takes all the weight, and lse
    equals that key's logit."""
    for dtype in DTYPES:
        N, d = 8, 4
        q = _t16(np.full((1, 1, N, d), 4.0), dtype)
        kk = np.zeros((1, 1, N, d))
        kk[0, 0, :, 0] = [-3.0, 1.0, 2.0, -1.0, 0.0, 3.0, 0.5, -2.0]  # key 5 wins
        k = _t16(kk, dtype)
        v = _rand16((1, 1, N, d), dtype, 111)
        for scale in (100.0, 250.0):  # logits scale*4*k0 reach 3000 and -3000
            o, lse = _run(orc, q, k, v, dtype, scale)
            assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
            assert np.allclose(o[0, 0], np.broadcast_to(_f64(v)[0, 0, 5], (N, d)),
                               rtol=0, atol=1e-12)
            assert np.allclose(lse[0, 0], scale * 4 * 3.0, rtol=1e-15, atol=0)
        # every logit very negative: still a proper softmax
        kk[0, 0, :, 0] = -np.array([3.0, 2.0, 2.5, 3.0, 2.0, 3.0, 2.25, 3.0])
        k = _t16(kk, dtype)
        o, lse = _run(orc, q, k, v, dtype, 100.0)
        assert np.all(np.isfinite(o))
        w = np.zeros(N)
        w[[1, 4]] = 0.5  # the two keys at logit -800 share the weight
        assert np.allclose(o[0, 0], np.broadcast_to(w @ _f64(v)[0, 0], (N, d)),
                           rtol=0, atol=1e-12)
        assert np.allclose(lse[0, 0], -800.0 + math.log(2.0), rtol=1e-15, atol=0)


# --------------------------------------------------------------------------
# causal masking, unequal lengths, grouped heads

def pin_causal_is_prefix_attention(orc):
    """Causal row i equals plain attention of q_i over the keys it sees, bit
    for bit; rows that see no key get O = 0 and lse = -inf."""
    for dtype in DTYPES:
        for Nq, Nk in ((40, 40), (24, 40), (40, 24), (1, 9)):
            q = _rand16((1, 2, Nq, 8), dtype, 121)
            k = _rand16((1, 2, Nk, 8), dtype, 122)
            v = _rand16((1, 2, Nk, 8), dtype, 123)
            o, lse = _run(orc, q, k, v, dtype, 0.7, causal=True)
            for h in range(2):
                for i in range(Nq):
                    n = _visible(i, Nq, Nk)
                    if n == 0:
                        assert np.all(o[0, h, i] == 0.0) and lse[0, h, i] == -np.inf
                        continue
                    sl = (slice(0, 1), slice(h, h + 1))
                    op, lp = _run(orc, q[sl][:, :, i:i + 1], k[sl][:, :, :n].contiguous(),
                                  v[sl][:, :, :n].contiguous(), dtype, 0.7)
                    # a single query row against n keys: same arithmetic
                    assert np.array_equal(op[0, 0, 0], o[0, h, i]), (Nq, Nk, i)
                    assert np.array_equal(lp[0, 0, 0], lse[0, h, i]), (Nq, Nk, i)


def pin_causal_first_row(orc):
    """Nq == Nk, causal: row 0 sees key 0 only, so O_0 = v_0 exactly and lse_0 is
    its logit."""
    for dtype in DTYPES:
        q = _rand16((2, 2, 16, 8), dtype, 131)
        k = _rand16((2, 2, 16, 8), dtype, 132)
        v = _rand16((2, 2, 16, 8), dtype, 133)
        o, lse = _run(orc, q, k, v, dtype, 0.5, causal=True)
        assert np.array_equal(o[:, :, 0], _f64(v)[:, :, 0])
        s00 = 0.5 * np.einsum("bhc,bhc->bh", _f64(q)[:, :, 0], _f64(k)[:, :, 0])
        assert np.allclose(lse[:, :, 0], s00, rtol=1e-14, atol=1e-15)


def pin_causal_and_lengths_torch(orc):
    """torch fp64 SDPA with an explicit bottom-right boolean mask (causal) or
    none, for Nq != Nk."""
    import torch.nn.functional as F
    for dtype in DTYPES:
        for Nq, Nk, causal in ((48, 80, True), (80, 48, True), (48, 80, False),
                               (64, 64, True)):
            q = _rand16((1, 2, Nq, 16), dtype, 141)
            k = _rand16((1, 2, Nk, 16), dtype, 142)
            v = _rand16((1, 2, Nk, 16), dtype, 143)
            o, lse = _run(orc, q, k, v, dtype, 0.25, causal=causal)
            qd, kd, vd = q.double(), k.double(), v.double()
            if causal:
                i = torch.arange(Nq)[:, None]
                j = torch.arange(Nk)[None, :]
                mask = j <= i + (Nk - Nq)
            else:
                mask = torch.ones(Nq, Nk, dtype=torch.bool)
            rows = mask.any(dim=1).numpy()
            ref = F.scaled_dot_product_attention(qd, kd, vd, attn_mask=mask, scale=0.25)
            logits = (0.25 * qd @ kd.transpose(-1, -2)).masked_fill(~mask, float("-inf"))
            lref = torch.logsumexp(logits, dim=-1)
            assert np.allclose(o[:, :, rows], ref.numpy()[:, :, rows], rtol=0, atol=1e-10)
            assert np.allclose(lse[:, :, rows], lref.numpy()[:, :, rows], rtol=1e-12, atol=0)
            assert np.all(o[:, :, ~rows] == 0.0) and np.all(lse[:, :, ~rows] == -np.inf)


def pin_causal_brute_force(orc):
    rng = np.random.default_rng(151)
    for dtype in DTYPES:
        for (Nq, Nk) in ((3, 3), (2, 4), (4, 2), (1, 3)):
            q = rng.integers(-8, 9, size=(1, 1, Nq, 3)) / 4.0
            k = rng.integers(-8, 9, size=(1, 1, Nk, 3)) / 4.0
            v = rng.integers(-8, 9, size=(1, 1, Nk, 3)) / 4.0
            o, lse = _run(orc, _t16(q, dtype), _t16(k, dtype), _t16(v, dtype), dtype, 0.9,
                          causal=True)
            for i in range(Nq):
                n = _visible(i, Nq, Nk)
                if n == 0:
                    assert lse[0, 0, i] == -np.inf
                    continue
                ob, lb = _brute_row(q[0, 0, i].tolist(), k[0, 0, :n].tolist(),
                                    v[0, 0, :n].tolist(), 0.9)
                assert np.allclose(o[0, 0, i], ob, rtol=0, atol=1e-12)
                assert abs(lse[0, 0, i] - lb) <= 1e-12 * max(1.0, abs(lb))


def pin_grouped_heads_are_repeated_heads(orc):
    """Hkv < Hq: identical, bit for bit, to repeating each key/value head for
    its Hq/Hkv query heads; and equal to torch SDPA with enable_gqa."""
    import torch.nn.functional as F
    for dtype in DTYPES:
        for Hq, Hkv in ((4, 2), (6, 1), (4, 4)):
            q = _rand16((2, Hq, 20, 8), dtype, 161)
            k = _rand16((2, Hkv, 28, 8), dtype, 162)
            v = _rand16((2, Hkv, 28, 8), dtype, 163)
            for causal in (False, True):
                o, lse = _run(orc, q, k, v, dtype, 0.6, causal=causal)
                rep = Hq // Hkv
                kr = k.repeat_interleave(rep, dim=1).contiguous()
                vr = v.repeat_interleave(rep, dim=1).contiguous()
                o2, l2 = _run(orc, q, kr, vr, dtype, 0.6, causal=causal)
                assert np.array_equal(o, o2) and np.array_equal(lse, l2)
            ref = F.scaled_dot_product_attention(q.double(), k.double(), v.double(),
                                                 scale=0.6, enable_gqa=True)
            o, _ = _run(orc, q, k, v, dtype, 0.6)
            assert np.allclose(o, ref.numpy(), rtol=0, atol=1e-10)


def pin_single_key_any_length(orc):
    """Nk = 1: every row (non-causal) is v_0 exactly, whatever Nq."""
    for dtype in DTYPES:
        q = _rand16((1, 3, 7, 8), dtype, 171)
        k = _rand16((1, 3, 1, 8), dtype, 172)
        v = _rand16((1, 3, 1, 8), dtype, 173)
        o, _ = _run(orc, q, k, v, dtype, 1.3)
        assert np.array_equal(o, np.broadcast_to(_f64(v), o.shape))


# --------------------------------------------------------------------------
# INT8 key/value cache: the reading spelled out in oracle/attn_ref.c (int8
# codes with per-channel scales; query rows quantized in binary32 after the
# key scales are folded in).


def pin_int8_query_codes_golden(orc):
    """Hand-derived codes and row scales (tests/golden/int8_query_codes.json):
    ties to even, key scales folded into the row, a zero row, a negative
    extreme, and a row where binary32 rounding gives a different code than
    exact rationals would."""
    with open(os.path.join(GOLDEN, "int8_query_codes.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q = _t16(c["q"], c["dtype"])
        codes, sq = orc.quantize_q(bits(q)[None, :], np.asarray(c["ks"], np.float32), c["dtype"])
        assert codes[0].tolist() == c["codes"], (c["name"], codes[0].tolist())
        assert int(sq.view(np.uint32)[0]) == int(c["sq_bits"], 16), (c["name"], hex(sq.view(np.uint32)[0]))


def _int8_cache(B, Hkv, Nk, d, seed, pow2_scales=False):
    """Random int8 codes [B, Hkv, Nk, d] and float32 scales [B, Hkv, d]."""
    rng = np.random.default_rng(seed)
    kq = rng.integers(-127, 128, size=(B, Hkv, Nk, d)).astype(np.int8)
    vq = rng.integers(-127, 128, size=(B, Hkv, Nk, d)).astype(np.int8)
    if pow2_scales:
        ks = np.exp2(-rng.integers(2, 7, size=(B, Hkv, d))).astype(np.float32)
        vs = np.exp2(-rng.integers(2, 7, size=(B, Hkv, d))).astype(np.float32)
    else:
        ks = rng.uniform(0.01, 0.05, size=(B, Hkv, d)).astype(np.float32)
        vs = rng.uniform(0.01, 0.05, size=(B, Hkv, d)).astype(np.float32)
    return kq, ks, vq, vs


def pin_int8_reduces_to_dequantized_attention(orc):
    """A query row whose key-scaled values u = q*ks are integers with max |u| =
    127 quantizes to itself (codes u, sq = 1), so its logits are exactly those
    of plain attention on q and the dequantized k = ks*kq; with v = vs*vq the
    whole result must equal the (separately pinned) 16-bit oracle on q,
    ks*kq, vs*vq.  Power-of-two scales keep every value exact in 16 bits."""
    rng = np.random.default_rng(7)
    for dtype in DTYPES:
        for causal in (False, True):
            B, Hq, Hkv, Nq, Nk, d = 2, 4, 2, 5, 7, 16
            kq, ks, vq, vs = _int8_cache(B, Hkv, Nk, d, seed=11, pow2_scales=True)
            u = rng.integers(-126, 127, size=(B, Hq, Nq, d)).astype(np.float64)
            u[..., 3] = np.where(rng.random((B, Hq, Nq)) < 0.5, 127.0, -127.0)
            group = Hq // Hkv
            ks_q = np.repeat(ks, group, axis=1)[:, :, None, :].astype(np.float64)
            q = _t16(u / ks_q, dtype)
            kd = _t16(ks[:, :, None, :].astype(np.float64) * kq, dtype)
            vd = _t16(vs[:, :, None, :].astype(np.float64) * vq, dtype)
            o8, l8 = orc.attention_kv_int8(bits(q), kq, ks, vq, vs, dtype, 0.125, causal=causal)
            o, lse = _run(orc, q, kd, vd, dtype, 0.125, causal=causal)
            np.testing.assert_allclose(o8, o, rtol=1e-13, atol=1e-13)
            np.testing.assert_allclose(l8, lse, rtol=1e-13, atol=0)


def pin_int8_zero_query_is_uniform(orc):
    """A zero query row has codes 0 and sq = 0, so every logit is 0: O is the
    mean of the dequantized values the row sees and lse = ln(keys seen)."""
    B, Hq, Hkv, Nq, Nk, d = 1, 2, 1, 3, 6, 8
    kq, ks, vq, vs = _int8_cache(B, Hkv, Nk, d, seed=5)
    q = _t16(np.zeros((B, Hq, Nq, d)), "bf16")
    for causal in (False, True):
        o, lse = orc.attention_kv_int8(bits(q), kq, ks, vq, vs, "bf16", 0.3, causal=causal)
        vdq = vs[:, :, None, :].astype(np.float64) * vq
        for i in range(Nq):
            n = _visible(i, Nq, Nk) if causal else Nk
            want = vdq[0, 0, :n].mean(axis=0)
            np.testing.assert_allclose(o[0, :, i], np.broadcast_to(want, (Hq, d)), rtol=1e-12, atol=1e-15)
            np.testing.assert_allclose(lse[0, :, i], math.log(n), rtol=1e-14)


def _int8_brute_row(q16, ksh, kqh, vsh, vqh, n, scale):
    """The scheme term by term: numpy binary32 for the query quantization,
    Python integers for the code dot products, math.exp / math.fsum after."""
    u = (q16.astype(np.float32) * ksh).astype(np.float32)
    amax = np.float32(np.max(np.abs(u)))
    if amax > 0:
        inv = np.float32(np.float32(127.0) / amax)
        codes = np.clip(np.rint((u * inv).astype(np.float32)), -127, 127).astype(np.int64)
        sq = float(np.float32(amax / np.float32(127.0)))
    else:
        codes = np.zeros(u.shape, np.int64)
        sq = 0.0
    d = u.size
    if n == 0:
        return [0.0] * d, -math.inf
    s = [scale * sq * float(sum(int(codes[c]) * int(kqh[j, c]) for c in range(d))) for j in range(n)]
    m = max(s)
    w = [math.exp(x - m) for x in s]
    l = math.fsum(w)
    o = [math.fsum(w[j] * float(vsh[c]) * float(vqh[j, c]) for j in range(n)) / l for c in range(d)]
    return o, m + math.log(l)


def pin_int8_brute_force(orc):
    """Tiny random problems (grouped heads, both masks, Nq != Nk) against the
    term-by-term evaluation above."""
    for dtype, causal, (B, Hq, Hkv, Nq, Nk, d) in (
            ("bf16", False, (1, 4, 2, 3, 5, 8)), ("fp16", True, (2, 2, 1, 4, 3, 16)),
            ("bf16", True, (1, 3, 3, 2, 6, 4))):
        kq, ks, vq, vs = _int8_cache(B, Hkv, Nk, d, seed=Nk + d)
        q = _rand16((B, Hq, Nq, d), dtype, seed=d)
        o, lse = orc.attention_kv_int8(bits(q), kq, ks, vq, vs, dtype, 0.7, causal=causal)
        qn = _f64(q)
        group = Hq // Hkv
        for b in range(B):
            for h in range(Hq):
                g = h // group
                for i in range(Nq):
                    n = _visible(i, Nq, Nk) if causal else Nk
                    ob, lb = _int8_brute_row(qn[b, h, i], ks[b, g], kq[b, g], vs[b, g], vq[b, g], n, 0.7)
                    np.testing.assert_allclose(o[b, h, i], ob, rtol=1e-12, atol=1e-14)
                    if n:
                        assert abs(lse[b, h, i] - lb) <= 1e-12 * max(1.0, abs(lb))
                    else:
                        assert lse[b, h, i] == -math.inf


# --------------------------------------------------------------------------
# FP8 key/value cache: the same scheme with OCP E4M3 codes (oracle/attn_ref.c).


def _golden_value(txt):
    """'2^-9', '7*2^-9', '-0', 'nan', '1.125' -> float."""
    if txt == "nan":
        return math.nan
    sign = -1.0 if txt.startswith("-") else 1.0
    body = txt.lstrip("-")
    val = 1.0
    for part in body.split("*"):
        val *= 2.0 ** float(part[2:]) if part.startswith("2^") else float(part)
    return math.copysign(val, sign)


def pin_e4m3_codes_golden(orc):
    """Hand-derived E4M3 values and roundings (tests/golden/e4m3_codes.json):
    subnormals, the bias, the largest finite value, NaN, signed zero, ties to
    even in the normal and subnormal ranges, and saturation."""
    with open(os.path.join(GOLDEN, "e4m3_codes.json")) as f:
        g = json.load(f)
    codes = np.array([int(e["code"], 16) for e in g["decode"]], np.uint8)
    got = orc.e4m3_decode(codes)
    for e, v in zip(g["decode"], got):
        want = _golden_value(e["value"])
        if math.isnan(want):
            assert math.isnan(v), e
        else:
            assert v == want and math.copysign(1.0, v) == math.copysign(1.0, want), (e, v)
    xs = np.array([_golden_value(e["x"]) for e in g["round"]], np.float32)
    got = orc.e4m3_round(xs)
    for e, c in zip(g["round"], got):
        assert int(c) == int(e["code"], 16), (e, hex(int(c)))


def pin_e4m3_matches_torch(orc):
    """Every code decodes as torch.float8_e4m3fn does; rounding matches
    torch's conversion on every value within +-448: random values, every
    representable value, and every midpoint between neighbours (the ties)."""
    codes = np.arange(256, dtype=np.uint8)
    mine = orc.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok]) and np.array_equal(np.signbit(mine[ok]), np.signbit(ref[ok]))
    vals = np.unique(ref[ok & (ref >= 0)])
    mids = (vals[1:] + vals[:-1]) / 2
    rng = np.random.default_rng(3)
    rnd = np.clip(rng.standard_normal(20000) * 40, -448, 448)
    xs = np.concatenate([vals, -vals, mids, -mids, rnd, rnd * 1e-3]).astype(np.float32)
    assert np.all(np.abs(xs) <= 448)
    got = orc.e4m3_round(xs)
    want = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want), np.flatnonzero(got != want)[:5]


def pin_fp8_query_codes_golden(orc):
    """Hand-derived E4M3 query codes and row scales
    (tests/golden/fp8_query_codes.json)."""
    with open(os.path.join(GOLDEN, "fp8_query_codes.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q = _t16(c["q"], c["dtype"])
        codes, sq = orc.quantize_q_fp8(bits(q)[None, :], np.asarray(c["ks"], np.float32), c["dtype"])
        assert codes[0].tolist() == [int(x, 16) for x in c["codes"]], (c["name"], [hex(x) for x in codes[0]])
        assert int(sq.view(np.uint32)[0]) == int(c["sq_bits"], 16), (c["name"], hex(sq.view(np.uint32)[0]))


def _fp8_cache(B, Hkv, Nk, d, seed, pow2_scales=False):
    """Random finite E4M3 codes [B, Hkv, Nk, d] (no NaN) and float32 scales."""
    rng = np.random.default_rng(seed)
    def codes():
        c = rng.integers(0, 256, size=(B, Hkv, Nk, d)).astype(np.uint8)
        return np.where((c & 0x7F) == 0x7F, c ^ 0x01, c).astype(np.uint8)
    kf, vf = codes(), codes()
    if pow2_scales:
        ks = np.exp2(-rng.integers(2, 7, size=(B, Hkv, d))).astype(np.float32)
        vs = np.exp2(-rng.integers(2, 7, size=(B, Hkv, d))).astype(np.float32)
    else:
        ks = rng.uniform(0.005, 0.02, size=(B, Hkv, d)).astype(np.float32)
        vs = rng.uniform(0.005, 0.02, size=(B, Hkv, d)).astype(np.float32)
    return kf, ks, vf, vs


def _e4m3_torch(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()


def pin_fp8_reduces_to_dequantized_attention(orc):
    """A query row whose key-scaled values u = q*ks are E4M3 values with max
    |u| = 448 quantizes to itself (448/amax = 1, sq = 1), so its logits are
    exactly those of plain attention on q and the dequantized k = ks*e4m3(kf);
    with v = vs*e4m3(vf) the whole result must equal the 16-bit oracle on
    those values.  Power-of-two scales keep every value exact in 16 bits."""
    rng = np.random.default_rng(9)
    for dtype in DTYPES:
        for causal in (False, True):
            B, Hq, Hkv, Nq, Nk, d = 2, 4, 2, 5, 7, 16
            kf, ks, vf, vs = _fp8_cache(B, Hkv, Nk, d, seed=13, pow2_scales=True)
            # query values: E4M3 values of at most 2^-2 .. 448 in magnitude (exact in fp16 after /ks)
            qc = rng.integers(0x10, 0x7F, size=(B, Hq, Nq, d)).astype(np.uint8) | \
                (rng.integers(0, 2, size=(B, Hq, Nq, d)).astype(np.uint8) << 7)
            u = _e4m3_torch(qc)
            u[..., 5] = np.where(rng.random((B, Hq, Nq)) < 0.5, 448.0, -448.0)
            group = Hq // Hkv
            ks_q = np.repeat(ks, group, axis=1)[:, :, None, :].astype(np.float64)
            q = _t16(u / ks_q, dtype)
            kd = _t16(ks[:, :, None, :].astype(np.float64) * _e4m3_torch(kf), dtype)
            vd = _t16(vs[:, :, None, :].astype(np.float64) * _e4m3_torch(vf), dtype)
            o8, l8 = orc.attention_kv_fp8(bits(q), kf, ks, vf, vs, dtype, 0.01, causal=causal)
            o, lse = _run(orc, q, kd, vd, dtype, 0.01, causal=causal)
            np.testing.assert_allclose(o8, o, rtol=1e-13, atol=1e-13)
            np.testing.assert_allclose(l8, lse, rtol=1e-13, atol=0)


def pin_fp8_zero_query_is_uniform(orc):
    """A zero query row has codes 0 and sq = 0: O is the mean of the
    dequantized values the row sees and lse = ln(keys seen)."""
    B, Hq, Hkv, Nq, Nk, d = 1, 2, 1, 3, 6, 8
    kf, ks, vf, vs = _fp8_cache(B, Hkv, Nk, d, seed=6)
    q = _t16(np.zeros((B, Hq, Nq, d)), "bf16")
    for causal in (False, True):
        o, lse = orc.attention_kv_fp8(bits(q), kf, ks, vf, vs, "bf16", 0.3, causal=causal)
        vdq = vs[:, :, None, :].astype(np.float64) * _e4m3_torch(vf)
        for i in range(Nq):
            n = _visible(i, Nq, Nk) if causal else Nk
            want = vdq[0, 0, :n].mean(axis=0)
            np.testing.assert_allclose(o[0, :, i], np.broadcast_to(want, (Hq, d)), rtol=1e-12, atol=1e-15)
            np.testing.assert_allclose(lse[0, :, i], math.log(n), rtol=1e-14)


def _fp8_brute_row(q16, ksh, kfh, vsh, vfh, n, scale):
    """The scheme term by term: numpy binary32 for the query scaling, torch's
    float8_e4m3fn conversion for its rounding, exact Fractions for the code
    dot products, math.exp / math.fsum after."""
    u = (q16.astype(np.float32) * ksh).astype(np.float32)
    amax = np.float32(np.max(np.abs(u)))
    d = u.size
    if amax > 0:
        to448 = np.float32(np.float32(448.0) / amax)
        t = (u * to448).astype(np.float32)
        qv = torch.from_numpy(t).to(torch.float8_e4m3fn).double().numpy()
        sq = float(np.float32(amax / np.float32(448.0)))
    else:
        qv = np.zeros(d)
        sq = 0.0
    if n == 0:
        return [0.0] * d, -math.inf
    kv = _e4m3_torch(kfh)
    s = [scale * sq * float(sum(Fraction(qv[c]) * Fraction(kv[j, c]) for c in range(d))) for j in range(n)]
    m = max(s)
    w = [math.exp(x - m) for x in s]
    l = math.fsum(w)
    vv = _e4m3_torch(vfh)
    o = [math.fsum(w[j] * float(vsh[c]) * vv[j, c] for j in range(n)) / l for c in range(d)]
    return o, m + math.log(l)


def pin_fp8_brute_force(orc):
    """Tiny random problems (grouped heads, both masks, Nq != Nk) against the
    term-by-term evaluation above."""
    for dtype, causal, (B, Hq, Hkv, Nq, Nk, d) in (
            ("bf16", False, (1, 4, 2, 3, 5, 8)), ("fp16", True, (2, 2, 1, 4, 3, 16)),
            ("bf16", True, (1, 3, 3, 2, 6, 4))):
        kf, ks, vf, vs = _fp8_cache(B, Hkv, Nk, d, seed=Nk + 2 * d)
        q = _rand16((B, Hq, Nq, d), dtype, seed=d + 1)
        o, lse = orc.attention_kv_fp8(bits(q), kf, ks, vf, vs, dtype, 0.7, causal=causal)
        qn = _f64(q)
        group = Hq // Hkv
        for b in range(B):
            for h in range(Hq):
                g = h // group
                for i in range(Nq):
                    n = _visible(i, Nq, Nk) if causal else Nk
                    ob, lb = _fp8_brute_row(qn[b, h, i], ks[b, g], kf[b, g], vs[b, g], vf[b, g], n, 0.7)
                    np.testing.assert_allclose(o[b, h, i], ob, rtol=1e-12, atol=1e-14)
                    if n:
                        assert abs(lse[b, h, i] - lb) <= 1e-12 * max(1.0, abs(lb))
                    else:
                        assert lse[b, h, i] == -math.inf


def pin_rows_subset_with_every_option(orc):
    """rows= picks exactly the full result's rows with every option at once
    (causal mask, grouped heads, Nq != Nk, both dtypes, and the INT8 cache):
    the sampled comparisons of the GPU tests rest on it.  A row's position
    within its head, which the mask needs, comes from its flat id, not from
    its place in the sample."""
    rng = np.random.default_rng(7)
    B, Hq, Hkv, Nq, Nk, d = 2, 4, 2, 37, 53, 8
    flat = B * Hq * Nq
    rows = rng.choice(flat, size=41, replace=False)
    for causal in (False, True):
        for dtype in DTYPES:
            q = _rand16((B, Hq, Nq, d), dtype, 150)
            k = _rand16((B, Hkv, Nk, d), dtype, 151)
            v = _rand16((B, Hkv, Nk, d), dtype, 152)
            o, lse = _run(orc, q, k, v, dtype, 0.4, causal=causal)
            orow, lrow = _run(orc, q, k, v, dtype, 0.4, causal=causal, rows=rows)
            assert np.array_equal(orow, o.reshape(-1, d)[rows]), (causal, dtype)
            assert np.array_equal(lrow, lse.reshape(-1)[rows]), (causal, dtype)
        q = _rand16((B, Hq, Nq, 128), "bf16", 153)
        kq, ks, vq, vs = _int8_cache(B, Hkv, Nk, 128, 154)
        o, lse = orc.attention_kv_int8(bits(q), kq, ks, vq, vs, "bf16", 0.1, causal=causal)
        orow, lrow = orc.attention_kv_int8(bits(q), kq, ks, vq, vs, "bf16", 0.1,
                                           causal=causal, rows=rows)
        assert np.array_equal(orow, o.reshape(-1, 128)[rows]), causal
        assert np.array_equal(lrow, lse.reshape(-1)[rows]), causal


ALL_PINS = [
    pin_decode_every_pattern,
    pin_worked_examples,
    pin_brute_force_tiny,
    pin_torch_fp64,
    pin_identity_values_are_probabilities,
    pin_constant_values,
    pin_uniform_attention,
    pin_single_key,
    pin_two_keys,
    pin_logit_shift,
    pin_permutations,
    pin_value_linearity,
    pin_head_independence,
    pin_extreme_logits,
    pin_causal_is_prefix_attention,
    pin_causal_first_row,
    pin_causal_and_lengths_torch,
    pin_causal_brute_force,
    pin_grouped_heads_are_repeated_heads,
    pin_single_key_any_length,
    pin_int8_query_codes_golden,
    pin_int8_reduces_to_dequantized_attention,
    pin_int8_zero_query_is_uniform,
    pin_int8_brute_force,
    pin_e4m3_codes_golden,
    pin_e4m3_matches_torch,
    pin_fp8_query_codes_golden,
    pin_fp8_reduces_to_dequantized_attention,
    pin_fp8_zero_query_is_uniform,
    pin_fp8_brute_force,
    pin_rows_subset_with_every_option,
]
