"""Seeded synthetic inputs for the attention forward pass.

This module holds input generation and bit-level marshalling only, none of the
attention arithmetic.  Tests hand the same tensors to the GPU path and to the
fp64 oracle; the benchmark uses it to build its resident inputs.

Workloads follow the problem shape of the "Flash Attention 2 from scratch on
Ampere" Part 1 page (Kernel Specification: head dimension 128, equal lengths,
16-bit inputs; Performance: sequence length 4096 as the focus and a harmonic
mean over 512..16384).  Batch and head counts are not given there; the sizes
below fix them.  No dataset is involved: every tensor is drawn from a seeded
generator.

Recipe (one ``torch.Generator`` on the CPU, seeded, drawing Q then K then V in
fp32, rounded to the 16-bit dtype by round-to-nearest-even):
  * "normal": Q, K, V i.i.d. N(0, 1).
  * "stress": Q, K i.i.d. N(0, 1), Q then multiplied by 4 (a power of two, so
    exact after rounding), V i.i.d. U(-1, 1) drawn as 2*rand - 1.  Logits have
    standard deviation about 4, which exercises the running-max rescale.
"""
import math
from dataclasses import dataclass

import numpy as np
import torch

_TORCH_DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16}


@dataclass(frozen=True)
class Workload:
    """H query heads of N rows; Hkv key/value heads of Nk rows (default H, N)."""
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str = "bf16"
    dist: str = "normal"
    Hkv: int = 0
    Nk: int = 0
    causal: bool = False
    kv_int8: bool = False   # keys/values as an INT8 cache (int8 codes, fp32 channel scales)
    kv_fp8: bool = False    # keys/values as an FP8 cache (E4M3 codes, fp32 channel scales)
    split: bool = False     # run with key splits (fa2_fwd_split, split count chosen by the library)

    @property
    def quantized(self) -> bool:
        """Keys and values arrive as 8-bit codes with channel scales."""
        return self.kv_int8 or self.kv_fp8

    @property
    def kv_heads(self) -> int:
        return self.Hkv or self.H

    @property
    def keys(self) -> int:
        return self.Nk or self.N

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def visible_pairs(self) -> int:
        """(query row, key) pairs that enter the softmax, per (b, h)."""
        nq, nk = self.N, self.keys
        if not self.causal:
            return nq * nk
        # row i sees min(nk, max(0, i + 1 + nk - nq)) keys
        total = 0
        first = max(0, nq - nk)           # rows before this see nothing
        full = max(first, nq)             # rows never exceed nk keys here
        for i in range(first, full):
            total += min(nk, i + 1 + nk - nq)
        return total

    @property
    def flops(self) -> int:
        """Two contractions over the visible pairs: 4 * B * H * pairs * d
        (4 * B * H * N^2 * d without a mask)."""
        return 4 * self.B * self.H * self.visible_pairs * self.d

    @property
    def algo_bytes(self) -> int:
        """Q, K, V read once and O written once (16-bit), LSE written (fp32)."""
        q = self.B * self.H * self.N * self.d
        kv = self.B * self.kv_heads * self.keys * self.d
        lse = self.B * self.H * self.N * 4
        if self.quantized:  # 1-byte codes plus two fp32 scales per K/V channel
            return 2 * 2 * q + 2 * kv + 2 * 4 * self.B * self.kv_heads * self.d + lse
        return 2 * (2 * q + 2 * kv) + lse

    def describe(self) -> dict:
        out = {"workload": self.name, "B": self.B, "H": self.H, "N": self.N,
               "d": self.d, "dtype": self.dtype, "inputs": self.dist,
               "causal": self.causal, "scale": "1/sqrt(d)"}
        if self.kv_heads != self.H:
            out["Hkv"] = self.kv_heads
        if self.keys != self.N:
            out["Nk"] = self.keys
        if self.kv_int8:
            out["kv"] = "int8 codes, fp32 per-channel scales"
        if self.kv_fp8:
            out["kv"] = "FP8 E4M3 codes, fp32 per-channel scales"
        if self.split:
            out["key_splits"] = "chosen by the library (fa2_fwd_split, splits = 0)"
        return out


def _sweep():
    out = {}
    for n, b in ((512, 32), (1024, 16), (2048, 8), (4096, 4), (8192, 2),
                 (16384, 1)):
        out["sweep_n%d" % n] = Workload("sweep_n%d" % n, b, 16, n, 128, "fp16")
    return out


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 256, 128, "bf16"),
    "stress": Workload("stress", 8, 16, 1024, 128, "bf16", "stress"),
    "headline": Workload("headline", 4, 16, 4096, 128, "bf16"),
    **_sweep(),
    "d64": Workload("d64", 4, 16, 4096, 64, "bf16"),
    "d256": Workload("d256", 4, 8, 4096, 256, "bf16"),
    # the rows the Kernel Specification section leaves out
    "causal": Workload("causal", 4, 16, 4096, 128, "bf16", causal=True),
    "gqa": Workload("gqa", 4, 16, 4096, 128, "bf16", Hkv=2),
    "kv_cache": Workload("kv_cache", 4, 16, 1024, 128, "bf16", Hkv=4, Nk=8192, causal=True),
    # a 64-row prefill chunk against a 4096-key cache, 4 query heads per K/V
    # head: the rows of a K/V head's query heads share workgroups
    "gqa_chunk": Workload("gqa_chunk", 16, 32, 64, 128, "bf16", Hkv=8, Nk=4096, causal=True),
    # the headline shape over an INT8 key/value cache
    "int8_kv": Workload("int8_kv", 4, 16, 4096, 128, "bf16", kv_int8=True),
    "int8_kv_causal": Workload("int8_kv_causal", 4, 16, 4096, 128, "bf16", causal=True,
                               kv_int8=True),
    # the same over an FP8 (E4M3) key/value cache
    "fp8_kv": Workload("fp8_kv", 4, 16, 4096, 128, "bf16", kv_fp8=True),
    "fp8_kv_causal": Workload("fp8_kv_causal", 4, 16, 4096, 128, "bf16", causal=True,
                              kv_fp8=True),
    # decoding: one new query row per head against a long cache, with key
    # splits (32 query heads on 8 K/V heads)
    "decode": Workload("decode", 4, 32, 1, 128, "bf16", Hkv=8, Nk=32768, causal=True,
                       split=True),
    "decode_long": Workload("decode_long", 1, 32, 1, 128, "bf16", Hkv=8, Nk=131072,
                            causal=True, split=True),
    # the same decoding step over INT8 and FP8 caches
    "decode_int8": Workload("decode_int8", 4, 32, 1, 128, "bf16", Hkv=8, Nk=32768, causal=True,
                            kv_int8=True, split=True),
    "decode_fp8": Workload("decode_fp8", 4, 32, 1, 128, "bf16", Hkv=8, Nk=32768, causal=True,
                           kv_fp8=True, split=True),
}


def torch_dtype(dtype: str) -> torch.dtype:
    return _TORCH_DTYPES[dtype]


def make_inputs(B, H, N, d, dtype="bf16", dist="normal", seed=0, Hkv=None, Nk=None):
    """Seeded CPU tensors q [B, H, N, d] and k, v [B, Hkv, Nk, d] (default Hkv =
    H, Nk = N) in the 16-bit dtype."""
    g = torch.Generator().manual_seed(seed)
    shape = (B, H, N, d)
    kv_shape = (B, Hkv or H, Nk if Nk is not None else N, d)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(kv_shape, generator=g, dtype=torch.float32)
    if dist == "normal":
        v = torch.randn(kv_shape, generator=g, dtype=torch.float32)
    elif dist == "stress":
        q.mul_(4.0)
        v = torch.rand(kv_shape, generator=g, dtype=torch.float32).mul_(2.0).sub_(1.0)
    else:
        raise ValueError("unknown input distribution %r" % dist)
    t = _TORCH_DTYPES[dtype]
    return q.to(t), k.to(t), v.to(t)


def make_inputs_kv_int8(B, Hq, Hkv, Nq, Nk, d, dtype="bf16", seed=0):
    """Seeded CPU inputs for attention over an INT8 key/value cache: q
    [B, Hq, Nq, d] in the 16-bit dtype (standard normal), kq and vq
    [B, Hkv, Nk, d] int8 codes (a standard normal times 127/4.5, rounded and
    clipped to [-127, 127], the shape of a per-channel symmetric cache of
    normal data), and ks, vs [B, Hkv, d] float32 per-channel scales
    (4.5/127 times a factor drawn uniformly from [0.5, 1.5))."""
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, Hq, Nq, d), generator=g, dtype=torch.float32)
    codes = []
    for _ in range(2):
        c = torch.randn((B, Hkv, Nk, d), generator=g, dtype=torch.float32) * (127.0 / 4.5)
        codes.append(c.round().clamp(-127, 127).to(torch.int8))
    scales = []
    for _ in range(2):
        u = torch.rand((B, Hkv, d), generator=g, dtype=torch.float32)
        scales.append(((u + 0.5) * (4.5 / 127.0)).to(torch.float32))
    return q.to(_TORCH_DTYPES[dtype]), codes[0], scales[0], codes[1], scales[1]


def make_inputs_kv_fp8(B, Hq, Hkv, Nq, Nk, d, dtype="bf16", seed=0):
    """Seeded CPU inputs for attention over an FP8 key/value cache: q
    [B, Hq, Nq, d] in the 16-bit dtype (standard normal), kq and vq
    [B, Hkv, Nk, d] uint8 OCP E4M3 codes of a standard normal times 448/4.5,
    clipped to [-448, 448] (torch's float8_e4m3fn conversion; the shape of a
    per-channel symmetric FP8 cache of normal data, never a NaN code), and
    ks, vs [B, Hkv, d] float32 per-channel scales (4.5/448 times a factor
    drawn uniformly from [0.5, 1.5))."""
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, Hq, Nq, d), generator=g, dtype=torch.float32)
    codes = []
    for _ in range(2):
        c = torch.randn((B, Hkv, Nk, d), generator=g, dtype=torch.float32) * (448.0 / 4.5)
        codes.append(c.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8))
    scales = []
    for _ in range(2):
        u = torch.rand((B, Hkv, d), generator=g, dtype=torch.float32)
        scales.append(((u + 0.5) * (4.5 / 448.0)).to(torch.float32))
    return q.to(_TORCH_DTYPES[dtype]), codes[0], scales[0], codes[1], scales[1]


def workload_inputs(w: Workload, seed=0):
    """(q, k, v), or (q, kq, ks, vq, vs) for a quantized cache workload."""
    if w.kv_int8:
        return make_inputs_kv_int8(w.B, w.H, w.kv_heads, w.N, w.keys, w.d, w.dtype, seed)
    if w.kv_fp8:
        return make_inputs_kv_fp8(w.B, w.H, w.kv_heads, w.N, w.keys, w.d, w.dtype, seed)
    return make_inputs(w.B, w.H, w.N, w.d, w.dtype, w.dist, seed, w.kv_heads, w.keys)


def bits(t: torch.Tensor) -> np.ndarray:
    """The raw 16-bit patterns of a bf16/fp16 tensor, as a numpy uint16 array."""
    if t.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("expected a 16-bit float tensor, got %s" % t.dtype)
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bits(b: np.ndarray, dtype: str) -> torch.Tensor:
    """Inverse of bits(): a CPU tensor of the 16-bit dtype holding patterns b."""
    arr = np.ascontiguousarray(b, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(arr.copy()).view(_TORCH_DTYPES[dtype])
