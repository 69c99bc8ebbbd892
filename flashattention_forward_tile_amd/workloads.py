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
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str = "bf16"
    dist: str = "normal"

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def flops(self) -> int:
        """Two N x N x d contractions per (b, h): 4 * B * H * N^2 * d."""
        return 4 * self.B * self.H * self.N * self.N * self.d

    @property
    def algo_bytes(self) -> int:
        """Q, K, V read once and O written once (16-bit), LSE written (fp32)."""
        elems = self.B * self.H * self.N * self.d
        return 4 * elems * 2 + self.B * self.H * self.N * 4

    def describe(self) -> dict:
        return {"workload": self.name, "B": self.B, "H": self.H, "N": self.N,
                "d": self.d, "dtype": self.dtype, "inputs": self.dist,
                "causal": False, "scale": "1/sqrt(d)"}


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
}


def torch_dtype(dtype: str) -> torch.dtype:
    return _TORCH_DTYPES[dtype]


def make_inputs(B, H, N, d, dtype="bf16", dist="normal", seed=0):
    """Seeded CPU tensors (q, k, v) of shape [B, H, N, d] in the 16-bit dtype."""
    g = torch.Generator().manual_seed(seed)
    shape = (B, H, N, d)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    if dist == "normal":
        v = torch.randn(shape, generator=g, dtype=torch.float32)
    elif dist == "stress":
        q.mul_(4.0)
        v = torch.rand(shape, generator=g, dtype=torch.float32).mul_(2.0).sub_(1.0)
    else:
        raise ValueError("unknown input distribution %r" % dist)
    t = _TORCH_DTYPES[dtype]
    return q.to(t), k.to(t), v.to(t)


def workload_inputs(w: Workload, seed=0):
    return make_inputs(w.B, w.H, w.N, w.d, w.dtype, w.dist, seed)


def bits(t: torch.Tensor) -> np.ndarray:
    """The raw 16-bit patterns of a bf16/fp16 tensor, as a numpy uint16 array."""
    if t.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("expected a 16-bit float tensor, got %s" % t.dtype)
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bits(b: np.ndarray, dtype: str) -> torch.Tensor:
    """Inverse of bits(): a CPU tensor of the 16-bit dtype holding patterns b."""
    arr = np.ascontiguousarray(b, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(arr.copy()).view(_TORCH_DTYPES[dtype])
