"""fp64 CPU oracle for non-causal scaled dot-product attention.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the GPU path and never calls it; the GPU path never calls it either.

It computes the plain definition (scaled dot-product attention from "Attention
Is All You Need", the operation that the FlashAttention-2 forward pass of the
Hopper/CUTLASS case-study abstract and of the "Flash Attention 2 from scratch on
Ampere" series fuses): for each (b, h, i), over the keys j row i may see

    s_j = scale * <q_i, k_j>,  m = max_j s_j,  l = sum_j exp(s_j - m),
    O_i = sum_j exp(s_j - m) v_j / l,  lse_i = m + ln l,

in fp64 from the exact values of the 16-bit inputs (``attn_ref.c``).  Options:
causal masking (row i sees keys j <= i + Nk - Nq), unequal query/key lengths,
and grouped key/value heads.  Inputs
are passed as raw 16-bit patterns (numpy ``uint16``) with a dtype tag, so the
oracle sees bit for bit what the GPU sees.
"""
import ctypes
import os

import numpy as np

from . import build as _build

BF16 = 0
FP16 = 1
_DTYPES = {"bf16": BF16, "bfloat16": BF16, "fp16": FP16, "float16": FP16,
           BF16: BF16, FP16: FP16}


def _ptr(a, ct):
    return a.ctypes.data_as(ctypes.POINTER(ct))


class Oracle:
    """ctypes view of one compiled copy of attn_ref.c."""

    def __init__(self, lib_path=None):
        if lib_path is None:
            if not os.path.exists(_build.LIB):
                _build.build()
            lib_path = _build.LIB
        lib = ctypes.CDLL(lib_path)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        f64p = ctypes.POINTER(ctypes.c_double)
        i64p = ctypes.POINTER(ctypes.c_int64)
        lib.oracle_attn_rows.argtypes = [
            u16p, u16p, u16p, ctypes.c_int,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_double, i64p, ctypes.c_int64, f64p, f64p, ctypes.c_int]
        lib.oracle_attn_rows.restype = ctypes.c_int
        lib.oracle_attn_general.argtypes = [
            u16p, u16p, u16p, ctypes.c_int,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_double, ctypes.c_int,
            i64p, ctypes.c_int64, f64p, f64p, ctypes.c_int]
        lib.oracle_attn_general.restype = ctypes.c_int
        lib.oracle_decode.argtypes = [u16p, ctypes.c_int64, ctypes.c_int, f64p]
        lib.oracle_decode.restype = ctypes.c_int
        lib.oracle_host_threads.argtypes = []
        lib.oracle_host_threads.restype = ctypes.c_int
        self.lib = lib
        self.path = lib_path

    def host_threads(self) -> int:
        """Number of host cores in this process's affinity mask."""
        return int(self.lib.oracle_host_threads())

    def decode(self, bits, dtype) -> np.ndarray:
        """Exact fp64 value of each 16-bit pattern (bf16 or IEEE binary16)."""
        bits = np.ascontiguousarray(bits, dtype=np.uint16)
        out = np.empty(bits.shape, dtype=np.float64)
        rc = self.lib.oracle_decode(_ptr(bits, ctypes.c_uint16), bits.size,
                                    _DTYPES[dtype], _ptr(out, ctypes.c_double))
        if rc != 0:
            raise ValueError("oracle_decode failed (%d)" % rc)
        return out

    def attention(self, q_bits, k_bits, v_bits, dtype, scale, rows=None,
                  nthreads=0, causal=False):
        """fp64 attention forward.

        q_bits: uint16 [B, Hq, Nq, d]; k_bits, v_bits: uint16 [B, Hkv, Nk, d]
        (16-bit patterns), Hq a multiple of Hkv (query head h reads key/value
        head h // (Hq // Hkv)); dtype: "bf16" or "fp16"; scale: any real.
        causal: row i sees keys j <= i + Nk - Nq (a row that sees none gets
        O = 0 and lse = -inf).
        rows: None for every row (O shaped [B, Hq, Nq, d], lse [B, Hq, Nq]), or
        a 1-D array of distinct flat row ids (b*Hq + h)*Nq + i in any order (O
        shaped [len, d], lse [len]).  nthreads <= 0 uses every core in the
        affinity mask.  Returns (O, lse) as fp64 numpy arrays.
        """
        q = np.ascontiguousarray(q_bits, dtype=np.uint16)
        k = np.ascontiguousarray(k_bits, dtype=np.uint16)
        v = np.ascontiguousarray(v_bits, dtype=np.uint16)
        if q.ndim != 4 or k.ndim != 4 or k.shape != v.shape:
            raise ValueError("q must be [B, Hq, Nq, d], k and v one [B, Hkv, Nk, d] shape")
        B, Hq, Nq, d = q.shape
        if k.shape[0] != B or k.shape[3] != d or k.shape[1] < 1 or Hq % k.shape[1]:
            raise ValueError("k/v batch and head dim must match q, Hq a multiple of Hkv")
        if rows is None:
            o = np.empty((B, Hq, Nq, d), dtype=np.float64)
            lse = np.empty((B, Hq, Nq), dtype=np.float64)
            self._run(q, k, v, dtype, scale, causal, None, o, lse, nthreads)
            return o, lse
        rows = np.asarray(rows, dtype=np.int64).ravel()
        order = np.argsort(rows, kind="stable")
        srt = np.ascontiguousarray(rows[order])
        if srt.size and np.any(np.diff(srt) <= 0):
            raise ValueError("rows must not repeat")
        o_s = np.empty((srt.size, d), dtype=np.float64)
        lse_s = np.empty((srt.size,), dtype=np.float64)
        self._run(q, k, v, dtype, scale, causal, srt, o_s, lse_s, nthreads)
        o = np.empty_like(o_s)
        lse = np.empty_like(lse_s)
        o[order] = o_s
        lse[order] = lse_s
        return o, lse

    def _run(self, q, k, v, dtype, scale, causal, rows, o, lse, nthreads):
        B, Hq, Nq, d = q.shape
        Hkv, Nk = k.shape[1], k.shape[2]
        rp = None if rows is None else _ptr(rows, ctypes.c_int64)
        nr = 0 if rows is None else rows.size
        if Hq == 0 or B == 0 or Nq == 0:
            return
        rc = self.lib.oracle_attn_general(
            _ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16),
            _ptr(v, ctypes.c_uint16), _DTYPES[dtype], B, Hq, Hkv, Nq, Nk, d,
            float(scale), 1 if causal else 0, rp, nr, _ptr(o, ctypes.c_double),
            _ptr(lse, ctypes.c_double), int(nthreads))
        if rc != 0:
            raise RuntimeError("oracle_attn_general failed (%d)" % rc)


_default = None


def default() -> Oracle:
    """The oracle built from attn_ref.c beside this file (built on demand)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def host_threads() -> int:
    return default().host_threads()


def decode(bits, dtype) -> np.ndarray:
    return default().decode(bits, dtype)


def attention(q_bits, k_bits, v_bits, dtype, scale, rows=None, nthreads=0,
              causal=False):
    """See Oracle.attention."""
    return default().attention(q_bits, k_bits, v_bits, dtype, scale, rows,
                               nthreads, causal)
