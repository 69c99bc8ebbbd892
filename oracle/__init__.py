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

``attention_kv_int8`` computes the same over an INT8 key/value cache (int8
codes with fp32 per-channel scales; the query rows quantized to int8 after the
key scales are folded in, every quantization step in binary32 as spelled out in
``attn_ref.c``), and ``quantize_q`` exposes that query quantization alone.
``attention_kv_fp8`` and ``quantize_q_fp8`` do the same for an FP8 cache whose
codes are OCP E4M3 values (the query rows rounded to E4M3, ties to even, after
scaling their largest magnitude to 448); ``e4m3_decode`` and ``e4m3_round``
expose the code conversions.
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
        i8p = ctypes.POINTER(ctypes.c_int8)
        f32p = ctypes.POINTER(ctypes.c_float)
        lib.oracle_attn_kv_int8.argtypes = [
            u16p, ctypes.c_int, i8p, f32p, i8p, f32p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_double, ctypes.c_int,
            i64p, ctypes.c_int64, f64p, f64p, ctypes.c_int]
        lib.oracle_attn_kv_int8.restype = ctypes.c_int
        lib.oracle_quantize_q.argtypes = [u16p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                          f32p, i8p, f32p]
        lib.oracle_quantize_q.restype = ctypes.c_int
        u8p = ctypes.POINTER(ctypes.c_uint8)
        lib.oracle_attn_kv_fp8.argtypes = [
            u16p, ctypes.c_int, u8p, f32p, u8p, f32p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_double, ctypes.c_int,
            i64p, ctypes.c_int64, f64p, f64p, ctypes.c_int]
        lib.oracle_attn_kv_fp8.restype = ctypes.c_int
        lib.oracle_quantize_q_fp8.argtypes = [u16p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                              f32p, u8p, f32p]
        lib.oracle_quantize_q_fp8.restype = ctypes.c_int
        lib.oracle_e4m3_decode.argtypes = [u8p, ctypes.c_int64, f64p]
        lib.oracle_e4m3_decode.restype = ctypes.c_int
        lib.oracle_e4m3_round.argtypes = [f32p, ctypes.c_int64, u8p]
        lib.oracle_e4m3_round.restype = ctypes.c_int
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
        Hkv, Nk = k.shape[1], k.shape[2]

        def run(rp, nr, o, lse):
            return self.lib.oracle_attn_general(
                _ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16),
                _ptr(v, ctypes.c_uint16), _DTYPES[dtype], B, Hq, Hkv, Nq, Nk, d,
                float(scale), 1 if causal else 0, rp, nr, _ptr(o, ctypes.c_double),
                _ptr(lse, ctypes.c_double), int(nthreads))
        return self._rows_call(q.shape, rows, run, "oracle_attn_general")

    def attention_kv_int8(self, q_bits, kq, ks, vq, vs, dtype, scale, rows=None,
                          nthreads=0, causal=False):
        """fp64 attention over an INT8 key/value cache.

        q_bits: uint16 [B, Hq, Nq, d] (16-bit patterns of `dtype`); kq, vq:
        int8 [B, Hkv, Nk, d] codes; ks, vs: float32 [B, Hkv, d] per-channel
        scales (k = ks * kq, v = vs * vq).  Each query row is quantized to int8
        after the key scales are folded in (see the module docstring); the
        other arguments and the result are those of `attention`.
        """
        q = np.ascontiguousarray(q_bits, dtype=np.uint16)
        kq = np.ascontiguousarray(kq, dtype=np.int8)
        vq = np.ascontiguousarray(vq, dtype=np.int8)
        ks = np.ascontiguousarray(ks, dtype=np.float32)
        vs = np.ascontiguousarray(vs, dtype=np.float32)
        if q.ndim != 4 or kq.ndim != 4 or kq.shape != vq.shape:
            raise ValueError("q must be [B, Hq, Nq, d], kq and vq one [B, Hkv, Nk, d] shape")
        B, Hq, Nq, d = q.shape
        Hkv, Nk = kq.shape[1], kq.shape[2]
        if kq.shape[0] != B or kq.shape[3] != d or Hkv < 1 or Hq % Hkv:
            raise ValueError("kq/vq batch and head dim must match q, Hq a multiple of Hkv")
        if ks.shape != (B, Hkv, d) or vs.shape != (B, Hkv, d):
            raise ValueError("ks and vs must be [B, Hkv, d]")

        def run(rp, nr, o, lse):
            return self.lib.oracle_attn_kv_int8(
                _ptr(q, ctypes.c_uint16), _DTYPES[dtype], _ptr(kq, ctypes.c_int8),
                _ptr(ks, ctypes.c_float), _ptr(vq, ctypes.c_int8), _ptr(vs, ctypes.c_float),
                B, Hq, Hkv, Nq, Nk, d, float(scale), 1 if causal else 0, rp, nr,
                _ptr(o, ctypes.c_double), _ptr(lse, ctypes.c_double), int(nthreads))
        return self._rows_call(q.shape, rows, run, "oracle_attn_kv_int8")

    def quantize_q(self, q_bits, ks, dtype):
        """INT8 codes and row scales of query rows: q_bits uint16 [..., d]
        (16-bit patterns), ks float32 [d] key scales.  Returns (codes int8
        [..., d], sq float32 [...])."""
        q = np.ascontiguousarray(q_bits, dtype=np.uint16)
        ks = np.ascontiguousarray(ks, dtype=np.float32).ravel()
        d = q.shape[-1]
        if ks.size != d:
            raise ValueError("ks must hold d scales")
        n = q.size // d
        codes = np.empty(q.shape, dtype=np.int8)
        sq = np.empty(q.shape[:-1], dtype=np.float32)
        rc = self.lib.oracle_quantize_q(_ptr(q, ctypes.c_uint16), _DTYPES[dtype], n, d,
                                        _ptr(ks, ctypes.c_float), _ptr(codes, ctypes.c_int8),
                                        _ptr(sq, ctypes.c_float))
        if rc != 0:
            raise ValueError("oracle_quantize_q failed (%d)" % rc)
        return codes, sq

    def attention_kv_fp8(self, q_bits, kf, ks, vf, vs, dtype, scale, rows=None,
                         nthreads=0, causal=False):
        """fp64 attention over an FP8 (OCP E4M3) key/value cache.

        As `attention_kv_int8` with kf, vf uint8 [B, Hkv, Nk, d] E4M3 codes
        (k = ks * e4m3(kf), v = vs * e4m3(vf)) and the query rows rounded to
        E4M3 (see the module docstring).
        """
        q = np.ascontiguousarray(q_bits, dtype=np.uint16)
        kf = np.ascontiguousarray(kf, dtype=np.uint8)
        vf = np.ascontiguousarray(vf, dtype=np.uint8)
        ks = np.ascontiguousarray(ks, dtype=np.float32)
        vs = np.ascontiguousarray(vs, dtype=np.float32)
        if q.ndim != 4 or kf.ndim != 4 or kf.shape != vf.shape:
            raise ValueError("q must be [B, Hq, Nq, d], kf and vf one [B, Hkv, Nk, d] shape")
        B, Hq, Nq, d = q.shape
        Hkv, Nk = kf.shape[1], kf.shape[2]
        if kf.shape[0] != B or kf.shape[3] != d or Hkv < 1 or Hq % Hkv:
            raise ValueError("kf/vf batch and head dim must match q, Hq a multiple of Hkv")
        if ks.shape != (B, Hkv, d) or vs.shape != (B, Hkv, d):
            raise ValueError("ks and vs must be [B, Hkv, d]")

        def run(rp, nr, o, lse):
            return self.lib.oracle_attn_kv_fp8(
                _ptr(q, ctypes.c_uint16), _DTYPES[dtype], _ptr(kf, ctypes.c_uint8),
                _ptr(ks, ctypes.c_float), _ptr(vf, ctypes.c_uint8), _ptr(vs, ctypes.c_float),
                B, Hq, Hkv, Nq, Nk, d, float(scale), 1 if causal else 0, rp, nr,
                _ptr(o, ctypes.c_double), _ptr(lse, ctypes.c_double), int(nthreads))
        return self._rows_call(q.shape, rows, run, "oracle_attn_kv_fp8")

    def quantize_q_fp8(self, q_bits, ks, dtype):
        """E4M3 codes and row scales of query rows (the FP8 scheme): as
        `quantize_q`, codes uint8 [..., d]."""
        q = np.ascontiguousarray(q_bits, dtype=np.uint16)
        ks = np.ascontiguousarray(ks, dtype=np.float32).ravel()
        d = q.shape[-1]
        if ks.size != d:
            raise ValueError("ks must hold d scales")
        n = q.size // d
        codes = np.empty(q.shape, dtype=np.uint8)
        sq = np.empty(q.shape[:-1], dtype=np.float32)
        rc = self.lib.oracle_quantize_q_fp8(_ptr(q, ctypes.c_uint16), _DTYPES[dtype], n, d,
                                            _ptr(ks, ctypes.c_float), _ptr(codes, ctypes.c_uint8),
                                            _ptr(sq, ctypes.c_float))
        if rc != 0:
            raise ValueError("oracle_quantize_q_fp8 failed (%d)" % rc)
        return codes, sq

    def e4m3_decode(self, codes) -> np.ndarray:
        """Exact fp64 value of each OCP E4M3 code (uint8)."""
        codes = np.ascontiguousarray(codes, dtype=np.uint8)
        out = np.empty(codes.shape, dtype=np.float64)
        self.lib.oracle_e4m3_decode(_ptr(codes, ctypes.c_uint8), codes.size,
                                    _ptr(out, ctypes.c_double))
        return out

    def e4m3_round(self, x) -> np.ndarray:
        """The E4M3 code nearest to each float32 (ties to even, saturating)."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        codes = np.empty(x.shape, dtype=np.uint8)
        rc = self.lib.oracle_e4m3_round(_ptr(x, ctypes.c_float), x.size, _ptr(codes, ctypes.c_uint8))
        if rc != 0:
            raise ValueError("e4m3_round: NaN input")
        return codes

    @staticmethod
    def _rows_call(qshape, rows, run, name):
        """Run `run(rows_ptr, nrows, o, lse)` over every row (O shaped [B, Hq,
        Nq, d]) or over the given distinct flat row ids (O shaped [len, d], in
        the caller's order)."""
        B, Hq, Nq, d = qshape
        if rows is None:
            o = np.empty((B, Hq, Nq, d), dtype=np.float64)
            lse = np.empty((B, Hq, Nq), dtype=np.float64)
            if B and Hq and Nq:
                rc = run(None, 0, o, lse)
                if rc != 0:
                    raise RuntimeError("%s failed (%d)" % (name, rc))
            return o, lse
        rows = np.asarray(rows, dtype=np.int64).ravel()
        order = np.argsort(rows, kind="stable")
        srt = np.ascontiguousarray(rows[order])
        if srt.size and np.any(np.diff(srt) <= 0):
            raise ValueError("rows must not repeat")
        o_s = np.empty((srt.size, d), dtype=np.float64)
        lse_s = np.empty((srt.size,), dtype=np.float64)
        if srt.size and B and Hq and Nq:
            rc = run(_ptr(srt, ctypes.c_int64), srt.size, o_s, lse_s)
            if rc != 0:
                raise RuntimeError("%s failed (%d)" % (name, rc))
        o = np.empty_like(o_s)
        lse = np.empty_like(lse_s)
        o[order] = o_s
        lse[order] = lse_s
        return o, lse


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


def attention_kv_int8(q_bits, kq, ks, vq, vs, dtype, scale, rows=None, nthreads=0,
                      causal=False):
    """See Oracle.attention_kv_int8."""
    return default().attention_kv_int8(q_bits, kq, ks, vq, vs, dtype, scale, rows,
                                       nthreads, causal)


def quantize_q(q_bits, ks, dtype):
    """See Oracle.quantize_q."""
    return default().quantize_q(q_bits, ks, dtype)


def attention_kv_fp8(q_bits, kf, ks, vf, vs, dtype, scale, rows=None, nthreads=0,
                     causal=False):
    """See Oracle.attention_kv_fp8."""
    return default().attention_kv_fp8(q_bits, kf, ks, vf, vs, dtype, scale, rows,
                                      nthreads, causal)


def quantize_q_fp8(q_bits, ks, dtype):
    """See Oracle.quantize_q_fp8."""
    return default().quantize_q_fp8(q_bits, ks, dtype)


def e4m3_decode(codes):
    """See Oracle.e4m3_decode."""
    return default().e4m3_decode(codes)


def e4m3_round(x):
    """See Oracle.e4m3_round."""
    return default().e4m3_round(x)
