"""Thin Python binding of the C ABI in include/fa2.h (argument marshalling only).

Every step of the computation runs in the HIP kernels of libfa2.so; this module
checks tensor metadata, allocates outputs with torch, passes raw device
pointers and the current HIP stream, and turns status codes into exceptions.
There is no fallback: if libfa2.so is missing, every call raises.
"""
import ctypes
import math
import os

import torch

from . import _build

OK = 0
ERR_NULL = -1
ERR_SHAPE = -2
ERR_HEADDIM = -3
ERR_DTYPE = -4
ERR_ALIGN = -5
ERR_SCALE = -6
ERR_ALIAS = -7
ERR_HIP = -8
ERR_OPTION = -9
ERR_WORKSPACE = -10
ERR_SCRATCH = -11

BF16 = 0
FP16 = 1
CACHE_INT8 = 1
CACHE_FP8 = 2
_DTYPE = {torch.bfloat16: BF16, torch.float16: FP16}

# Entry points declared in include/fa2.h, with their ctypes signatures.
_SIGNATURES = {
    "fa2_fwd": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                               ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                               ctypes.c_float, ctypes.c_int, ctypes.c_void_p]),
    "fa2_fwd_ext": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                   ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_int64, ctypes.c_int64, ctypes.c_float,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_void_p]),
    "fa2_fwd_kv_int8": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_int64, ctypes.c_float, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_void_p]),
    "fa2_fwd_kv_fp8": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_int64, ctypes.c_float, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_void_p]),
    "fa2_fwd_split": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                     ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                     ctypes.c_int64, ctypes.c_int64, ctypes.c_float,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                     ctypes.c_int64, ctypes.c_void_p]),
    "fa2_fwd_split_workspace": (ctypes.c_int64, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                                 ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                                 ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                 ctypes.c_int]),
    "fa2_fwd_kv_split": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_int64, ctypes.c_float, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]),
    "fa2_fwd_split_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                             ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                             ctypes.c_int64, ctypes.c_float, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_int, ctypes.c_void_p]),
    "fa2_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "fa2_tile_config": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int,
                                       ctypes.POINTER(ctypes.c_int),
                                       ctypes.POINTER(ctypes.c_int),
                                       ctypes.POINTER(ctypes.c_int)]),
}

_lib = None


class FA2Error(RuntimeError):
    def __init__(self, code):
        self.code = code
        super().__init__("fa2_fwd failed (%d): %s" % (code, strerror(code)))


def library_path() -> str:
    return _build.LIB


def load(path: str) -> ctypes.CDLL:
    """Load a build of the library at `path` with the declared signatures."""
    if not os.path.exists(path):
        raise RuntimeError("%s is not built; run __graft_entry__.build()" % path)
    handle = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    return handle


def lib() -> ctypes.CDLL:
    """The loaded libfa2.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        _lib = load(_build.LIB)
    return _lib


def strerror(code: int) -> str:
    return lib().fa2_strerror(int(code)).decode()


def tile_config(d: int, dtype=torch.bfloat16):
    """(block_q, block_k, waves) that fa2_fwd uses for this head dim / dtype."""
    code_dtype = _DTYPE.get(dtype, -1) if isinstance(dtype, torch.dtype) else int(dtype)
    bq, bk, nw = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    code = lib().fa2_tile_config(int(d), code_dtype, ctypes.byref(bq),
                                 ctypes.byref(bk), ctypes.byref(nw))
    if code != OK:
        raise FA2Error(code)
    return bq.value, bk.value, nw.value


def fwd_raw(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, N, d, scale, dtype,
            stream=0) -> int:
    """Direct C-ABI call with integer pointers; returns the status code."""
    return lib().fa2_fwd(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, N, d,
                         float(scale), int(dtype), stream)


def fwd_ext_raw(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, Hq, Hkv, Nq, Nk, d, scale,
                causal, dtype, stream=0) -> int:
    """Direct call of fa2_fwd_ext with integer pointers; returns the status."""
    return lib().fa2_fwd_ext(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, Hq, Hkv, Nq, Nk,
                             d, float(scale), int(causal), int(dtype), stream)


def fwd_split_raw(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, Hq, Hkv, Nq, Nk, d, scale, causal,
                  dtype, splits, ws_ptr, ws_bytes, stream=0) -> int:
    """Direct call of fa2_fwd_split with integer pointers; returns the status."""
    return lib().fa2_fwd_split(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, Hq, Hkv, Nq, Nk, d,
                               float(scale), int(causal), int(dtype), int(splits), ws_ptr,
                               int(ws_bytes), stream)


def split_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, causal=False, dtype=BF16, splits=0,
                          cache=0) -> int:
    """fa2_fwd_split_workspace: workspace bytes for these arguments (cache 0:
    fwd_split, CACHE_INT8 / CACHE_FP8: fwd_kv_split; 0 bytes: the call runs
    without splits); raises FA2Error for arguments it rejects."""
    code_dtype = _DTYPE.get(dtype, -1) if isinstance(dtype, torch.dtype) else int(dtype)
    n = lib().fa2_fwd_split_workspace(B, Hq, Hkv, Nq, Nk, d, 1 if causal else 0, code_dtype,
                                      int(cache), int(splits))
    if n < 0:
        raise FA2Error(int(n))
    return int(n)


def fwd_kv_int8_raw(q_ptr, kq_ptr, ks_ptr, vq_ptr, vs_ptr, o_ptr, lse_ptr, B, Hq, Hkv, Nq,
                    Nk, d, scale, causal, dtype, stream=0) -> int:
    """Direct call of fa2_fwd_kv_int8 with integer pointers; returns the status."""
    return lib().fa2_fwd_kv_int8(q_ptr, kq_ptr, ks_ptr, vq_ptr, vs_ptr, o_ptr, lse_ptr, B, Hq,
                                 Hkv, Nq, Nk, d, float(scale), int(causal), int(dtype), stream)


def fwd_kv_fp8_raw(q_ptr, kq_ptr, ks_ptr, vq_ptr, vs_ptr, o_ptr, lse_ptr, B, Hq, Hkv, Nq,
                   Nk, d, scale, causal, dtype, stream=0) -> int:
    """Direct call of fa2_fwd_kv_fp8 with integer pointers; returns the status."""
    return lib().fa2_fwd_kv_fp8(q_ptr, kq_ptr, ks_ptr, vq_ptr, vs_ptr, o_ptr, lse_ptr, B, Hq,
                                Hkv, Nq, Nk, d, float(scale), int(causal), int(dtype), stream)


def _outputs(q, out, lse):
    B, Hq, Nq, _ = q.shape
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or out.device != q.device \
            or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    elif lse.shape != (B, Hq, Nq) or lse.dtype != torch.float32 \
            or lse.device != q.device or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, Hq, Nq] tensor")
    return out, lse


def _kv_quantized(raw, code_dtype, what, q, kq, ks, vq, vs, scale, causal, out, lse):
    """Shared marshalling of the quantized-cache entry points."""
    if q.dim() != 4 or kq.dim() != 4 or kq.shape != vq.shape:
        raise ValueError("q must be [B, Hq, Nq, d] and kq, vq one [B, Hkv, Nk, d] shape")
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, dk = kq.shape
    if kq.shape[0] != B or dk != d:
        raise ValueError("kq, vq must share q's batch and head dimension")
    if q.dtype not in _DTYPE or kq.dtype != code_dtype or vq.dtype != code_dtype:
        raise ValueError("q must be bfloat16 or float16 and kq, vq %s" % what)
    if ks.shape != (B, Hkv, d) or vs.shape != (B, Hkv, d) or ks.dtype != torch.float32 \
            or vs.dtype != torch.float32:
        raise ValueError("ks and vs must be float32 [B, Hkv, d]")
    tensors = (q, kq, ks, vq, vs)
    if not all(t.is_cuda and t.device == q.device for t in tensors):
        raise ValueError("all inputs must be on one GPU")
    if not all(t.is_contiguous() for t in tensors):
        raise ValueError("all inputs must be contiguous")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out, lse = _outputs(q, out, lse)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        code = raw(q.data_ptr(), kq.data_ptr(), ks.data_ptr(), vq.data_ptr(), vs.data_ptr(),
                   out.data_ptr(), lse.data_ptr(), B, Hq, Hkv, Nq, Nk, d, scale,
                   1 if causal else 0, _DTYPE[q.dtype], stream)
    if code != OK:
        raise FA2Error(code)
    return out, lse


def fwd_kv_int8(q, kq, ks, vq, vs, scale=None, causal=False, out=None, lse=None):
    """Attention over an INT8 key/value cache: returns (o, lse).

    q: [B, Hq, Nq, d] bf16 or fp16 (d = 64, 128 or 256); kq, vq: [B, Hkv, Nk, d]
    int8 codes; ks, vs: [B, Hkv, d] float32 per-channel scales (k = ks * kq, v = vs *
    vq).  The query rows are quantized to int8 in the kernel (see fa2.h);
    other arguments as in `fwd`.  All tensors contiguous on one GPU.
    """
    return _kv_quantized(fwd_kv_int8_raw, torch.int8, "int8", q, kq, ks, vq, vs, scale,
                         causal, out, lse)


def fwd_kv_fp8(q, kq, ks, vq, vs, scale=None, causal=False, out=None, lse=None):
    """Attention over an FP8 (OCP E4M3) key/value cache: returns (o, lse).

    As `fwd_kv_int8` with kq, vq uint8 tensors of E4M3 codes (k = ks *
    e4m3(kq), v = vs * e4m3(vq)); the query rows are rounded to E4M3 in the
    kernel (see fa2.h).
    """
    return _kv_quantized(fwd_kv_fp8_raw, torch.uint8, "uint8 E4M3 codes", q, kq, ks, vq, vs,
                         scale, causal, out, lse)


def fwd(q, k, v, scale=None, causal=False, out=None, lse=None):
    """Attention forward: returns (o, lse).

    q: [B, Hq, Nq, d]; k, v: [B, Hkv, Nk, d] with Hq a multiple of Hkv; all
    contiguous bf16 or fp16 CUDA(HIP) tensors of one dtype on one device.
    scale: logit multiplier, default 1/sqrt(d).  causal: row i sees keys
    j <= i + Nk - Nq.  out, lse: optional preallocated outputs ([B, Hq, Nq, d]
    of q's dtype and [B, Hq, Nq] float32, contiguous, on q's device).
    Equal shapes and causal=False call fa2_fwd; anything else fa2_fwd_ext.
    The kernel is enqueued on torch's current stream of q's device.
    """
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("q must be [B, Hq, Nq, d] and k, v one [B, Hkv, Nk, d] shape")
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, dk = k.shape
    if k.shape[0] != B or dk != d:
        raise ValueError("k, v must share q's batch and head dimension")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _DTYPE:
        raise ValueError("q, k, v must all be bfloat16 or all float16")
    if not (q.is_cuda and k.device == q.device and v.device == q.device):
        raise ValueError("q, k, v must be on one GPU")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out, lse = _outputs(q, out, lse)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        if q.shape == k.shape and not causal:
            code = fwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                           lse.data_ptr(), B, Hq, Nq, d, scale, _DTYPE[q.dtype], stream)
        else:
            code = fwd_ext_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                               lse.data_ptr(), B, Hq, Hkv, Nq, Nk, d, scale,
                               1 if causal else 0, _DTYPE[q.dtype], stream)
    if code != OK:
        raise FA2Error(code)
    return out, lse


def fwd_split(q, k, v, scale=None, causal=False, splits=0, workspace=None, out=None, lse=None):
    """Attention forward with key splits (fa2_fwd_split): returns (o, lse).

    Arguments as in `fwd`; splits: 0 (chosen by the library for the current
    device), 1 (no split) or up to 128 key parts per query tile.
    workspace: an optional device tensor of at least split_workspace_bytes()
    bytes (any dtype, contiguous, 16-byte aligned); without one a uint8
    tensor of that size is allocated with torch for the call.  The kernels
    are enqueued on torch's current stream of q's device.
    """
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("q must be [B, Hq, Nq, d] and k, v one [B, Hkv, Nk, d] shape")
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, dk = k.shape
    if k.shape[0] != B or dk != d:
        raise ValueError("k, v must share q's batch and head dimension")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _DTYPE:
        raise ValueError("q, k, v must all be bfloat16 or all float16")
    if not (q.is_cuda and k.device == q.device and v.device == q.device):
        raise ValueError("q, k, v must be on one GPU")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out, lse = _outputs(q, out, lse)
    with torch.cuda.device(q.device):
        need = split_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, causal, q.dtype, splits)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        elif not (workspace.is_cuda and workspace.device == q.device
                  and workspace.is_contiguous()):
            raise ValueError("workspace must be a contiguous tensor on q's device")
        ws_bytes = workspace.numel() * workspace.element_size()
        stream = torch.cuda.current_stream(q.device).cuda_stream
        code = fwd_split_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                             lse.data_ptr(), B, Hq, Hkv, Nq, Nk, d, scale, 1 if causal else 0,
                             _DTYPE[q.dtype], splits, workspace.data_ptr(), ws_bytes, stream)
    if code != OK:
        raise FA2Error(code)
    return out, lse


def fwd_kv_split_raw(q_ptr, kq_ptr, ks_ptr, vq_ptr, vs_ptr, o_ptr, lse_ptr, B, Hq, Hkv, Nq, Nk,
                     d, scale, causal, dtype, cache, splits, ws_ptr, ws_bytes, stream=0) -> int:
    """Direct call of fa2_fwd_kv_split with integer pointers; returns the status."""
    return lib().fa2_fwd_kv_split(q_ptr, kq_ptr, ks_ptr, vq_ptr, vs_ptr, o_ptr, lse_ptr, B, Hq,
                                  Hkv, Nq, Nk, d, float(scale), int(causal), int(dtype),
                                  int(cache), int(splits), ws_ptr, int(ws_bytes), stream)


def fwd_kv_split(q, kq, ks, vq, vs, cache, scale=None, causal=False, splits=0, workspace=None,
                 out=None, lse=None):
    """Key splits over a quantized cache (fa2_fwd_kv_split): returns (o, lse).

    As `fwd_kv_int8` (cache = CACHE_INT8, kq/vq int8) or `fwd_kv_fp8`
    (cache = CACHE_FP8, kq/vq uint8 E4M3 codes), with splits and workspace
    as in `fwd_split`.
    """
    code_dtype = {CACHE_INT8: torch.int8, CACHE_FP8: torch.uint8}.get(cache)
    if code_dtype is None:
        raise ValueError("cache must be CACHE_INT8 or CACHE_FP8")
    B, Hq, Nq, d = q.shape
    Hkv, Nk = kq.shape[1], kq.shape[2]
    if workspace is None:
        need = split_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, causal, q.dtype, splits, cache) \
            if q.dtype in _DTYPE else 0
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    elif not (workspace.is_cuda and workspace.device == q.device and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor on q's device")
    ws_bytes = workspace.numel() * workspace.element_size()

    def raw(qp, kqp, ksp, vqp, vsp, op, lp, B_, Hq_, Hkv_, Nq_, Nk_, d_, sc, ca, dt, st):
        return fwd_kv_split_raw(qp, kqp, ksp, vqp, vsp, op, lp, B_, Hq_, Hkv_, Nq_, Nk_, d_, sc,
                                ca, dt, cache, splits, workspace.data_ptr(), ws_bytes, st)

    return _kv_quantized(raw, code_dtype, "int8" if cache == CACHE_INT8 else "uint8 E4M3 codes",
                         q, kq, ks, vq, vs, scale, causal, out, lse)
