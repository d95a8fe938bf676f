"""Python binding of libattn (exact attention for MI355X / gfx950).

Argument marshalling only: torch tensors are turned into device pointers,
element strides and the current HIP stream, and handed to the C ABI declared
in include/attn.h.  Every step of the computation runs in the library's HIP
kernels; there is no fallback.  If libattn.so is missing, importing this
package raises ImportError (build it with ``python
exact_attention_qk_amd/build.py`` or ``__graft_entry__.build()``).

Names follow the pages: ``attn_fwd`` (flash_attn_func), ``attn_fwd_kvcache``
(flash_attn_with_kvcache) and ``rope_apply`` (the non-fused rotary kernel).
"""
from __future__ import annotations

import ctypes
import math
import os

import torch  # loads the HIP runtime the library must share (load order matters)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn.so")

if not os.path.exists(LIB_PATH):
    raise ImportError("libattn.so not found at %s: build it first "
                      "(python exact_attention_qk_amd/build.py)" % LIB_PATH)

_lib = ctypes.CDLL(LIB_PATH)

ATTN_OK = 0
ERRORS = {-1: "ATTN_E_NULL", -2: "ATTN_E_SHAPE", -3: "ATTN_E_UNSUPPORTED", -4: "ATTN_E_ALIGN",
          -5: "ATTN_E_WORKSPACE", -6: "ATTN_E_OVERFLOW", -7: "ATTN_E_HIP"}
EXPORTED = ["attn_fwd", "attn_fwd_varlen", "attn_fwd_kvcache", "attn_fwd_kvcache_workspace_size",
            "attn_fwd_kvcache_noalloc",
            "attn_bwd", "attn_bwd_workspace_size", "attn_fwd_fp8", "attn_fwd_fp8_workspace_size",
            "rope_apply", "attn_validate_fwd", "attn_validate_varlen", "attn_validate_kvcache",
            "attn_validate_bwd", "attn_validate_fp8", "attn_validate_rope", "attn_last_error",
            "attn_abi_version"]


class AttnError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("%s (%d): %s" % (ERRORS.get(code, "?"), code, msg))
        self.code = code


class Tensor4(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("stride_b", ctypes.c_int64),
                ("stride_s", ctypes.c_int64), ("stride_h", ctypes.c_int64)]


class FwdParams(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("B", ctypes.c_int), ("Sq", ctypes.c_int),
                ("Sk", ctypes.c_int), ("Hq", ctypes.c_int), ("Hkv", ctypes.c_int),
                ("Dqk", ctypes.c_int), ("Dv", ctypes.c_int),
                ("q", Tensor4), ("k", Tensor4), ("v", Tensor4), ("out", Tensor4),
                ("lse", ctypes.c_void_p), ("causal", ctypes.c_int),
                ("softmax_scale", ctypes.c_float),
                ("window_left", ctypes.c_int), ("window_right", ctypes.c_int)]


class Fp8Params(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("Sq", ctypes.c_int), ("Sk", ctypes.c_int), ("Hq", ctypes.c_int),
                ("Hkv", ctypes.c_int), ("D", ctypes.c_int),
                ("q", Tensor4), ("k", Tensor4), ("v", Tensor4), ("out", Tensor4),
                ("lse", ctypes.c_void_p), ("causal", ctypes.c_int), ("softmax_scale", ctypes.c_float),
                ("descale_q", ctypes.c_float), ("descale_k", ctypes.c_float), ("descale_v", ctypes.c_float),
                ("window_left", ctypes.c_int), ("window_right", ctypes.c_int),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


class VarlenParams(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("B", ctypes.c_int), ("total_q", ctypes.c_int),
                ("total_k", ctypes.c_int), ("max_seqlen_q", ctypes.c_int), ("Hq", ctypes.c_int),
                ("Hkv", ctypes.c_int), ("Dqk", ctypes.c_int), ("Dv", ctypes.c_int),
                ("q", Tensor4), ("k", Tensor4), ("v", Tensor4), ("out", Tensor4),
                ("cu_seqlens_q", ctypes.c_void_p), ("cu_seqlens_k", ctypes.c_void_p),
                ("lse", ctypes.c_void_p), ("causal", ctypes.c_int), ("softmax_scale", ctypes.c_float),
                ("window_left", ctypes.c_int), ("window_right", ctypes.c_int)]


class BwdParams(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("B", ctypes.c_int), ("Sq", ctypes.c_int),
                ("Sk", ctypes.c_int), ("Hq", ctypes.c_int), ("Hkv", ctypes.c_int),
                ("Dqk", ctypes.c_int), ("Dv", ctypes.c_int),
                ("q", Tensor4), ("k", Tensor4), ("v", Tensor4), ("out", Tensor4), ("dout", Tensor4),
                ("dq", Tensor4), ("dk", Tensor4), ("dv", Tensor4),
                ("lse", ctypes.c_void_p), ("causal", ctypes.c_int), ("softmax_scale", ctypes.c_float),
                ("window_left", ctypes.c_int), ("window_right", ctypes.c_int),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


class KVCacheParams(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("B", ctypes.c_int), ("Sq", ctypes.c_int),
                ("Hq", ctypes.c_int), ("Hkv", ctypes.c_int), ("Dqk", ctypes.c_int),
                ("Dv", ctypes.c_int), ("capacity", ctypes.c_int), ("Snew", ctypes.c_int),
                ("q", Tensor4), ("k_cache", Tensor4), ("v_cache", Tensor4),
                ("k_new", Tensor4), ("v_new", Tensor4), ("out", Tensor4),
                ("cache_seqlens_scalar", ctypes.c_int), ("cache_seqlens", ctypes.c_void_p),
                ("rotary_cos", ctypes.c_void_p), ("rotary_sin", ctypes.c_void_p),
                ("rotary_dim", ctypes.c_int), ("seqlen_ro", ctypes.c_int),
                ("rotary_interleaved", ctypes.c_int), ("causal", ctypes.c_int),
                ("softmax_scale", ctypes.c_float), ("lse", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("num_splits", ctypes.c_int),
                ("window_left", ctypes.c_int), ("window_right", ctypes.c_int)]


class RopeParams(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("B", ctypes.c_int), ("S", ctypes.c_int),
                ("H", ctypes.c_int), ("D", ctypes.c_int), ("x", Tensor4), ("out", Tensor4),
                ("cos", ctypes.c_void_p), ("sin", ctypes.c_void_p),
                ("rotary_dim", ctypes.c_int), ("seqlen_ro", ctypes.c_int),
                ("interleaved", ctypes.c_int), ("conjugate", ctypes.c_int),
                ("offset_scalar", ctypes.c_int), ("offsets", ctypes.c_void_p)]


_lib.attn_fwd.argtypes = [ctypes.POINTER(FwdParams), ctypes.c_void_p]
_lib.attn_fwd_varlen.argtypes = [ctypes.POINTER(VarlenParams), ctypes.c_void_p]
_lib.attn_validate_varlen.argtypes = [ctypes.POINTER(VarlenParams)]
_lib.attn_bwd.argtypes = [ctypes.POINTER(BwdParams), ctypes.c_void_p]
_lib.attn_validate_bwd.argtypes = [ctypes.POINTER(BwdParams)]
_lib.attn_bwd_workspace_size.argtypes = [ctypes.POINTER(BwdParams)]
_lib.attn_bwd_workspace_size.restype = ctypes.c_size_t
_lib.attn_fwd_kvcache.argtypes = [ctypes.POINTER(KVCacheParams), ctypes.c_void_p]
_lib.attn_fwd_kvcache_workspace_size.argtypes = [ctypes.POINTER(KVCacheParams)]
_lib.attn_fwd_kvcache_workspace_size.restype = ctypes.c_size_t
_lib.attn_fwd_kvcache_noalloc.argtypes = [ctypes.POINTER(KVCacheParams), ctypes.c_void_p]
_lib.rope_apply.argtypes = [ctypes.POINTER(RopeParams), ctypes.c_void_p]
_lib.attn_validate_fwd.argtypes = [ctypes.POINTER(FwdParams)]
_lib.attn_validate_kvcache.argtypes = [ctypes.POINTER(KVCacheParams)]
_lib.attn_validate_rope.argtypes = [ctypes.POINTER(RopeParams)]
_lib.attn_fwd_fp8.argtypes = [ctypes.POINTER(Fp8Params), ctypes.c_void_p]
_lib.attn_validate_fp8.argtypes = [ctypes.POINTER(Fp8Params)]
_lib.attn_fwd_fp8_workspace_size.argtypes = [ctypes.POINTER(Fp8Params)]
_lib.attn_fwd_fp8_workspace_size.restype = ctypes.c_size_t
_lib.attn_last_error.restype = ctypes.c_char_p
for _n in ("attn_fwd", "attn_fwd_varlen", "attn_fwd_kvcache", "attn_fwd_kvcache_noalloc", "attn_bwd", "attn_fwd_fp8", "rope_apply",
           "attn_validate_fwd", "attn_validate_varlen", "attn_validate_kvcache", "attn_validate_bwd",
           "attn_validate_fp8", "attn_validate_rope", "attn_abi_version"):
    getattr(_lib, _n).restype = ctypes.c_int

_DT = {torch.float16: 0, torch.bfloat16: 1}


def lib():
    return _lib


def _check(code):
    if code != ATTN_OK:
        raise AttnError(code, _lib.attn_last_error().decode())


def _on_gpu(*tensors):
    """Every tensor a call hands to the kernels must be a GPU tensor, all on one device
    (a host pointer reaching a kernel would be a memory fault, not an error code)."""
    dev = None
    for t in tensors:
        if t is None or not isinstance(t, torch.Tensor):
            continue
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU, got one on %s" % t.device)
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("tensors on different devices: %s and %s" % (dev, t.device))


def _t4(t):
    if t is None:
        return Tensor4(None, 0, 0, 0)
    if t.dim() != 4:
        raise ValueError("expected a [batch, seqlen, heads, head_dim] tensor, got %d dims" % t.dim())
    if t.shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError("head_dim must be contiguous (stride 1)")
    return Tensor4(t.data_ptr(), t.stride(0), t.stride(1), t.stride(2))


def _expect(t, shape, dtype, name):
    """Refuse a tensor whose shape or dtype does not match what the call's other
    arguments imply: a mismatch would make a kernel read or write outside it."""
    if t is None:
        return
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))


def _lse_ok(lse, shape):
    if lse is None:
        return
    if not (lse.dtype == torch.float32 and lse.is_contiguous() and tuple(lse.shape) == tuple(shape)):
        raise ValueError("lse must be a contiguous float32 tensor of shape %s" % (tuple(shape),))


def _tables_ok(cos, sin, dtype, max_rd):
    """cos/sin tables: [seqlen_ro, rotary_dim/2], the working dtype, contiguous rows
    of exactly rotary_dim/2 elements (the kernels index row p at p * rotary_dim/2)."""
    if (cos is None) != (sin is None):
        raise ValueError("rotary_cos and rotary_sin must both be given or both be None")
    if cos is None:
        return
    for name, t in (("rotary_cos", cos), ("rotary_sin", sin)):
        if t.dim() != 2 or not t.is_contiguous():
            raise ValueError("%s must be a contiguous [seqlen_ro, rotary_dim/2] tensor" % name)
        if t.dtype != dtype:
            raise ValueError("%s has dtype %s, expected the working dtype %s" % (name, t.dtype, dtype))
    if tuple(cos.shape) != tuple(sin.shape):
        raise ValueError("rotary_cos %s and rotary_sin %s differ in shape" % (tuple(cos.shape), tuple(sin.shape)))
    if 2 * cos.shape[1] > max_rd:
        raise ValueError("rotary width 2*%d exceeds head_dim %d" % (cos.shape[1], max_rd))


def _offsets_ok(t, B, name):
    if isinstance(t, torch.Tensor):
        if not (t.dtype == torch.int32 and t.is_contiguous() and t.dim() == 1):
            raise ValueError("%s must be an int or a contiguous 1-d int32 tensor" % name)
        if t.numel() < B:
            raise ValueError("%s has %d entries for %d batch elements" % (name, t.numel(), B))


def _dtype(t):
    if t.dtype not in _DT:
        raise AttnError(-3, "dtype %s is not float16 or bfloat16" % t.dtype)
    return _DT[t.dtype]


def _scale(s):
    return float("nan") if s is None else float(s)


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream) if t.is_cuda else None


# ---------------------------------------------------------------- attn_fwd

def fwd_params(q, k, v, out, causal=False, softmax_scale=None, lse=None, window_size=(-1, -1)):
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if t.dim() != 4:
            raise ValueError("%s must be a [batch, seqlen, heads, head_dim] tensor" % name)
    B, Sq, Hq, Dqk = q.shape
    Sk, Hkv, Dv = k.shape[1], k.shape[2], v.shape[3]
    _expect(k, (B, Sk, Hkv, Dqk), q.dtype, "k")
    _expect(v, (B, Sk, Hkv, Dv), q.dtype, "v")
    _expect(out, (B, Sq, Hq, Dv), q.dtype, "out")
    _lse_ok(lse, (B, Hq, Sq))
    return FwdParams(_dtype(q), B, Sq, Sk, Hq, Hkv, Dqk, Dv, _t4(q), _t4(k), _t4(v), _t4(out),
                     lse.data_ptr() if lse is not None else None, int(bool(causal)),
                     _scale(softmax_scale), int(window_size[0]), int(window_size[1]))


def attn_fwd(q, k, v, causal=False, softmax_scale=None, out=None, return_lse=False,
             window_size=(-1, -1)):
    """Exact attention.  q [B,Sq,Hq,Dqk], k [B,Sk,Hkv,Dqk], v [B,Sk,Hkv,Dv] -> out [B,Sq,Hq,Dv].

    ``window_size=(left, right)``: local attention, -1 for an unbounded side.
    """
    B, Sq, Hq, _ = q.shape
    Dv = v.shape[3]
    if out is None:
        out = torch.empty((B, Sq, Hq, Dv), dtype=q.dtype, device=q.device)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device) if return_lse else None
    p = fwd_params(q, k, v, out, causal, softmax_scale, lse, window_size)
    _on_gpu(q, k, v, out)
    _check(_lib.attn_fwd(ctypes.byref(p), _stream(q)))
    return (out, lse) if return_lse else out


# ---------------------------------------------------------------- gradients

def bwd_params(q, k, v, out, dout, lse, dq, dk, dv, causal=False, softmax_scale=None,
               window_size=(-1, -1)):
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        if t.dim() != 4:
            raise ValueError("%s must be a [batch, seqlen, heads, head_dim] tensor" % name)
    B, Sq, Hq, Dqk = q.shape
    Sk, Hkv, Dv = k.shape[1], k.shape[2], v.shape[3]
    _expect(k, (B, Sk, Hkv, Dqk), q.dtype, "k")
    _expect(v, (B, Sk, Hkv, Dv), q.dtype, "v")
    _expect(out, (B, Sq, Hq, Dv), q.dtype, "out")
    _expect(dout, (B, Sq, Hq, Dv), q.dtype, "dout")
    _expect(dq, (B, Sq, Hq, Dqk), q.dtype, "dq")
    _expect(dk, (B, Sk, Hkv, Dqk), q.dtype, "dk")
    _expect(dv, (B, Sk, Hkv, Dv), q.dtype, "dv")
    if lse is None or not (lse.dtype == torch.float32 and lse.is_contiguous() and tuple(lse.shape) == (B, Hq, Sq)):
        raise ValueError("lse must be a contiguous float32 [B, Hq, Sq] tensor from the forward call")
    return BwdParams(_dtype(q), B, Sq, Sk, Hq, Hkv, Dqk, Dv, _t4(q), _t4(k), _t4(v), _t4(out), _t4(dout),
                     _t4(dq), _t4(dk), _t4(dv), lse.data_ptr(), int(bool(causal)), _scale(softmax_scale),
                     int(window_size[0]), int(window_size[1]), None, 0)


def _bwd_workspace(p, device):
    need = int(_lib.attn_bwd_workspace_size(ctypes.byref(p)))
    ws = torch.empty(need + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    p.workspace = ws.data_ptr() + off if need else None
    p.workspace_bytes = need
    return ws


def attn_bwd(dout, q, k, v, out, lse, causal=False, softmax_scale=None, window_size=(-1, -1),
             dq=None, dk=None, dv=None):
    """Gradients of ``attn_fwd``: returns (dq, dk, dv).  ``out`` and ``lse`` come from the
    forward call (``return_lse=True``) with the same arguments."""
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty(k.shape, dtype=k.dtype, device=k.device) if dk is None else dk
    dv = torch.empty(v.shape, dtype=v.dtype, device=v.device) if dv is None else dv
    p = bwd_params(q, k, v, out, dout, lse, dq, dk, dv, causal, softmax_scale, window_size)
    _on_gpu(dout, q, k, v, out, lse, dq, dk, dv)
    ws = _bwd_workspace(p, q.device)
    _check(_lib.attn_bwd(ctypes.byref(p), _stream(q)))
    del ws
    return dq, dk, dv


def prepare_bwd(dout, q, k, v, out, lse, dq, dk, dv, causal=False, softmax_scale=None,
                window_size=(-1, -1)):
    p = bwd_params(q, k, v, out, dout, lse, dq, dk, dv, causal, softmax_scale, window_size)
    _on_gpu(dout, q, k, v, out, lse, dq, dk, dv)
    ws = _bwd_workspace(p, q.device)
    return PreparedCall(_lib.attn_bwd, p, _stream(q), (dout, q, k, v, out, lse, dq, dk, dv, ws))


# ---------------------------------------------------------------- FP8 inputs

def _codes(t):
    """e4m3 codes: a torch.float8_e4m3fn tensor or its uint8 bit pattern."""
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8)
    if t.dtype != torch.uint8:
        raise AttnError(-3, "fp8 inputs must be float8_e4m3fn or uint8 codes, got %s" % t.dtype)
    return t


def fp8_params(q, k, v, out, causal=False, softmax_scale=None, lse=None, window_size=(-1, -1),
               descale_q=1.0, descale_k=1.0, descale_v=1.0):
    q, k, v = _codes(q), _codes(k), _codes(v)
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if t.dim() != 4:
            raise ValueError("%s must be a [batch, seqlen, heads, head_dim] tensor" % name)
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    _expect(k, (B, Sk, Hkv, D), None, "k")
    _expect(v, (B, Sk, Hkv, D), None, "v")
    _expect(out, (B, Sq, Hq, D), torch.bfloat16, "out")
    _lse_ok(lse, (B, Hq, Sq))
    return Fp8Params(B, Sq, Sk, Hq, Hkv, D, _t4(q), _t4(k), _t4(v), _t4(out),
                     lse.data_ptr() if lse is not None else None, int(bool(causal)), _scale(softmax_scale),
                     float(descale_q), float(descale_k), float(descale_v),
                     int(window_size[0]), int(window_size[1]), None, 0)


def _fp8_workspace(p, device):
    need = int(_lib.attn_fwd_fp8_workspace_size(ctypes.byref(p)))
    if need == 0:
        p.workspace, p.workspace_bytes = None, 0
        return None
    ws = torch.empty(need + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    p.workspace = ws.data_ptr() + off
    p.workspace_bytes = need
    return ws


def attn_fwd_fp8(q, k, v, causal=False, softmax_scale=None, out=None, return_lse=False,
                 window_size=(-1, -1), descale_q=1.0, descale_k=1.0, descale_v=1.0):
    """Exact attention of e4m3 inputs (float8_e4m3fn or uint8 codes) q [B,Sq,Hq,D],
    k, v [B,Sk,Hkv,D], each element times its tensor's descale; out [B,Sq,Hq,D] bf16."""
    B, Sq, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, Sq, Hq, D), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device) if return_lse else None
    p = fp8_params(q, k, v, out, causal, softmax_scale, lse, window_size, descale_q, descale_k, descale_v)
    _on_gpu(q, k, v, out)
    ws = _fp8_workspace(p, q.device)
    _check(_lib.attn_fwd_fp8(ctypes.byref(p), _stream(q)))
    del ws
    return (out, lse) if return_lse else out


def prepare_fp8(q, k, v, out, causal=False, softmax_scale=None, lse=None, window_size=(-1, -1),
                descale_q=1.0, descale_k=1.0, descale_v=1.0):
    p = fp8_params(q, k, v, out, causal, softmax_scale, lse, window_size, descale_q, descale_k, descale_v)
    _on_gpu(q, k, v, out, lse)
    ws = _fp8_workspace(p, q.device)
    return PreparedCall(_lib.attn_fwd_fp8, p, _stream(q), (q, k, v, out, lse, ws))


# ---------------------------------------------------------------- packed sequences

def _t3(x):
    """A packed [total, H, D] tensor as the ABI's tensor block (batch stride unused)."""
    if x is None:
        return Tensor4(None, 0, 0, 0)
    if x.dim() != 3 or x.stride(2) != 1:
        raise ValueError("expected a packed [total, heads, head_dim] tensor with contiguous head_dim")
    return Tensor4(x.data_ptr(), 0, x.stride(0), x.stride(1))


def varlen_params(q, k, v, out, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, causal=False,
                  softmax_scale=None, lse=None, window_size=(-1, -1)):
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if t.dim() != 3:
            raise ValueError("%s must be a packed [total, heads, head_dim] tensor" % name)
    total_q, Hq, Dqk = q.shape
    total_k, Hkv, Dv = k.shape[0], k.shape[1], v.shape[2]
    _expect(k, (total_k, Hkv, Dqk), q.dtype, "k")
    _expect(v, (total_k, Hkv, Dv), q.dtype, "v")
    _expect(out, (total_q, Hq, Dv), q.dtype, "out")
    _lse_ok(lse, (Hq, total_q))
    for cu in (cu_seqlens_q, cu_seqlens_k):
        if not (cu.dtype == torch.int32 and cu.is_contiguous() and cu.dim() == 1 and cu.is_cuda == q.is_cuda):
            raise ValueError("cu_seqlens must be contiguous 1-d int32 tensors on q's device")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel() or cu_seqlens_q.numel() < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold B + 1 offsets")
    B = cu_seqlens_q.numel() - 1
    return VarlenParams(_dtype(q), B, total_q, total_k, int(max_seqlen_q), Hq, Hkv, Dqk, Dv,
                        _t3(q), _t3(k), _t3(v), _t3(out), cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(),
                        lse.data_ptr() if lse is not None else None, int(bool(causal)),
                        _scale(softmax_scale), int(window_size[0]), int(window_size[1]))


def attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, causal=False,
                    softmax_scale=None, out=None, return_lse=False, window_size=(-1, -1)):
    """Attention over packed sequences: q [total_q, Hq, Dqk], k/v [total_k, Hkv, D*],
    cu_seqlens_* int32 [B+1] on the device -> out [total_q, Hq, Dv] (lse [Hq, total_q])."""
    total_q, Hq, _ = q.shape
    Dv = v.shape[2]
    if out is None:
        out = torch.empty((total_q, Hq, Dv), dtype=q.dtype, device=q.device)
    lse = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device) if return_lse else None
    p = varlen_params(q, k, v, out, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, causal, softmax_scale,
                      lse, window_size)
    _on_gpu(q, k, v, out, cu_seqlens_q, cu_seqlens_k)
    _check(_lib.attn_fwd_varlen(ctypes.byref(p), _stream(q)))
    return (out, lse) if return_lse else out


def prepare_varlen(q, k, v, out, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, causal=False,
                   softmax_scale=None, lse=None, window_size=(-1, -1)):
    p = varlen_params(q, k, v, out, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, causal, softmax_scale,
                      lse, window_size)
    _on_gpu(q, k, v, out, cu_seqlens_q, cu_seqlens_k, lse)
    return PreparedCall(_lib.attn_fwd_varlen, p, _stream(q),
                        (q, k, v, out, cu_seqlens_q, cu_seqlens_k, lse))


# ---------------------------------------------------------------- kvcache

def kvcache_params(q, k_cache, v_cache, k=None, v=None, rotary_cos=None, rotary_sin=None,
                   cache_seqlens=0, causal=False, softmax_scale=None, rotary_interleaved=False,
                   out=None, lse=None, workspace=None, num_splits=0, window_size=(-1, -1)):
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("k", k), ("v", v), ("out", out)):
        if t is not None and t.dim() != 4:
            raise ValueError("%s must be a [batch, seqlen, heads, head_dim] tensor" % name)
    if (k is None) != (v is None):
        raise ValueError("k and v (the new rows) must both be given or both be None")
    B, Sq, Hq, Dqk = q.shape
    cap, Hkv, Dv = k_cache.shape[1], k_cache.shape[2], v_cache.shape[3]
    snew = 0 if k is None else k.shape[1]
    _expect(k_cache, (B, cap, Hkv, Dqk), q.dtype, "k_cache")
    _expect(v_cache, (B, cap, Hkv, Dv), q.dtype, "v_cache")
    _expect(k, (B, snew, Hkv, Dqk), q.dtype, "k")
    _expect(v, (B, snew, Hkv, Dv), q.dtype, "v")
    _expect(out, (B, Sq, Hq, Dv), q.dtype, "out")
    _lse_ok(lse, (B, Hq, Sq))
    _tables_ok(rotary_cos, rotary_sin, q.dtype, Dqk)
    _offsets_ok(cache_seqlens, B, "cache_seqlens")
    if isinstance(cache_seqlens, torch.Tensor):
        cs_scalar, cs_ptr = 0, cache_seqlens.data_ptr()
    else:
        cs_scalar, cs_ptr = int(cache_seqlens), None
    rd = seq_ro = 0
    if rotary_cos is not None:
        seq_ro, rd = rotary_cos.shape[0], 2 * rotary_cos.shape[1]
    return KVCacheParams(
        _dtype(q), B, Sq, Hq, Hkv, Dqk, Dv, cap, snew,
        _t4(q), _t4(k_cache), _t4(v_cache), _t4(k), _t4(v), _t4(out),
        cs_scalar, cs_ptr,
        rotary_cos.data_ptr() if rotary_cos is not None else None,
        rotary_sin.data_ptr() if rotary_sin is not None else None,
        rd, seq_ro, int(bool(rotary_interleaved)), int(bool(causal)), _scale(softmax_scale),
        lse.data_ptr() if lse is not None else None,
        workspace.data_ptr() if workspace is not None and workspace.numel() else None,
        workspace.numel() if workspace is not None else 0, int(num_splits),
        int(window_size[0]), int(window_size[1]))


def kvcache_workspace_size(params: KVCacheParams) -> int:
    return int(_lib.attn_fwd_kvcache_workspace_size(ctypes.byref(params)))


def attn_fwd_kvcache(q, k_cache, v_cache, k=None, v=None, rotary_cos=None, rotary_sin=None,
                     cache_seqlens=0, causal=False, softmax_scale=None, rotary_interleaved=None,
                     num_splits=0, out=None, return_lse=False, workspace=None, window_size=(-1, -1)):
    """flash_attn_with_kvcache: append k/v at cache_seqlens (in place), then attend.

    ``rotary_interleaved`` must be given whenever rotary tables are passed.
    ``window_size=(left, right)``: local attention around each query's absolute position.
    """
    if rotary_cos is not None and rotary_interleaved is None:
        raise ValueError("rotary_interleaved must be given explicitly with rotary tables")
    B, Sq, Hq, _ = q.shape
    Dv = v_cache.shape[3]
    if out is None:
        out = torch.empty((B, Sq, Hq, Dv), dtype=q.dtype, device=q.device)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device) if return_lse else None
    p = kvcache_params(q, k_cache, v_cache, k, v, rotary_cos, rotary_sin, cache_seqlens, causal,
                       softmax_scale, bool(rotary_interleaved), out, lse, None, num_splits, window_size)
    _on_gpu(q, k_cache, v_cache, k, v, rotary_cos, rotary_sin, cache_seqlens, out, workspace)
    need = kvcache_workspace_size(p)
    if workspace is None or workspace.numel() < need + 256:
        workspace = torch.empty(need + 256, dtype=torch.uint8, device=q.device)
    off = (-workspace.data_ptr()) % 256
    ws = workspace[off:]
    p.workspace = ws.data_ptr() if need else None
    p.workspace_bytes = ws.numel()
    _check(_lib.attn_fwd_kvcache(ctypes.byref(p), _stream(q)))
    return (out, lse) if return_lse else out


def attn_fwd_kvcache_noalloc(q, k_cache, v_cache, k=None, v=None, rotary_cos=None, rotary_sin=None,
                             cache_seqlens=0, causal=False, softmax_scale=None, rotary_interleaved=None,
                             num_splits=0, out=None, lse=None, window_size=(-1, -1)):
    """``attn_fwd_kvcache`` through the entry point that allocates nothing: the
    library's own 16 MiB device scratch replaces the workspace.  ``out`` (and
    ``lse`` when wanted) must be given, so this call allocates nothing either."""
    if rotary_cos is not None and rotary_interleaved is None:
        raise ValueError("rotary_interleaved must be given explicitly with rotary tables")
    if out is None:
        raise ValueError("attn_fwd_kvcache_noalloc needs a preallocated out tensor")
    p = kvcache_params(q, k_cache, v_cache, k, v, rotary_cos, rotary_sin, cache_seqlens, causal,
                       softmax_scale, bool(rotary_interleaved), out, lse, None, num_splits, window_size)
    _on_gpu(q, k_cache, v_cache, k, v, rotary_cos, rotary_sin, cache_seqlens, out, lse)
    _check(_lib.attn_fwd_kvcache_noalloc(ctypes.byref(p), _stream(q)))
    return out


# ---------------------------------------------------------------- rope

def rope_params(x, cos, sin, offsets=0, interleaved=False, conjugate=False, out=None):
    if x.dim() != 4:
        raise ValueError("x must be a [batch, seqlen, heads, head_dim] tensor")
    B, S, H, D = x.shape
    _expect(out, (B, S, H, D), x.dtype, "out")
    if cos is None or sin is None:
        raise ValueError("rope_apply needs cos and sin tables")
    _tables_ok(cos, sin, x.dtype, D)
    _offsets_ok(offsets, B, "offsets")
    if isinstance(offsets, torch.Tensor):
        off_s, off_p = 0, offsets.data_ptr()
    else:
        off_s, off_p = int(offsets), None
    return RopeParams(_dtype(x), B, S, H, D, _t4(x), _t4(out if out is not None else x),
                      cos.data_ptr(), sin.data_ptr(), 2 * cos.shape[1], cos.shape[0],
                      int(bool(interleaved)), int(bool(conjugate)), off_s, off_p)


def rope_apply(x, cos, sin, offsets=0, interleaved=False, conjugate=False, out=None, inplace=False):
    """Rotate the first 2*cos.shape[1] dims of x [B,S,H,D] at positions offsets + s."""
    if out is None:
        out = x if inplace else torch.empty_like(x)
    p = rope_params(x, cos, sin, offsets, interleaved, conjugate, out)
    _on_gpu(x, cos, sin, offsets, out)
    _check(_lib.rope_apply(ctypes.byref(p), _stream(x)))
    return out


# ---------------------------------------------------------------- prepared calls

class PreparedCall:
    """A C-ABI call whose parameter block is built once (for timing loops and graphs).

    The tensors referenced by the parameters must stay alive and in place for as
    long as the prepared call is used.
    """

    def __init__(self, fn, params, stream, keep):
        self._fn, self._p, self._stream, self._keep = fn, params, stream, keep
        self._ref = ctypes.byref(params)

    def __call__(self):
        code = self._fn(self._ref, self._stream)
        if code != ATTN_OK:
            _check(code)


def prepare_fwd(q, k, v, out, causal=False, softmax_scale=None, lse=None, window_size=(-1, -1)):
    p = fwd_params(q, k, v, out, causal, softmax_scale, lse, window_size)
    _on_gpu(q, k, v, out, lse)
    return PreparedCall(_lib.attn_fwd, p, _stream(q), (q, k, v, out, lse))


def prepare_kvcache(q, k_cache, v_cache, k, v, out, *, rotary_cos=None, rotary_sin=None,
                    cache_seqlens=0, causal=False, softmax_scale=None, rotary_interleaved=False,
                    num_splits=0, lse=None, window_size=(-1, -1)):
    p = kvcache_params(q, k_cache, v_cache, k, v, rotary_cos, rotary_sin, cache_seqlens, causal,
                       softmax_scale, rotary_interleaved, out, lse, None, num_splits, window_size)
    _on_gpu(q, k_cache, v_cache, k, v, out, rotary_cos, rotary_sin, cache_seqlens, lse)
    need = kvcache_workspace_size(p)
    ws = torch.empty(need + 256, dtype=torch.uint8, device=q.device)
    off = (-ws.data_ptr()) % 256
    p.workspace = ws.data_ptr() + off if need else None
    p.workspace_bytes = need
    return PreparedCall(_lib.attn_fwd_kvcache, p, _stream(q),
                        (q, k_cache, v_cache, k, v, out, rotary_cos, rotary_sin, cache_seqlens,
                         lse, ws))


__all__ = ["PreparedCall", "prepare_fwd", "prepare_varlen", "prepare_kvcache", "prepare_bwd", "attn_bwd",
           "BwdParams", "bwd_params", "attn_fwd", "attn_fwd_varlen",
           "attn_fwd_kvcache", "attn_fwd_kvcache_noalloc", "rope_apply", "kvcache_workspace_size", "AttnError",
           "FwdParams", "VarlenParams", "KVCacheParams", "RopeParams", "Tensor4", "fwd_params",
           "varlen_params", "kvcache_params", "Fp8Params", "fp8_params", "attn_fwd_fp8", "prepare_fp8",
           "rope_params", "lib", "EXPORTED", "LIB_PATH"]
