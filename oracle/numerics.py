"""Rounding helpers of the fp64 oracle (test infrastructure only).

fp16 and bf16 values are carried as exact fp64 numbers.  Rounding to a
working dtype follows IEEE round-to-nearest-even from fp32, the only
conversion the rounding contract of ``rope_ref`` needs:

* fp32 -> fp16: numpy's ``astype(float16)``, which rounds to nearest even
  including subnormals;
* fp32 -> bf16: written out on the fp32 bit pattern: add 0x7FFF plus the
  lowest kept bit, keep the upper 16 bits (ties go to the even pattern).
  NaN stays NaN.
"""
from __future__ import annotations

import numpy as np
import torch


def to_f64(t) -> np.ndarray:
    """Exact fp64 copy of a torch tensor (fp16/bf16/fp32 upcasts are exact) or array."""
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy().copy()
    return np.asarray(t, dtype=np.float64).copy()


def f32_to_bf16_rne_bits(x32: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns of fp32 values, round-to-nearest-even."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x32)
    if nan.any():
        r = np.where(nan, ((u >> 16) | 0x40).astype(np.uint16), r)
    return r


def bits_to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == "fp16":
        return bits.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def round_to_dtype(x, dtype: str) -> np.ndarray:
    """Round fp32 (or fp64 through fp32) values to ``dtype``; return them as fp64.

    The input is first converted to fp32 with ``astype(float32)`` (one correct
    rounding), then to the 16-bit dtype (a second correct rounding).
    """
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == "fp16":
        return x32.astype(np.float16).astype(np.float64)
    if dtype == "bf16":
        return bits_to_f64(f32_to_bf16_rne_bits(x32), "bf16")
    if dtype == "fp32":
        return x32.astype(np.float64)
    raise ValueError(dtype)


def dtype_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """uint16 bit patterns of fp64 values that are exactly representable in ``dtype``."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == "fp16":
        h = x.astype(np.float16)
        return h.view(np.uint16)
    if dtype == "bf16":
        f = x.astype(np.float32)
        return (f.view(np.uint32) >> 16).astype(np.uint16)
    raise ValueError(dtype)
