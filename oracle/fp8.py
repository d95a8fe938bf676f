"""Exact attention of FP8 (e4m3) inputs, fp64 (test infrastructure only).

The skill page "Flash Attention - Fast Memory-Efficient Attention", Workflow 3
(H100 FP8 optimization with FlashAttention-3), converts q, k and v to FP8 and
runs attention on them.  The page breaks off inside the conversion step, so
the format and the scaling are readings:

* the 8-bit format is e4m3 in its "fn" form: 1 sign bit, 4 exponent bits with
  bias 7, 3 mantissa bits, subnormals when the exponent field is 0, no
  infinities, and the all-ones exponent-and-mantissa pattern (S.1111.111) as
  NaN, so the largest finite magnitude is 1.75 * 2^8 = 448;
* each input tensor carries one descale factor: an element stands for
  decode(code) * descale;
* the result is the plain attention (``attention_ref``) of the decoded,
  descaled tensors, with the default scale 1/sqrt(head_dim).
"""
from __future__ import annotations

import numpy as np

from .attention import attention_ref


def e4m3_decode(codes) -> np.ndarray:
    """uint8 e4m3 codes -> fp64 values, from the bit-field definition."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    subnormal = (m / 8.0) * 2.0 ** -6
    mag = np.where(e == 0, subnormal, normal)
    mag = np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, mag)
    return sign * mag


def attention_fp8_ref(q8, k8, v8, *, descale_q: float = 1.0, descale_k: float = 1.0,
                      descale_v: float = 1.0, causal: bool = False, softmax_scale=None,
                      window=(-1, -1)):
    """q8 [B,Sq,Hq,D], k8 [B,Sk,Hkv,D], v8 [B,Sk,Hkv,Dv]: uint8 e4m3 codes.

    Returns (out, lse) of ``attention_ref`` on the decoded tensors times their
    descale factors.
    """
    q = e4m3_decode(q8) * float(descale_q)
    k = e4m3_decode(k8) * float(descale_k)
    v = e4m3_decode(v8) * float(descale_v)
    return attention_ref(q, k, v, causal=causal, softmax_scale=softmax_scale, window=window)
