"""Rotary position embedding in the oracle (test infrastructure only).

Follows the pages' description: each 2-D chunk of a q/k vector is rotated by
an angle set by the token's absolute position m and the chunk index
(ROCm/flash-attention PR #99, "Motivation" and "A more detailed
explanation"); the angle's cos and sin are read from tables of shape
[seqlen_ro, rotary_dim/2] at row m (PR #99, rotary kernel argument review:
the tables are offset by the sequence offset, scalar or per batch).

Pairing (flash-attention issue #1402, second script, ``rotate_half`` with
doubled cos/sin tables): non-interleaved pairs dimension j with j + rd/2;
interleaved pairs 2j with 2j+1.  For pair (x1, x2) and table entries (c, s):

    y1 = x1*c - x2*s,   y2 = x1*s + x2*c

``conjugate`` rotates by the opposite angle (s -> -s).  Dimensions at or past
``rotary_dim`` pass through unchanged.

Rounding contract (the pages are silent; this is the reading taken):
inputs and tables are dtype values; each output is the exact value
x1*c - x2*s (or x1*s + x2*c) rounded once to fp32, then rounded to the dtype
(round-to-nearest-even both times).  The products of two 16-bit floats are
exact in fp64 and their difference is exact in fp64 here, so computing in fp64
and rounding with ``astype(float32)`` realises that contract.
"""
from __future__ import annotations

import numpy as np

from .numerics import round_to_dtype


def rope_ref(x, cos, sin, positions, *, rotary_dim: int, interleaved: bool,
             conjugate: bool = False, dtype: str | None = None):
    """Rotate x [B, S, H, D] (fp64 values) at positions [B, S] (ints).

    cos/sin: [seqlen_ro, rotary_dim // 2] fp64 values.
    dtype: 'fp16' / 'bf16' -> apply the rounding contract; None -> return
    the unrounded fp64 rotation (used by the invariant pins).
    """
    x = np.asarray(x, np.float64)
    cos = np.asarray(cos, np.float64)
    sin = np.asarray(sin, np.float64)
    B, S, H, D = x.shape
    rd = int(rotary_dim)
    assert rd % 2 == 0 and 0 <= rd <= D
    half = rd // 2
    pos = np.asarray(positions, np.int64).reshape(B, S)
    c = cos[pos][:, :, None, :half]          # [B, S, 1, half]
    s = sin[pos][:, :, None, :half]
    if conjugate:
        s = -s
    if interleaved:
        i1 = np.arange(half) * 2
        i2 = i1 + 1
    else:
        i1 = np.arange(half)
        i2 = i1 + half
    x1 = x[..., i1]
    x2 = x[..., i2]
    y1 = x1 * c - x2 * s
    y2 = x1 * s + x2 * c
    y = x.copy()
    y[..., i1] = y1
    y[..., i2] = y2
    if dtype is not None:
        y[..., :rd] = round_to_dtype(y[..., :rd], dtype)
    return y
