"""Gradients of exact attention, fp64 (test infrastructure only).

Subject of flash-attention PR #1604 "Support hdimQK != hdimV backward": the
gradients dQ, dK, dV of attention for a given upstream gradient dO, with the
key/query head size allowed to differ from the value head size.  The pages
give no formulas; these are the plain derivatives of the forward definition
(``attention_ref``), written out one (batch, head) at a time:

    S  = scale * Q K^T  (masked entries -inf),  P = softmax_rows(S),  O = P V
    dV = P^T dO
    dP = dO V^T
    dS = P * (dP - rowsum(P * dP))
    dQ = scale * dS K,   dK = scale * dS^T Q

With grouped-query heads, the dK and dV of a kv head are the sums over the q
heads that read it.  Rows without an allowed key contribute nothing.
"""
from __future__ import annotations

import math

import numpy as np


def attention_bwd_ref(q, k, v, dout, *, causal: bool = False, softmax_scale=None,
                      window=(-1, -1)):
    """q [B,Sq,Hq,Dqk], k [B,Sk,Hkv,Dqk], v [B,Sk,Hkv,Dv], dout [B,Sq,Hq,Dv] (fp64).

    Masks as in ``attention_ref`` (bottom-right causal alignment, local window).
    Returns (dq, dk, dv) in fp64 with the shapes of q, k, v.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(dout, np.float64)
    B, Sq, Hq, Dqk = q.shape
    _, Sk, Hkv, _ = k.shape
    group = Hq // Hkv
    scale = (1.0 / math.sqrt(Dqk)) if softmax_scale is None else float(softmax_scale)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    pos = np.arange(Sq) + (Sk - Sq)
    keys = np.arange(Sk)[None, :]
    allowed = np.ones((Sq, Sk), bool)
    if causal:
        allowed &= keys <= pos[:, None]
    left, right = int(window[0]), int(window[1])
    if left >= 0:
        allowed &= keys >= pos[:, None] - left
    if right >= 0:
        allowed &= keys <= pos[:, None] + right
    has = allowed.any(axis=1)
    for b in range(B):
        for h in range(Hq):
            hk = h // group
            Kb, Vb = k[b, :, hk, :], v[b, :, hk, :]
            s = np.where(allowed, scale * (q[b, :, h, :] @ Kb.T), -np.inf)
            m = np.where(has, s.max(axis=1, initial=-np.inf), 0.0)
            e = np.exp(s - m[:, None])
            l = e.sum(axis=1)
            p = np.zeros_like(e)
            p[has] = e[has] / l[has][:, None]
            dO = do[b, :, h, :]
            dv[b, :, hk, :] += p.T @ dO
            dp = dO @ Vb.T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dq[b, :, h, :] = scale * (ds @ Kb)
            dk[b, :, hk, :] += scale * (ds.T @ q[b, :, h, :])
    return dq, dk, dv
