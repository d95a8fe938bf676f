"""Plain attention in fp64 (test infrastructure only).

Definition followed: the "standard attention" of the skill page "Flash
Attention - Fast Memory-Efficient Attention" (Workflow 1, Step 2 and the
accuracy check of Step 4): scores = Q K^T scaled by ``softmax_scale``,
row softmax, weights times V.  The full score matrix of one (batch, head) is
materialised; nothing is tiled, fused or reordered.

Readings of points the pages leave open:

* default scale is 1/sqrt(head_dim of q and k) (Workflow 2 Step 2 passes
  ``softmax_scale=None`` for the automatic scale; Workflow 1 divides by
  sqrt(d_k), i.e. by 8 at d=64);
* causal masking keeps key j for query i iff ``j <= i + Sk - Sq``
  (bottom-right alignment; identical to ``j <= i`` when Sq == Sk);
* grouped-query heads: q head ``h`` reads kv head ``h // (Hq // Hkv)``
  (Workflow 2 Step 3, fewer K/V heads than q heads);
* a row with no allowed key has output 0 and lse = -inf;
* ``lse`` is the natural-log sum of exp(scale * score) over allowed keys;
* local (sliding-window) attention, ``window=(left, right)`` (Workflow 2,
  Step 3: a window of tokens before and after each query, ``(-1, -1)``
  meaning none): the query at position p keeps key j iff
  ``p - left <= j <= p + right``, a side given as -1 being unbounded; with
  ``causal`` the causal test applies as well.
"""
from __future__ import annotations

import math

import numpy as np


def attention_ref(q, k, v, *, causal: bool = False, softmax_scale=None,
                  key_lens=None, q_pos=None, window=(-1, -1)):
    """Exact attention, fp64.

    q: [B, Sq, Hq, Dqk], k: [B, Sk, Hkv, Dqk], v: [B, Sk, Hkv, Dv] (fp64 arrays).
    key_lens: optional [B] ints; keys j >= key_lens[b] are excluded (the rows
      are sliced away, so their content -- NaN included -- never matters).
    q_pos: optional [B, Sq] absolute query positions for the causal and
      window tests; default ``i + Sk - Sq``.
    window: (left, right) local-attention window, -1 = unbounded side.
    Returns (out [B, Sq, Hq, Dv] fp64, lse [B, Hq, Sq] fp64).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, Sq, Hq, Dqk = q.shape
    _, Sk, Hkv, _ = k.shape
    Dv = v.shape[-1]
    assert k.shape[0] == B and v.shape[:3] == (B, Sk, Hkv) and k.shape[3] == Dqk
    assert Hq % Hkv == 0
    group = Hq // Hkv
    scale = (1.0 / math.sqrt(Dqk)) if softmax_scale is None else float(softmax_scale)
    out = np.zeros((B, Sq, Hq, Dv), np.float64)
    lse = np.full((B, Hq, Sq), -np.inf, np.float64)
    for b in range(B):
        L = Sk if key_lens is None else int(key_lens[b])
        if q_pos is None:
            pos = np.arange(Sq) + (L - Sq)
        else:
            pos = np.asarray(q_pos[b], np.int64)
        keys = np.arange(L)[None, :]
        allowed = np.ones((Sq, L), bool)
        if causal:
            allowed &= keys <= pos[:, None]
        left, right = int(window[0]), int(window[1])
        if left >= 0:
            allowed &= keys >= pos[:, None] - left
        if right >= 0:
            allowed &= keys <= pos[:, None] + right
        for h in range(Hq):
            hk = h // group
            Kb = k[b, :L, hk, :]
            Vb = v[b, :L, hk, :]
            s = scale * (q[b, :, h, :] @ Kb.T)          # [Sq, L]
            s = np.where(allowed, s, -np.inf)
            m = s.max(axis=1, initial=-np.inf)        # row max
            has = np.isfinite(m)
            msafe = np.where(has, m, 0.0)
            p = np.exp(s - msafe[:, None])            # masked -> exp(-inf) = 0
            l = p.sum(axis=1)
            o = np.zeros((Sq, Dv))
            o[has] = (p[has] @ Vb) / l[has][:, None]
            out[b, :, h, :] = o
            lse[b, h, has] = m[has] + np.log(l[has])
    return out, lse


def attention_varlen_ref(q, k, v, cu_seqlens_q, cu_seqlens_k, *, causal: bool = False,
                         softmax_scale=None, window=(-1, -1)):
    """Attention over packed variable-length sequences, fp64.

    Reading (the pages only name a variable-length mode, for the rotary kernel,
    and say decode uses the batched layout): sequence b owns query rows
    ``cu_seqlens_q[b] : cu_seqlens_q[b+1]`` of q [total_q, Hq, Dqk] and key rows
    ``cu_seqlens_k[b] : cu_seqlens_k[b+1]`` of k [total_k, Hkv, Dqk] and
    v [total_k, Hkv, Dv]; each sequence is attended exactly like one batch
    element of ``attention_ref`` (same masks, positions counted inside the
    sequence).  Returns (out [total_q, Hq, Dv], lse [Hq, total_q]).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    cq = [int(x) for x in cu_seqlens_q]
    ck = [int(x) for x in cu_seqlens_k]
    assert len(cq) == len(ck) and cq[0] == 0 and ck[0] == 0
    total_q, Hq, _ = q.shape
    Dv = v.shape[-1]
    out = np.zeros((total_q, Hq, Dv), np.float64)
    lse = np.full((Hq, total_q), -np.inf, np.float64)
    for b in range(len(cq) - 1):
        q0, q1, k0, k1 = cq[b], cq[b + 1], ck[b], ck[b + 1]
        if q1 == q0:
            continue
        o, l = attention_ref(q[None, q0:q1], k[None, k0:k1], v[None, k0:k1], causal=causal,
                             softmax_scale=softmax_scale, window=window)
        out[q0:q1] = o[0]
        lse[:, q0:q1] = l[0]
    return out, lse
