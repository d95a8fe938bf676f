"""KV-cache attention in the oracle (test infrastructure only).

What ``flash_attn_with_kvcache`` computes, as the pages describe it
(flash-attention issue #1402, both scripts; ROCm/flash-attention PR #99):

1. per batch b the cache already holds ``c_b = cache_seqlens[b]`` rows
   (an int applies to every batch, a tensor gives one value per batch);
2. the new keys are rotated (RoPE, when tables are given) at absolute
   positions c_b + i and written, with the raw new values, to cache rows
   [c_b, c_b + Snew); no other row changes, and old rows are not re-rotated;
3. the query tokens, at positions c_b + i, are rotated with the same tables
   and rounded to the dtype; they are not written anywhere;
4. attention of the rotated queries over cache rows [0, c_b + Snew), causal
   on absolute position (key j allowed iff j <= c_b + i) when ``causal``,
   and restricted to the local window around the query's absolute position
   when ``window`` is given.

Step 4 is ``attention_ref``; step 2/3's rotation is ``rope_ref`` with its
rounding contract.
"""
from __future__ import annotations

import numpy as np

from .attention import attention_ref
from .rope import rope_ref


def kvcache_ref(q, k_cache, v_cache, k_new, v_new, cache_seqlens, *, dtype: str,
                rotary_cos=None, rotary_sin=None, rotary_interleaved=False,
                causal=False, softmax_scale=None, window=(-1, -1)):
    """All array arguments are fp64 values of ``dtype`` tensors.

    q [B,Sq,Hq,Dqk]; k_cache [B,cap,Hkv,Dqk]; v_cache [B,cap,Hkv,Dv];
    k_new [B,Snew,Hkv,Dqk] / v_new [B,Snew,Hkv,Dv] or None;
    cache_seqlens: int or sequence of B ints; rotary tables [seqlen_ro, rd/2]
    or None.
    Returns (out fp64 [B,Sq,Hq,Dv], lse [B,Hq,Sq], k_cache', v_cache').
    """
    q = np.asarray(q, np.float64)
    kc = np.array(k_cache, np.float64, copy=True)
    vc = np.array(v_cache, np.float64, copy=True)
    B, Sq, Hq, Dqk = q.shape
    cap = kc.shape[1]
    if np.isscalar(cache_seqlens):
        lens = [int(cache_seqlens)] * B
    else:
        lens = [int(x) for x in np.asarray(cache_seqlens).reshape(-1)]
    snew = 0 if k_new is None else np.asarray(k_new).shape[1]
    rot = rotary_cos is not None
    rd = 2 * np.asarray(rotary_cos).shape[1] if rot else 0

    qpos = np.array([[lens[b] + i for i in range(Sq)] for b in range(B)], np.int64)
    qr = q
    if rot:
        qr = rope_ref(q, rotary_cos, rotary_sin, qpos, rotary_dim=rd,
                      interleaved=rotary_interleaved, dtype=dtype)
    if snew:
        kn = np.asarray(k_new, np.float64)
        vn = np.asarray(v_new, np.float64)
        if rot:
            npos = np.array([[lens[b] + i for i in range(snew)] for b in range(B)], np.int64)
            kn = rope_ref(kn, rotary_cos, rotary_sin, npos, rotary_dim=rd,
                          interleaved=rotary_interleaved, dtype=dtype)
        for b in range(B):
            assert lens[b] + snew <= cap
            kc[b, lens[b]:lens[b] + snew] = kn[b]
            vc[b, lens[b]:lens[b] + snew] = vn[b]
    key_lens = [lens[b] + snew for b in range(B)]
    out, lse = attention_ref(qr, kc, vc, causal=causal, softmax_scale=softmax_scale,
                             key_lens=key_lens, q_pos=qpos, window=window)
    return out, lse, kc, vc
