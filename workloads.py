"""Seeded synthetic inputs for exact attention and its KV-cache decode variant.

This module only draws random tensors and builds the rotary cos/sin tables that
callers pass in as inputs.  It holds none of the attention arithmetic, so both
the fp64 oracle and the HIP path can consume what it produces without sharing
any method code.

Conventions (the pages' test scripts draw with ``torch.rand`` / ``torch.randn``
and seed with ``torch.random.manual_seed(0)``; flash-attention PR #99
"Added Support for Rotary Positional Embeddings", test parametrisation diff):

* one CPU ``torch.Generator`` per workload, seeded, draws in the listed order;
* integer draws (``cache_seqlens``) first, then floating draws in fp32,
  converted to the working dtype with round-to-nearest-even (``.to(dtype)``);
* tensors use the flash layout ``[batch, seqlen, heads, head_dim]`` (the
  skill page "Flash Attention - Fast Memory-Efficient Attention", Workflow 2
  Step 2), except the empty-cache workload, which draws in
  ``[batch, heads, seqlen, dim]`` and hands over ``.transpose(1, 2)`` views
  exactly like the first script of flash-attention issue #1402;
* rotary tables are ``[seqlen_ro, rotary_dim // 2]``: the angle of position p
  and pair j is ``p * base ** (-2j / rotary_dim)``, evaluated in fp64, then cos
  and sin are rounded to the working dtype (issue #1402, second script; PR #99,
  rotary kernel argument review).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

DTYPES = {"fp16": torch.float16, "bf16": torch.bfloat16}


def rope_tables(seqlen_ro: int, rotary_dim: int, base: float, dtype: torch.dtype):
    """cos/sin tables ``[seqlen_ro, rotary_dim // 2]`` in ``dtype`` (inputs, not results)."""
    assert rotary_dim % 2 == 0
    j = np.arange(rotary_dim // 2, dtype=np.float64)
    inv_freq = base ** (-2.0 * j / rotary_dim)
    pos = np.arange(seqlen_ro, dtype=np.float64)
    ang = np.outer(pos, inv_freq)
    cos = torch.from_numpy(np.cos(ang)).to(dtype)
    sin = torch.from_numpy(np.sin(ang)).to(dtype)
    return cos.contiguous(), sin.contiguous()


@dataclass
class FwdCase:
    """Inputs for ``attn_fwd``: q [B,Sq,Hq,Dqk], k [B,Sk,Hkv,Dqk], v [B,Sk,Hkv,Dv]."""
    name: str
    dtype: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    causal: bool
    softmax_scale: float | None


@dataclass
class KVCacheCase:
    """Inputs for ``attn_fwd_kvcache``.

    q [B,Sq,Hq,Dqk]; k_cache [B,cap,Hkv,Dqk]; v_cache [B,cap,Hkv,Dv];
    k_new/v_new [B,Snew,Hkv,D*] or None; cache_seqlens an int or an int32 [B]
    tensor; rotary_cos/sin [seqlen_ro, rd/2] or None.
    """
    name: str
    dtype: str
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    k_new: torch.Tensor | None
    v_new: torch.Tensor | None
    cache_seqlens: object
    rotary_cos: torch.Tensor | None = None
    rotary_sin: torch.Tensor | None = None
    rotary_interleaved: bool = False
    causal: bool = False
    softmax_scale: float | None = None
    extra: dict = field(default_factory=dict)


def _randn(g, shape, dtype):
    return torch.randn(shape, generator=g, dtype=torch.float32).to(DTYPES[dtype])


def _rand(g, shape, dtype):
    return torch.rand(shape, generator=g, dtype=torch.float32).to(DTYPES[dtype])


# ---------------------------------------------------------------------------
# The five workloads
# ---------------------------------------------------------------------------

def kvcache_empty(seed: int = 0) -> KVCacheCase:
    """Empty cache, B=4, H=16, D=16, Sq=Snew=2, fp16, k=v=q (aliased views).

    Mirrors the first script of flash-attention issue #1402: a uniform[0,1)
    query reused as key and value, a zero cache of the same shape, the
    integer ``cache_seqlens=0``, non-causal, default scale 1/sqrt(16).
    """
    g = torch.Generator().manual_seed(seed)
    q_bhsd = _rand(g, (4, 16, 2, 16), "fp16")
    kc = torch.zeros_like(q_bhsd)
    vc = torch.zeros_like(q_bhsd)
    q = q_bhsd.transpose(1, 2)
    return KVCacheCase("kvcache_empty_b4h16d16", "fp16", q=q,
                       k_cache=kc.transpose(1, 2), v_cache=vc.transpose(1, 2),
                       k_new=q, v_new=q, cache_seqlens=0, causal=False,
                       softmax_scale=None)


def fwd_d64(causal: bool, seed: int = 0) -> FwdCase:
    """attn_fwd B=2, H=8, S=2048, D=64, fp16, N(0,1), scale 1/8."""
    g = torch.Generator().manual_seed(seed)
    q = _randn(g, (2, 2048, 8, 64), "fp16")
    k = _randn(g, (2, 2048, 8, 64), "fp16")
    v = _randn(g, (2, 2048, 8, 64), "fp16")
    return FwdCase("fwd_b2h8s2048d64" + ("_causal" if causal else ""), "fp16",
                   q, k, v, causal, 1.0 / 8.0)


def decode_gqa(seed: int = 0, capacity: int = 8192) -> KVCacheCase:
    """Decode step: B=8, Hq=32, Hkv=8, D=128, bf16, cap 8192, Snew=1, RoPE rd=128 non-interleaved."""
    g = torch.Generator().manual_seed(seed)
    seqlens = torch.randint(1, 8000, (8,), generator=g, dtype=torch.int32)
    q = _randn(g, (8, 1, 32, 128), "bf16")
    k_new = _randn(g, (8, 1, 8, 128), "bf16")
    v_new = _randn(g, (8, 1, 8, 128), "bf16")
    k_cache = _randn(g, (8, capacity, 8, 128), "bf16")
    v_cache = _randn(g, (8, capacity, 8, 128), "bf16")
    cos, sin = rope_tables(capacity, 128, 10000.0, torch.bfloat16)
    return KVCacheCase("decode_gqa_b8hq32hkv8d128", "bf16", q=q, k_cache=k_cache,
                       v_cache=v_cache, k_new=k_new, v_new=v_new,
                       cache_seqlens=seqlens, rotary_cos=cos, rotary_sin=sin,
                       rotary_interleaved=False, causal=True,
                       softmax_scale=1.0 / math.sqrt(128))


def chunked_prefill(seed: int = 0, capacity: int = 4096, snew: int = 512) -> KVCacheCase:
    """Chunked prefill: B=4, H=16, D=128, bf16, cap 4096, 512 new tokens, RoPE rd=64 interleaved, causal."""
    g = torch.Generator().manual_seed(seed)
    seqlens = torch.randint(0, 2048, (4,), generator=g, dtype=torch.int32)
    q = _randn(g, (4, snew, 16, 128), "bf16")
    k_new = _randn(g, (4, snew, 16, 128), "bf16")
    v_new = _randn(g, (4, snew, 16, 128), "bf16")
    k_cache = _randn(g, (4, capacity, 16, 128), "bf16")
    v_cache = _randn(g, (4, capacity, 16, 128), "bf16")
    cos, sin = rope_tables(capacity, 64, 10000.0, torch.bfloat16)
    return KVCacheCase("chunked_prefill_b4h16d128", "bf16", q=q, k_cache=k_cache,
                       v_cache=v_cache, k_new=k_new, v_new=v_new,
                       cache_seqlens=seqlens, rotary_cos=cos, rotary_sin=sin,
                       rotary_interleaved=True, causal=True,
                       softmax_scale=1.0 / math.sqrt(128))


def fwd_asym(seed: int = 0, S: int = 4096) -> FwdCase:
    """attn_fwd causal B=2, H=16, S=4096, Dqk=192, Dv=128, bf16, scale 1/sqrt(192)."""
    g = torch.Generator().manual_seed(seed)
    q = _randn(g, (2, S, 16, 192), "bf16")
    k = _randn(g, (2, S, 16, 192), "bf16")
    v = _randn(g, (2, S, 16, 128), "bf16")
    return FwdCase("fwd_asym_b2h16s%dd192v128" % S, "bf16", q, k, v, True,
                   1.0 / math.sqrt(192))


# ---------------------------------------------------------------------------
# Generic random cases (parity tests at oracle-friendly sizes)
# ---------------------------------------------------------------------------

def random_fwd(B, Sq, Sk, Hq, Hkv, Dqk, Dv, dtype, causal, seed=0,
               softmax_scale=None, dist="randn") -> FwdCase:
    g = torch.Generator().manual_seed(seed)
    draw = _randn if dist == "randn" else _rand
    q = draw(g, (B, Sq, Hq, Dqk), dtype)
    k = draw(g, (B, Sk, Hkv, Dqk), dtype)
    v = draw(g, (B, Sk, Hkv, Dv), dtype)
    return FwdCase("random_fwd", dtype, q, k, v, causal, softmax_scale)


@dataclass
class Fp8Case:
    """Inputs for ``attn_fwd_fp8``: e4m3 codes (uint8) q [B,Sq,Hq,D], k, v [B,Sk,Hkv,D]."""
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    causal: bool
    descale: tuple = (1.0, 1.0, 1.0)
    softmax_scale: float | None = None


def _e4m3_codes(g, shape):
    """N(0,1) draws in fp32, rounded to e4m3 (torch's float8_e4m3fn cast, RNE), as uint8 codes."""
    return torch.randn(shape, generator=g, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)


def random_fp8(B, Sq, Sk, Hq, Hkv, D, causal, seed=0, descale=(1.0, 1.0, 1.0), softmax_scale=None) -> Fp8Case:
    g = torch.Generator().manual_seed(seed)
    q = _e4m3_codes(g, (B, Sq, Hq, D))
    k = _e4m3_codes(g, (B, Sk, Hkv, D))
    v = _e4m3_codes(g, (B, Sk, Hkv, D))
    return Fp8Case(q, k, v, causal, tuple(descale), softmax_scale)


def fwd_fp8_d64(causal: bool, seed: int = 0) -> Fp8Case:
    """The headline attn_fwd shape (B=2, H=8, S=2048, D=64) with e4m3 inputs."""
    return random_fp8(2, 2048, 2048, 8, 8, 64, causal, seed=seed)


@dataclass
class VarlenCase:
    """Packed sequences: q [total_q,Hq,Dqk], k/v [total_k,Hkv,D*], cu_seqlens int32 [B+1]."""
    name: str
    dtype: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    cu_seqlens_q: torch.Tensor
    cu_seqlens_k: torch.Tensor
    max_seqlen_q: int
    causal: bool
    softmax_scale: float | None = None


def random_varlen(lens_q, lens_k, Hq, Hkv, Dqk, Dv, dtype, causal, seed=0) -> VarlenCase:
    g = torch.Generator().manual_seed(seed)
    tq, tk = int(sum(lens_q)), int(sum(lens_k))
    q = _randn(g, (tq, Hq, Dqk), dtype)
    k = _randn(g, (tk, Hkv, Dqk), dtype)
    v = _randn(g, (tk, Hkv, Dv), dtype)
    cq = torch.tensor([0] + list(np.cumsum(lens_q)), dtype=torch.int32)
    ck = torch.tensor([0] + list(np.cumsum(lens_k)), dtype=torch.int32)
    return VarlenCase("random_varlen", dtype, q, k, v, cq, ck, int(max(lens_q) if lens_q else 0), causal)


def packed_lengths(total, n, seed, min_len=1):
    """n seeded lengths >= min_len summing to total (a uniform random composition)."""
    rng = np.random.default_rng(seed)
    cuts = np.sort(rng.choice(np.arange(1, total - n * (min_len - 1)), n - 1, replace=False))
    parts = np.diff(np.concatenate([[0], cuts, [total - n * (min_len - 1)]])) + (min_len - 1)
    return [int(x) for x in parts]


def random_kvcache(B, Sq, Hq, Hkv, Dqk, Dv, capacity, dtype, *, snew, seqlens,
                   rotary_dim=0, interleaved=False, causal=True, seed=0,
                   softmax_scale=None, seqlens_as_tensor=True,
                   tail_fill=None) -> KVCacheCase:
    """Random kvcache case.  ``seqlens`` is an int or a list of B ints.

    ``tail_fill`` (e.g. ``float('nan')``) overwrites every cache row at or
    beyond ``cache_seqlens[b] + snew`` so stray reads show up in the output.
    """
    g = torch.Generator().manual_seed(seed)
    q = _randn(g, (B, Sq, Hq, Dqk), dtype)
    k_new = _randn(g, (B, snew, Hkv, Dqk), dtype) if snew else None
    v_new = _randn(g, (B, snew, Hkv, Dv), dtype) if snew else None
    k_cache = _randn(g, (B, capacity, Hkv, Dqk), dtype)
    v_cache = _randn(g, (B, capacity, Hkv, Dv), dtype)
    lens = [seqlens] * B if isinstance(seqlens, int) else list(seqlens)
    if tail_fill is not None:
        for b in range(B):
            k_cache[b, lens[b] + snew:] = tail_fill
            v_cache[b, lens[b] + snew:] = tail_fill
    cos = sin = None
    if rotary_dim:
        cos, sin = rope_tables(capacity, rotary_dim, 10000.0, DTYPES[dtype])
    cs = torch.tensor(lens, dtype=torch.int32) if seqlens_as_tensor else int(lens[0])
    return KVCacheCase("random_kvcache", dtype, q=q, k_cache=k_cache, v_cache=v_cache,
                       k_new=k_new, v_new=v_new, cache_seqlens=cs,
                       rotary_cos=cos, rotary_sin=sin, rotary_interleaved=interleaved,
                       causal=causal, softmax_scale=softmax_scale)


def seqlens_list(cs, B):
    """cache_seqlens (int or tensor) as a list of B Python ints."""
    if isinstance(cs, torch.Tensor):
        return [int(x) for x in cs.tolist()]
    return [int(cs)] * B


# Algorithmic work per workload (what the method must do, independent of tiling).

def fwd_flops(B, Sq, Sk, Hq, Dqk, Dv, causal, window=(-1, -1)):
    """2*(Dqk+Dv) flop per unmasked (query, key) pair.

    Query i sits at position p = i + Sk - Sq; causal keeps keys j <= p and a
    local window (left, right) keeps p - left <= j <= p + right (-1: unbounded).
    """
    left, right = window
    pairs = 0
    for i in range(Sq):
        p = i + Sk - Sq
        hi = Sk - 1
        if causal:
            hi = min(hi, p)
        if right >= 0:
            hi = min(hi, p + right)
        lo = 0 if left < 0 else max(0, p - left)
        pairs += max(0, hi - lo + 1)
    return 2.0 * (Dqk + Dv) * B * Hq * pairs


def bwd_flops(B, Sq, Sk, Hq, Dqk, Dv, causal, window=(-1, -1)):
    """Gradient work: five products per unmasked (query, key) pair -- S = Q K^T, dV += P^T dO,
    dP = dO V^T, dQ += dS K, dK += dS^T Q -- i.e. 2*(3*Dqk + 2*Dv) flop per pair."""
    pairs = fwd_flops(B, Sq, Sk, Hq, 1, 0, causal, window) / 2.0
    return 2.0 * (3 * Dqk + 2 * Dv) * pairs


def kvcache_pairs(lens, Sq, snew, causal):
    tot = 0
    for c in lens:
        L = c + snew
        if causal:
            tot += sum(min(L, c + i + 1) for i in range(Sq))
        else:
            tot += Sq * L
    return tot
