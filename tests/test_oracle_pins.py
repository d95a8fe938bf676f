"""Pins of the fp64 oracle to things other than itself (CPU only).

Each test ties an oracle function to a closed form, a library routine, an
invariant the pages state, a printed result of the pages, or brute force on
tiny shapes, so that a dropped term, a wrong sign, a wrong index or a
transposed operand fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import workloads as W
from oracle import (attention_bwd_ref, attention_fp8_ref, attention_ref, attention_varlen_ref, bits_to_f64,
                    dtype_bits, e4m3_decode,
                    f32_to_bf16_rne_bits, kvcache_ref, rope_ref, round_to_dtype, to_f64)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(1234)


def _rand_qkv(B, Sq, Sk, Hq, Hkv, Dqk, Dv, seed=0):
    r = np.random.default_rng(seed)
    return (r.standard_normal((B, Sq, Hq, Dqk)), r.standard_normal((B, Sk, Hkv, Dqk)),
            r.standard_normal((B, Sk, Hkv, Dv)))


# ---------------------------------------------------------------- rounding

def test_bf16_rne_matches_torch_cast():
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * 10.0,
        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -1.0 - 2.0 ** -8, 3.0e38, 1e-40, 0.0, -0.0],
                 dtype=np.float32),
    ]).astype(np.float32)
    ours = f32_to_bf16_rne_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


@pytest.mark.parametrize("dt,tdt", [("fp16", torch.float16), ("bf16", torch.bfloat16)])
def test_round_to_dtype_matches_torch(dt, tdt):
    x = rng.standard_normal(100000) * 3.0
    ours = round_to_dtype(x, dt)
    ref = torch.from_numpy(x.astype(np.float32)).to(tdt).double().numpy()
    assert np.array_equal(ours, ref)
    assert np.array_equal(bits_to_f64(dtype_bits(ours, dt), dt), ours)


# ---------------------------------------------------------------- attention

def test_one_key_output_is_v_exactly():
    # A single key gets probability 1 whatever the score (issue #1402 seqlen 1 rows).
    q, k, v = _rand_qkv(2, 3, 1, 4, 2, 8, 5)
    out, _ = attention_ref(q, k, v, causal=False, softmax_scale=0.7)
    for h in range(4):
        assert np.array_equal(out[:, :, h, :], np.broadcast_to(v[:, :1, h // 2, :], (2, 3, 5)))
    # causal, Sq == Sk: row 0 sees only key 0
    q, k, v = _rand_qkv(2, 4, 4, 2, 2, 8, 5, seed=1)
    out, _ = attention_ref(q, k, v, causal=True, softmax_scale=0.7)
    assert np.array_equal(out[:, 0], v[:, 0])


def test_two_keys_logistic_closed_form():
    q, k, v = _rand_qkv(1, 4, 2, 1, 1, 6, 3, seed=3)
    scale = 0.37
    out, _ = attention_ref(q, k, v, softmax_scale=scale)
    for i in range(4):
        d = scale * (q[0, i, 0] @ (k[0, 0, 0] - k[0, 1, 0]))
        w0 = 1.0 / (1.0 + math.exp(-d))
        exp = w0 * v[0, 0, 0] + (1 - w0) * v[0, 1, 0]
        assert np.allclose(out[0, i, 0], exp, rtol=0, atol=1e-14)


def test_probabilities_sum_to_one_and_zero_scale_mean():
    q, k, v = _rand_qkv(2, 7, 7, 2, 2, 4, 3, seed=5)
    ones = np.ones_like(v)
    for causal in (False, True):
        out, _ = attention_ref(q, k, ones, causal=causal)
        assert np.allclose(out, 1.0, rtol=0, atol=1e-13)
    out, _ = attention_ref(q, k, v, causal=False, softmax_scale=0.0)
    assert np.allclose(out, v.mean(axis=1, keepdims=True).repeat(7, axis=1), atol=1e-13)
    out, _ = attention_ref(q, k, v, causal=True, softmax_scale=0.0)
    prefix_mean = np.cumsum(v, axis=1) / np.arange(1, 8)[None, :, None, None]
    assert np.allclose(out, prefix_mean, atol=1e-13)


def test_causal_rows_equal_truncated_noncausal():
    q, k, v = _rand_qkv(1, 6, 6, 2, 1, 5, 4, seed=7)
    oc, lc = attention_ref(q, k, v, causal=True)
    on, ln = attention_ref(q, k, v, causal=False)
    assert np.allclose(oc[:, -1], on[:, -1], atol=1e-14)        # last row agrees
    for i in range(6):
        oi, li = attention_ref(q[:, i:i + 1], k[:, :i + 1], v[:, :i + 1], causal=False)
        assert np.allclose(oc[:, i:i + 1], oi, atol=1e-14)
        assert np.allclose(lc[:, :, i:i + 1], li, atol=1e-14)


def test_causal_bottom_right_alignment_and_empty_rows():
    # Sq > Sk: query i sits at key position i + Sk - Sq; rows before 0 see no key.
    q, k, v = _rand_qkv(1, 5, 3, 1, 1, 4, 2, seed=9)
    out, lse = attention_ref(q, k, v, causal=True)
    assert np.all(out[0, :2] == 0.0) and np.all(np.isneginf(lse[0, 0, :2]))
    o2, _ = attention_ref(q[:, 2:3], k[:, :1], v[:, :1])
    assert np.allclose(out[:, 2:3], o2, atol=1e-14)
    assert np.array_equal(out[0, 2, 0], v[0, 0, 0])


def test_lse_matches_scipy_logsumexp():
    q, k, v = _rand_qkv(2, 5, 9, 4, 2, 6, 3, seed=11)
    for causal in (False, True):
        _, lse = attention_ref(q, k, v, causal=causal, softmax_scale=0.5)
        for b, h, i in itertools.product(range(2), range(4), range(5)):
            s = 0.5 * (k[b, :, h // 2] @ q[b, i, h])
            if causal:
                s = s[: i + 9 - 5 + 1]
            assert abs(lse[b, h, i] - logsumexp(s)) < 1e-12


def test_gqa_equals_repeated_kv_and_head_map():
    q, k, v = _rand_qkv(2, 4, 6, 8, 2, 4, 3, seed=13)
    out, _ = attention_ref(q, k, v, causal=True)
    ref, _ = attention_ref(q, np.repeat(k, 4, axis=2), np.repeat(v, 4, axis=2), causal=True)
    assert np.allclose(out, ref, atol=1e-14)
    vconst = np.zeros_like(v)
    vconst[:, :, 1, :] = 1.0                      # kv head 1 holds ones, head 0 zeros
    o, _ = attention_ref(q, k, vconst)
    for h in range(8):
        assert np.allclose(o[:, :, h, :], 1.0 if h // 4 == 1 else 0.0, atol=1e-14)


def test_default_scale_uses_qk_head_dim():
    q, k, v = _rand_qkv(1, 3, 4, 1, 1, 9, 2, seed=15)
    a, _ = attention_ref(q, k, v)
    b, _ = attention_ref(q, k, v, softmax_scale=1.0 / 3.0)
    assert np.array_equal(a, b)


def _brute_attention(q, k, v, causal, scale, key_lens=None, q_pos=None, window=(-1, -1)):
    B, Sq, Hq, Dqk = q.shape
    Sk, Hkv, Dv = k.shape[1], k.shape[2], v.shape[3]
    out = np.zeros((B, Sq, Hq, Dv))
    for b in range(B):
        L = Sk if key_lens is None else key_lens[b]
        for h in range(Hq):
            hk = h * Hkv // Hq
            for i in range(Sq):
                pos = (i + L - Sq) if q_pos is None else q_pos[b][i]
                # a key is kept when it is no more than `left` positions before
                # the query and no more than `right` after it (-1: no limit)
                keys = [j for j in range(L) if (not causal or j <= pos)
                        and (window[0] < 0 or pos - j <= window[0])
                        and (window[1] < 0 or j - pos <= window[1])]
                sc = []
                for j in keys:
                    s = 0.0
                    for d in range(Dqk):
                        s += q[b, i, h, d] * k[b, j, hk, d]
                    sc.append(scale * s)
                if not keys:
                    continue
                mx = max(sc)
                w = [math.exp(s - mx) for s in sc]
                tot = sum(w)
                for e in range(Dv):
                    out[b, i, h, e] = sum(w[t] * v[b, j, hk, e] for t, j in enumerate(keys)) / tot
    return out


@pytest.mark.parametrize("B,Sq,Sk,Hq,Hkv,Dqk,Dv", [(2, 3, 5, 2, 1, 3, 2), (1, 5, 5, 2, 2, 4, 4),
                                                  (2, 4, 2, 4, 2, 2, 3)])
@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_tiny(B, Sq, Sk, Hq, Hkv, Dqk, Dv, causal):
    q, k, v = _rand_qkv(B, Sq, Sk, Hq, Hkv, Dqk, Dv, seed=B * 100 + Sq)
    out, _ = attention_ref(q, k, v, causal=causal, softmax_scale=0.8)
    ref = _brute_attention(q, k, v, causal, 0.8)
    assert np.allclose(out, ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- local window
# Workflow 2, Step 3 of the skill page "Flash Attention - Fast Memory-Efficient
# Attention": window_size=(left, right) keeps the tokens before and after each
# query; (-1, -1) is no window.

@pytest.mark.parametrize("window", [(0, 0), (1, 0), (2, 1), (0, 3), (-1, 1), (2, -1)])
@pytest.mark.parametrize("causal", [False, True])
def test_window_brute_force_tiny(window, causal):
    q, k, v = _rand_qkv(2, 5, 6, 2, 1, 3, 2, seed=7 + window[0] * 3 + window[1])
    out, _ = attention_ref(q, k, v, causal=causal, softmax_scale=0.7, window=window)
    ref = _brute_attention(q, k, v, causal, 0.7, window=window)
    assert np.allclose(out, ref, rtol=0, atol=1e-12)


def test_window_zero_keeps_only_own_position():
    # window (0, 0): the only key of the query at position p is key p, so the
    # output is that value row exactly (rows whose position has no key are 0)
    q, k, v = _rand_qkv(2, 4, 6, 2, 2, 3, 5, seed=3)
    out, lse = attention_ref(q, k, v, softmax_scale=0.9, window=(0, 0))
    for b in range(2):
        for i in range(4):
            p = i + 6 - 4
            assert np.array_equal(out[b, i], v[b, p])
    # Sq > Sk: the first rows sit at negative positions and see no key
    q, k, v = _rand_qkv(1, 5, 3, 1, 1, 2, 2, seed=4)
    out, lse = attention_ref(q, k, v, window=(0, 0))
    assert np.all(out[0, :2] == 0) and np.all(np.isneginf(lse[0, 0, :2]))
    assert np.array_equal(out[0, 2:, 0], v[0, :, 0])


def test_window_right_zero_is_causal_and_wide_window_is_full():
    q, k, v = _rand_qkv(2, 6, 9, 4, 2, 4, 3, seed=11)
    causal, _ = attention_ref(q, k, v, causal=True)
    right0, _ = attention_ref(q, k, v, window=(-1, 0))
    assert np.array_equal(causal, right0)
    full, _ = attention_ref(q, k, v)
    wide, _ = attention_ref(q, k, v, window=(9, 9))
    assert np.array_equal(full, wide)


def test_window_uniform_weights_average_the_window():
    # scale 0 gives every allowed key the same weight: the output is the mean
    # of the value rows inside the window (closed form)
    q, k, v = _rand_qkv(1, 7, 7, 1, 1, 2, 3, seed=5)
    left, right = 2, 1
    out, _ = attention_ref(q, k, v, softmax_scale=0.0, window=(left, right))
    for i in range(7):
        lo, hi = max(0, i - left), min(7, i + right + 1)
        assert np.allclose(out[0, i, 0], v[0, lo:hi, 0].mean(axis=0), rtol=0, atol=1e-14)


# ---------------------------------------------------------------- packed sequences

def _pack(lens_q, lens_k, Hq, Hkv, Dqk, Dv, seed):
    rng = np.random.default_rng(seed)
    cq = np.concatenate([[0], np.cumsum(lens_q)]).astype(int)
    ck = np.concatenate([[0], np.cumsum(lens_k)]).astype(int)
    q = rng.standard_normal((cq[-1], Hq, Dqk))
    k = rng.standard_normal((ck[-1], Hkv, Dqk))
    v = rng.standard_normal((ck[-1], Hkv, Dv))
    return q, k, v, cq, ck


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("window", [(-1, -1), (1, 0)])
def test_varlen_brute_force_tiny(causal, window):
    # each packed sequence is attended on its own: brute force per sequence
    q, k, v, cq, ck = _pack([3, 0, 2, 4], [2, 3, 5, 4], 2, 1, 3, 2, seed=1)
    out, lse = attention_varlen_ref(q, k, v, cq, ck, causal=causal, softmax_scale=0.6, window=window)
    for b in range(4):
        qs, ks = slice(cq[b], cq[b + 1]), slice(ck[b], ck[b + 1])
        ref = _brute_attention(q[None, qs], k[None, ks], v[None, ks], causal, 0.6, window=window)
        assert np.allclose(out[qs], ref[0], rtol=0, atol=1e-12)


def test_varlen_equal_lengths_is_the_batched_layout():
    # B sequences of one length packed back to back = a [B, S, H, D] batch
    B, S, Sk = 3, 5, 7
    q, k, v, cq, ck = _pack([S] * B, [Sk] * B, 4, 2, 3, 2, seed=2)
    out, lse = attention_varlen_ref(q, k, v, cq, ck, causal=True, softmax_scale=0.5)
    bo, bl = attention_ref(q.reshape(B, S, 4, 3), k.reshape(B, Sk, 2, 3), v.reshape(B, Sk, 2, 2),
                           causal=True, softmax_scale=0.5)
    assert np.array_equal(out, bo.reshape(B * S, 4, 2))
    assert np.array_equal(lse, bl.transpose(1, 0, 2).reshape(4, B * S))


def test_varlen_empty_key_sequence_gives_zero_rows():
    q, k, v, cq, ck = _pack([2, 3], [0, 4], 1, 1, 2, 2, seed=3)
    out, lse = attention_varlen_ref(q, k, v, cq, ck)
    assert np.all(out[:2] == 0) and np.all(np.isneginf(lse[:, :2]))
    assert np.all(np.isfinite(lse[:, 2:]))


# ---------------------------------------------------------------- gradients
# flash-attention PR #1604 "Support hdimQK != hdimV backward": dQ, dK, dV with
# Dqk != Dv.  Pinned to the forward oracle by central differences and to
# torch's float64 autograd of a plain torch formulation.

def _loss(q, k, v, dout, **kw):
    out, _ = attention_ref(q, k, v, **kw)
    return float(np.sum(out * dout))


@pytest.mark.parametrize("causal,window", [(False, (-1, -1)), (True, (-1, -1)), (False, (1, 2)),
                                           (True, (2, -1))])
def test_bwd_central_differences(causal, window):
    B, Sq, Sk, Hq, Hkv, Dqk, Dv = 1, 4, 5, 2, 1, 3, 2
    q, k, v = _rand_qkv(B, Sq, Sk, Hq, Hkv, Dqk, Dv, seed=21)
    dout = np.random.default_rng(22).standard_normal((B, Sq, Hq, Dv))
    kw = dict(causal=causal, softmax_scale=0.7, window=window)
    dq, dk, dv = attention_bwd_ref(q, k, v, dout, **kw)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = _loss(args["q"], args["k"], args["v"], dout, **kw)
            args[name] = xm
            lm = _loss(args["q"], args["k"], args["v"], dout, **kw)
            assert abs((lp - lm) / (2 * eps) - g[idx]) < 1e-7, (name, idx)


def test_bwd_matches_torch_autograd_float64():
    B, Sq, Sk, Hq, Hkv, Dqk, Dv = 2, 6, 7, 4, 2, 5, 3
    q, k, v = _rand_qkv(B, Sq, Sk, Hq, Hkv, Dqk, Dv, seed=23)
    dout = np.random.default_rng(24).standard_normal((B, Sq, Hq, Dv))
    dq, dk, dv = attention_bwd_ref(q, k, v, dout, causal=True, softmax_scale=0.4)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    kr = tk.repeat_interleave(Hq // Hkv, dim=2)
    vr = tv.repeat_interleave(Hq // Hkv, dim=2)
    s = torch.einsum("bihd,bjhd->bhij", tq, kr) * 0.4
    mask = torch.ones(Sq, Sk, dtype=torch.bool).tril(Sk - Sq)
    s = s.masked_fill(~mask, float("-inf"))
    o = torch.einsum("bhij,bjhd->bihd", torch.softmax(s, dim=-1), vr)
    o.backward(torch.tensor(dout))
    assert np.allclose(tq.grad.numpy(), dq, rtol=0, atol=1e-12)
    assert np.allclose(tk.grad.numpy(), dk, rtol=0, atol=1e-12)
    assert np.allclose(tv.grad.numpy(), dv, rtol=0, atol=1e-12)


def test_bwd_one_key_closed_form():
    # one key: P = 1 for every row, so dV = sum of dO rows and dQ = dK = 0
    q, k, v = _rand_qkv(1, 3, 1, 2, 2, 4, 3, seed=25)
    dout = np.random.default_rng(26).standard_normal((1, 3, 2, 3))
    dq, dk, dv = attention_bwd_ref(q, k, v, dout)
    assert np.allclose(dv[0, 0], dout[0].sum(axis=0), rtol=0, atol=1e-14)
    assert np.all(np.abs(dq) < 1e-15) and np.all(np.abs(dk) < 1e-15)


def test_bwd_gqa_is_sum_over_repeated_heads():
    q, k, v = _rand_qkv(1, 5, 6, 4, 2, 3, 2, seed=27)
    dout = np.random.default_rng(28).standard_normal((1, 5, 4, 2))
    dq, dk, dv = attention_bwd_ref(q, k, v, dout, causal=True)
    rq, rk, rv = attention_bwd_ref(q, np.repeat(k, 2, axis=2), np.repeat(v, 2, axis=2), dout, causal=True)
    assert np.allclose(dq, rq, rtol=0, atol=1e-13)
    assert np.allclose(dk, rk[:, :, 0::2] + rk[:, :, 1::2], rtol=0, atol=1e-13)
    assert np.allclose(dv, rv[:, :, 0::2] + rv[:, :, 1::2], rtol=0, atol=1e-13)


# ---------------------------------------------------------------- rope

def _exact_tables(seqlen, rd, base=10000.0):
    j = np.arange(rd // 2)
    ang = np.outer(np.arange(seqlen), base ** (-2.0 * j / rd))
    return np.cos(ang), np.sin(ang)


def test_rope_worked_example():
    # x = (1, 2, 3, 4), rd = 4, position 1, base 10000: angles 1 and 0.01 rad.
    x = np.array([1.0, 2.0, 3.0, 4.0]).reshape(1, 1, 1, 4)
    c, s = _exact_tables(2, 4)
    y = rope_ref(x, c, s, [[1]], rotary_dim=4, interleaved=False)[0, 0, 0]
    c1, s1, c2, s2 = math.cos(1), math.sin(1), math.cos(0.01), math.sin(0.01)
    assert np.allclose(y, [1 * c1 - 3 * s1, 2 * c2 - 4 * s2, 1 * s1 + 3 * c1, 2 * s2 + 4 * c2], atol=1e-15)
    y = rope_ref(x, c, s, [[1]], rotary_dim=4, interleaved=True)[0, 0, 0]
    assert np.allclose(y, [1 * c1 - 2 * s1, 1 * s1 + 2 * c1, 3 * c2 - 4 * s2, 3 * s2 + 4 * c2], atol=1e-15)


def test_rope_matches_rotate_half_formula_of_issue1402():
    # The second script of issue #1402 rotates with x*cos + rotate_half(x)*sin
    # where cos/sin are the half-width tables repeated twice along the last dim.
    B, S, H, D = 2, 6, 3, 16
    x = rng.standard_normal((B, S, H, D))
    c, s = _exact_tables(32, D)
    pos = rng.integers(0, 32, size=(B, S))
    cd = np.concatenate([c, c], axis=-1)[pos][:, :, None, :]
    sd = np.concatenate([s, s], axis=-1)[pos][:, :, None, :]
    rot_half = np.concatenate([-x[..., D // 2:], x[..., :D // 2]], axis=-1)
    ref = x * cd + rot_half * sd
    y = rope_ref(x, c, s, pos, rotary_dim=D, interleaved=False)
    assert np.allclose(y, ref, atol=1e-14)


@pytest.mark.parametrize("interleaved", [False, True])
def test_rope_matches_complex_multiplication(interleaved):
    B, S, H, D, rd = 1, 5, 2, 12, 8
    x = rng.standard_normal((B, S, H, D))
    c, s = _exact_tables(16, rd)
    pos = np.array([[0, 3, 7, 11, 15]])
    y = rope_ref(x, c, s, pos, rotary_dim=rd, interleaved=interleaved)
    if interleaved:
        z = x[..., 0:rd:2] + 1j * x[..., 1:rd:2]
    else:
        z = x[..., :rd // 2] + 1j * x[..., rd // 2:rd]
    theta = np.outer(np.arange(16), 10000.0 ** (-2.0 * np.arange(rd // 2) / rd))[pos][:, :, None, :]
    zr = z * np.exp(1j * theta)
    if interleaved:
        assert np.allclose(y[..., 0:rd:2], zr.real, atol=1e-14)
        assert np.allclose(y[..., 1:rd:2], zr.imag, atol=1e-14)
    else:
        assert np.allclose(y[..., :rd // 2], zr.real, atol=1e-14)
        assert np.allclose(y[..., rd // 2:rd], zr.imag, atol=1e-14)
    assert np.array_equal(y[..., rd:], x[..., rd:])            # pass-through dims


@pytest.mark.parametrize("interleaved", [False, True])
def test_rope_relative_position_identity_norm_conjugate(interleaved):
    # PR #99 "Motivation": the rotated q.k product depends only on the
    # position difference; position 0 is the identity (issue #1402, seqlen 1).
    D = 16
    c, s = _exact_tables(64, D)
    qv = rng.standard_normal((1, 1, 1, D))
    kv = rng.standard_normal((1, 1, 1, D))

    def rot(x, p):
        return rope_ref(x, c, s, [[p]], rotary_dim=D, interleaved=interleaved)[0, 0, 0]

    for delta in (0, 1, 5, 17):
        vals = [rot(qv, m + delta) @ rot(kv, m) for m in (0, 3, 20, 40)]
        assert np.ptp(vals) < 1e-12
    assert np.array_equal(rot(qv, 0), qv[0, 0, 0])
    assert abs(np.linalg.norm(rot(qv, 33)) - np.linalg.norm(qv)) < 1e-12
    back = rope_ref(rot(qv, 33).reshape(1, 1, 1, D), c, s, [[33]], rotary_dim=D,
                    interleaved=interleaved, conjugate=True)
    assert np.allclose(back[0, 0, 0], qv[0, 0, 0], atol=1e-14)


@pytest.mark.parametrize("dt,tdt", [("fp16", torch.float16), ("bf16", torch.bfloat16)])
@pytest.mark.parametrize("interleaved", [False, True])
def test_rope_rounding_contract_vs_torch_fp32(dt, tdt, interleaved):
    # Contract: round(fp32(x1*c - x2*s)) to dtype.  torch evaluates the same
    # value in fp32 arithmetic (the products of 16-bit floats are exact in
    # fp32, the difference rounds once) and casts with RNE.
    B, S, H, D, rd = 3, 40, 4, 64, 32
    cos, sin = W.rope_tables(256, rd, 10000.0, tdt)
    x = torch.randn(B, S, H, D, generator=torch.Generator().manual_seed(2)).to(tdt)
    pos = torch.randint(0, 256, (B, S), generator=torch.Generator().manual_seed(3))
    y = rope_ref(to_f64(x), to_f64(cos), to_f64(sin), pos.numpy(), rotary_dim=rd,
                 interleaved=interleaved, dtype=dt)
    cf = cos.float()[pos][:, :, None, :]
    sf = sin.float()[pos][:, :, None, :]
    xf = x.float()
    if interleaved:
        x1, x2 = xf[..., 0:rd:2], xf[..., 1:rd:2]
    else:
        x1, x2 = xf[..., :rd // 2], xf[..., rd // 2:rd]
    y1 = (x1 * cf - x2 * sf).to(tdt).double().numpy()
    y2 = (x1 * sf + x2 * cf).to(tdt).double().numpy()
    if interleaved:
        assert np.array_equal(y[..., 0:rd:2], y1) and np.array_equal(y[..., 1:rd:2], y2)
    else:
        assert np.array_equal(y[..., :rd // 2], y1) and np.array_equal(y[..., rd // 2:rd], y2)
    assert np.array_equal(y[..., rd:], to_f64(x)[..., rd:])


# ---------------------------------------------------------------- kvcache

def test_issue1402_printed_allclose_tables():
    fx = json.load(open(os.path.join(GOLDEN, "issue1402_allclose.json")))
    atols = fx["atols"]
    # First script: zero cache, cache_seqlens=0, k = v = q, no rotary.
    for seqlen in (1, 2):
        g = torch.Generator().manual_seed(seqlen)
        qh = torch.rand((4, 16, seqlen, 16), generator=g).half().transpose(1, 2)
        q = to_f64(qh)
        exact, _ = attention_ref(q, q, q)
        zeros = np.zeros_like(q)
        kv, _, _, _ = kvcache_ref(q, zeros, zeros, q, q, 0, dtype="fp16")
        got = [bool(np.allclose(kv, exact, rtol=1e-5, atol=a)) for a in atols]
        assert got == fx["no_rotary"]["seqlen_%d" % seqlen]["EFFICIENT vs FLASHCACHE"]
    # Second script: q and k rotated by the script at positions 0..seqlen-1,
    # then handed to the kvcache call together with the tables (so the kernel
    # rotates them once more); value is the unrotated draw.
    cos, sin = W.rope_tables(512, 16, 10000.0, torch.float16)
    for seqlen in (1, 2):
        g = torch.Generator().manual_seed(10 + seqlen)
        qh = torch.rand((2, 16, seqlen, 16), generator=g).half().transpose(1, 2)
        x = to_f64(qh)
        pos = np.tile(np.arange(seqlen), (2, 1))
        xr = rope_ref(x, to_f64(cos), to_f64(sin), pos, rotary_dim=16, interleaved=False, dtype="fp16")
        exact, _ = attention_ref(xr, xr, x)
        zeros = np.zeros_like(x)
        kv, _, _, _ = kvcache_ref(xr, zeros, zeros, xr, x, 0, dtype="fp16",
                                  rotary_cos=to_f64(cos), rotary_sin=to_f64(sin),
                                  rotary_interleaved=False)
        got = [bool(np.allclose(kv, exact, rtol=1e-5, atol=a)) for a in atols]
        assert got == fx["rotary"]["seqlen_%d" % seqlen]["EFFICIENT vs FLASHCACHE"]


def test_kvcache_update_rows_and_untouched_rest():
    case = W.random_kvcache(3, 4, 4, 2, 16, 8, 20, "bf16", snew=4, seqlens=[0, 5, 16],
                            rotary_dim=8, interleaved=True, seed=21)
    f = to_f64
    out, lse, kc, vc = kvcache_ref(f(case.q), f(case.k_cache), f(case.v_cache), f(case.k_new),
                                   f(case.v_new), [0, 5, 16], dtype="bf16",
                                   rotary_cos=f(case.rotary_cos), rotary_sin=f(case.rotary_sin),
                                   rotary_interleaved=True, causal=True)
    k0, v0 = f(case.k_cache), f(case.v_cache)
    for b, c in enumerate([0, 5, 16]):
        rows = np.zeros(20, bool)
        rows[c:c + 4] = True
        assert np.array_equal(kc[b, ~rows], k0[b, ~rows]) and np.array_equal(vc[b, ~rows], v0[b, ~rows])
        assert np.array_equal(vc[b, rows], f(case.v_new)[b])
        pos = np.arange(c, c + 4)[None, :]
        kr = rope_ref(f(case.k_new)[b:b + 1], f(case.rotary_cos), f(case.rotary_sin), pos,
                      rotary_dim=8, interleaved=True, dtype="bf16")
        assert np.array_equal(kc[b, rows], kr[0])
    # every stored value is a bf16 value
    assert np.array_equal(round_to_dtype(kc, "bf16"), kc)


def test_kvcache_decode_causal_equals_noncausal_and_nan_tail_ignored():
    case = W.random_kvcache(2, 1, 8, 2, 16, 16, 64, "fp16", snew=1, seqlens=[9, 40],
                            rotary_dim=16, seed=23, tail_fill=float("nan"))
    f = to_f64
    args = (f(case.q), f(case.k_cache), f(case.v_cache), f(case.k_new), f(case.v_new), [9, 40])
    kw = dict(dtype="fp16", rotary_cos=f(case.rotary_cos), rotary_sin=f(case.rotary_sin))
    oc, lc, _, _ = kvcache_ref(*args, causal=True, **kw)
    on, ln, _, _ = kvcache_ref(*args, causal=False, **kw)
    assert np.isfinite(oc).all() and np.array_equal(oc, on) and np.array_equal(lc, ln)


def test_kvcache_brute_force_tiny():
    case = W.random_kvcache(2, 3, 4, 2, 4, 3, 10, "fp16", snew=3, seqlens=[0, 4],
                            rotary_dim=4, interleaved=False, seed=25)
    f = to_f64
    for causal in (False, True):
        out, _, kc, vc = kvcache_ref(f(case.q), f(case.k_cache), f(case.v_cache), f(case.k_new),
                                     f(case.v_new), [0, 4], dtype="fp16",
                                     rotary_cos=f(case.rotary_cos), rotary_sin=f(case.rotary_sin),
                                     causal=causal, softmax_scale=0.6)
        qpos = [[c + i for i in range(3)] for c in (0, 4)]
        qr = rope_ref(f(case.q), f(case.rotary_cos), f(case.rotary_sin), np.array(qpos),
                      rotary_dim=4, interleaved=False, dtype="fp16")
        ref = _brute_attention(qr, kc, vc, causal, 0.6, key_lens=[3, 7], q_pos=qpos)
        assert np.allclose(out, ref, rtol=0, atol=1e-12)


def test_empty_cache_config_equals_plain_attention():
    # The empty-cache workload itself: appending into a zero cache at 0 and
    # attending equals plain attention on the new tokens (issue #1402, first script).
    case = W.kvcache_empty()
    f = to_f64
    out, _, kc, _ = kvcache_ref(f(case.q), f(case.k_cache), f(case.v_cache), f(case.k_new),
                                f(case.v_new), 0, dtype="fp16")
    ref, _ = attention_ref(f(case.q), f(case.k_new), f(case.v_new))
    assert np.array_equal(out, ref)
    assert np.array_equal(kc, f(case.k_new))


# ---------------------------------------------------------------- FP8 inputs
# The skill page "Flash Attention - Fast Memory-Efficient Attention", Workflow
# 3: q, k, v converted to FP8 (e4m3); the decoding is pinned to torch's own
# float8_e4m3fn conversion on all 256 codes and to hand-decoded code points.

def test_e4m3_decode_matches_torch_on_every_code():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = e4m3_decode(codes.numpy())
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


@pytest.mark.parametrize("code,value", [(0x00, 0.0), (0x38, 1.0), (0x40, 2.0), (0x3C, 1.5), (0x7E, 448.0),
                                        (0x08, 2.0 ** -6), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9),
                                        (0xC0, -2.0), (0xB8, -1.0), (0x30, 0.5)])
def test_e4m3_code_points(code, value):
    assert e4m3_decode([code])[0] == value


def test_e4m3_nan_codes_and_order():
    vals = e4m3_decode(np.arange(256))
    assert np.isnan(vals[0x7F]) and np.isnan(vals[0xFF]) and np.isnan(vals).sum() == 2
    pos = vals[:0x7F]
    assert np.all(np.diff(pos) > 0)                       # codes 0..126 increase strictly
    assert np.array_equal(vals[0x80:0xFF], -pos)           # the sign bit only flips the sign
    assert np.signbit(vals[0x80]) and vals[0x80] == 0.0


def test_e4m3_round_trip_of_representable_values():
    vals = e4m3_decode(np.arange(0x7F))
    codes = torch.from_numpy(vals).to(torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, np.arange(0x7F))


def _fp8_codes(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_fp8_attention_is_attention_of_decoded_values():
    q8, k8, v8 = _fp8_codes((1, 5, 2, 4), 31), _fp8_codes((1, 7, 1, 4), 32), _fp8_codes((1, 7, 1, 3), 33)
    out, lse = attention_fp8_ref(q8, k8, v8, causal=True)
    # brute force on the decoded values, one row at a time
    q, k, v = e4m3_decode(q8), e4m3_decode(k8), e4m3_decode(v8)
    for h in range(2):
        for i in range(5):
            s = [float(np.dot(q[0, i, h], k[0, j, 0])) / 2.0 for j in range(7) if j <= i + 2]
            w = np.exp(np.array(s) - max(s))
            want = (w[:, None] * v[0, :len(s), 0]).sum(0) / w.sum()
            assert np.allclose(out[0, i, h], want, rtol=0, atol=1e-12)
            assert abs(lse[0, h, i] - (max(s) + math.log(w.sum()))) < 1e-12


def test_fp8_descales_enter_as_score_scale_and_output_scale():
    q8, k8, v8 = _fp8_codes((2, 6, 4, 8), 41), _fp8_codes((2, 9, 2, 8), 42), _fp8_codes((2, 9, 2, 8), 43)
    out, lse = attention_fp8_ref(q8, k8, v8, descale_q=0.5, descale_k=3.0, descale_v=0.25, causal=False)
    base, base_lse = attention_ref(e4m3_decode(q8), e4m3_decode(k8), e4m3_decode(v8),
                                   softmax_scale=1.5 / math.sqrt(8))
    assert np.allclose(out, 0.25 * base, rtol=1e-13, atol=1e-15)
    assert np.allclose(lse, base_lse, rtol=1e-13, atol=1e-13)
