"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Bars (stated for this method): outputs within max-abs 2e-3 (fp16) or 1.5e-2
(bf16) of the fp64 oracle, fp32 accumulation inside; KV-cache contents and
the positions written bit-exact; rotary outputs bit-exact (they are a single
rounding of an exactly-defined value).  Inputs are seeded (workloads.py).
"""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import (attention_bwd_ref, attention_fp8_ref, attention_ref, attention_varlen_ref, dtype_bits,
                    kvcache_ref, rope_ref, to_f64)

pytestmark = pytest.mark.gpu
TOL = {"fp16": 2e-3, "bf16": 1.5e-2}
# lse is ln(sum of P) with P rounded to the working type (the same weights as
# the numerator), so with few keys per row it can be off by up to
# ln(1 + u): u = 2^-11 (fp16), 2^-8 (bf16, 8 significant bits)
LSE_TOL = {"fp16": 2e-3, "bf16": 4.1e-3}
DEV = "cuda"


@pytest.fixture(autouse=True)
def _announce(request):
    print("\n[gpu-case] %s" % request.node.nodeid, flush=True)
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    yield
    torch.cuda.synchronize()


def E():
    import exact_attention_qk_amd as mod
    return mod


def dev(t):
    return None if t is None else t.to(DEV)


def maxabs(gpu_out, ref):
    g = to_f64(gpu_out.float().cpu())
    assert np.isfinite(g).all(), "non-finite output"
    return float(np.max(np.abs(g - ref))) if g.size else 0.0


def guarded_empty(shape, dtype, fill=-7.0):
    """A tensor view with canary elements before and after it in the same allocation."""
    n = int(np.prod(shape))
    buf = torch.full((n + 256,), fill, dtype=dtype, device=DEV)
    return buf, buf[128:128 + n].view(shape)


def canaries_intact(buf, n, fill=-7.0):
    b = buf.float().cpu()
    return bool((b[:128] == fill).all() and (b[128 + n:] == fill).all())


# ---------------------------------------------------------------- attn_fwd

DIMS = [(16, 16), (64, 64), (128, 128), (192, 128)]


def _fwd_check(case, sample_rows=None, tol=None, return_lse=False, window=(-1, -1)):
    q, k, v = dev(case.q), dev(case.k), dev(case.v)
    B, Sq, Hq, _ = q.shape
    Dv = v.shape[3]
    buf, out = guarded_empty((B, Sq, Hq, Dv), q.dtype)
    res = E().attn_fwd(q, k, v, causal=case.causal, softmax_scale=case.softmax_scale, out=out,
                       return_lse=return_lse, window_size=window)
    torch.cuda.synchronize()
    assert canaries_intact(buf, out.numel())
    qf, kf, vf = to_f64(case.q), to_f64(case.k), to_f64(case.v)
    Sk = kf.shape[1]
    if sample_rows is None:
        ref, lse = attention_ref(qf, kf, vf, causal=case.causal, softmax_scale=case.softmax_scale,
                                 window=window)
        got = out
    else:
        rows = np.asarray(sample_rows)
        pos = np.tile(rows + Sk - Sq, (B, 1))
        ref, lse = attention_ref(qf[:, rows], kf, vf, causal=case.causal,
                                 softmax_scale=case.softmax_scale, q_pos=pos, window=window)
        got = out[:, torch.as_tensor(rows, device=DEV)]
    err = maxabs(got, ref)
    assert err <= (tol or TOL[case.dtype]), "max abs err %.3e" % err
    if return_lse:
        l = res[1].cpu().double().numpy()
        if sample_rows is not None:
            l = l[:, :, rows]
        fin = np.isfinite(lse)
        assert np.array_equal(fin, np.isfinite(l))
        assert np.max(np.abs(l[fin] - lse[fin])) < LSE_TOL[case.dtype]
    return err


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("dqk,dv", DIMS)
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_multi_tile_ragged(dtype, dqk, dv, causal):
    # 200 rows/keys: two 128-row query tiles and four 64-key tiles, ragged tails; GQA 4:2.
    case = W.random_fwd(2, 200, 200, 4, 2, dqk, dv, dtype, causal, seed=dqk + causal)
    _fwd_check(case, return_lse=True)


@pytest.mark.parametrize("sq,sk", [(100, 333), (300, 77), (1, 129), (129, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_sq_ne_sk(sq, sk, causal):
    # causal uses bottom-right alignment; rows with no allowed key give 0 / -inf lse
    case = W.random_fwd(1, sq, sk, 2, 1, 64, 64, "fp16", causal, seed=sq * 7 + sk)
    _fwd_check(case, return_lse=True)


def test_fwd_strided_transposed_views():
    g = torch.Generator().manual_seed(5)
    q = torch.randn(2, 4, 150, 128, generator=g).to(torch.bfloat16)
    k = torch.randn(2, 4, 150, 128, generator=g).to(torch.bfloat16)
    v = torch.randn(2, 4, 150, 128, generator=g).to(torch.bfloat16)
    case = W.FwdCase("strided", "bf16", q.transpose(1, 2), k.transpose(1, 2), v.transpose(1, 2),
                     True, None)
    assert not case.q.is_contiguous()
    _fwd_check(case)


def test_fwd_empty_and_no_keys():
    q = torch.randn(1, 5, 2, 64, device=DEV).half()
    k = torch.zeros(1, 0, 2, 64, device=DEV).half()
    out, lse = E().attn_fwd(q, k, k, return_lse=True)
    torch.cuda.synchronize()
    assert (out.float() == 0).all() and torch.isinf(lse).all()
    e = E().attn_fwd(q[:, :0], q, q)
    assert e.shape[1] == 0


def test_fwd_softmax_scale_zero_is_mean():
    case = W.random_fwd(1, 64, 96, 2, 2, 64, 64, "fp16", False, seed=3, softmax_scale=0.0)
    _fwd_check(case)


@pytest.mark.parametrize("scale", [1.0, 1.5, -0.1])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_fwd_d64_scale_values(scale, dtype):
    # positive scales up to and beyond 1 take the fast path, non-positive ones the general path
    case = W.random_fwd(1, 200, 333, 2, 2, 64, 64, dtype, False, seed=11, softmax_scale=scale)
    _fwd_check(case, return_lse=True)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_fwd_d64_growing_scores(dtype):
    # scores grow along the keys (|lse| up to 15), so rows raise their running max on many
    # key tiles; large scores also expose any rounding of q or of the scaled scores
    case = W.random_fwd(1, 130, 700, 2, 2, 64, 64, dtype, False, seed=12)
    ramp = torch.linspace(0.5, 4.0, 700).view(1, 700, 1, 1)
    case.k = (case.k.float() * ramp).to(case.k.dtype)
    _fwd_check(case, return_lse=True)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_fwd_d64_large_queries(dtype):
    # q three times the unit normal: scores of tens, as in trained models
    case = W.random_fwd(1, 256, 512, 2, 2, 64, 64, dtype, False, seed=5)
    case.q = (case.q.float() * 3).to(case.q.dtype)
    _fwd_check(case, return_lse=True)


def test_fwd_ones_v_gives_ones():
    # probabilities sum to one: V = 1 gives O = 1 for every row
    case = W.random_fwd(1, 130, 130, 2, 1, 128, 128, "bf16", True, seed=4)
    case.v = torch.ones_like(case.v)
    out = E().attn_fwd(dev(case.q), dev(case.k), dev(case.v), causal=True)
    torch.cuda.synchronize()
    assert (out.float() - 1).abs().max().item() <= 2 ** -7


def test_fwd_first_causal_row_is_v0_bitwise():
    case = W.random_fwd(2, 256, 256, 4, 4, 64, 64, "fp16", True, seed=8)
    out = E().attn_fwd(dev(case.q), dev(case.k), dev(case.v), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(out[:, 0].cpu(), case.v[:, 0])


def test_skill_page_fp16_accuracy_check():
    # Workflow 1 Step 4 of the skill page: fp16, B=1, H=8, S=512, D=64, max diff below 1e-3.
    case = W.random_fwd(1, 512, 512, 8, 8, 64, 64, "fp16", False, seed=0, softmax_scale=1 / 8)
    assert _fwd_check(case) < 1e-3


@pytest.mark.parametrize("causal", [False, True])
def test_workload_fwd_d64_full(causal):
    case = W.fwd_d64(causal)
    _fwd_check(case, return_lse=True)


def test_workload_fwd_asym_sampled_rows():
    # fast pre-check of the largest configuration on 128 of its 4096 rows
    case = W.fwd_asym()
    rows = sorted(set(list(range(0, 8)) + list(range(4088, 4096)) +
                      list(np.random.default_rng(0).choice(4096, 112, replace=False))))
    _fwd_check(case, sample_rows=rows)


def test_workload_fwd_asym_full():
    # every output element and lse of the largest configuration (causal B=2 H=16
    # S=4096, Dqk=192 Dv=128, bf16; flash-attention PR #1604's head sizes), in the
    # launch configuration the benchmark times; the fp64 oracle takes ~20 s here
    err = _fwd_check(W.fwd_asym(), return_lse=True)
    print("fwd_asym full max abs err %.3e" % err, flush=True)


# ---------------------------------------------------------------- kvcache

def _kv_run(case, num_splits=0, return_lse=True, share_q=False, window=(-1, -1), workspace=None):
    """Run the HIP kvcache path on device copies; returns (out, lse, k_cache, v_cache)."""
    q = dev(case.q)
    if share_q:
        kn = vn = q                  # one tensor passed as q, k and v (issue #1402)
    else:
        kn, vn = dev(case.k_new), dev(case.v_new)
    kc, vc = dev(case.k_cache), dev(case.v_cache)
    cs = dev(case.cache_seqlens) if isinstance(case.cache_seqlens, torch.Tensor) else case.cache_seqlens
    out, lse = E().attn_fwd_kvcache(q, kc, vc, kn, vn, rotary_cos=dev(case.rotary_cos),
                                    rotary_sin=dev(case.rotary_sin), cache_seqlens=cs,
                                    causal=case.causal, softmax_scale=case.softmax_scale,
                                    rotary_interleaved=case.rotary_interleaved,
                                    num_splits=num_splits, return_lse=True, window_size=window,
                                    workspace=workspace)
    torch.cuda.synchronize()
    return out, lse, kc, vc


def _kv_oracle(case, window=(-1, -1)):
    f = to_f64
    B = case.q.shape[0]
    lens = W.seqlens_list(case.cache_seqlens, B)
    return kvcache_ref(f(case.q), f(case.k_cache), f(case.v_cache),
                       None if case.k_new is None else f(case.k_new),
                       None if case.v_new is None else f(case.v_new),
                       lens if isinstance(case.cache_seqlens, torch.Tensor) else case.cache_seqlens,
                       dtype=case.dtype,
                       rotary_cos=None if case.rotary_cos is None else f(case.rotary_cos),
                       rotary_sin=None if case.rotary_sin is None else f(case.rotary_sin),
                       rotary_interleaved=case.rotary_interleaved, causal=case.causal,
                       softmax_scale=case.softmax_scale, window=window)


def _bits_equal(gpu_cache, ref_cache, dtype):
    g = gpu_cache.cpu().view(torch.int16).numpy().view(np.uint16)
    r = dtype_bits(ref_cache, dtype)
    same = (g == r)
    # NaN sentinels compare as NaN == NaN here: both sides must be NaN
    nan_ref = np.isnan(ref_cache)
    if nan_ref.any():
        gv = to_f64(gpu_cache.float().cpu())
        same = same | (nan_ref & np.isnan(gv))
    return bool(same.all())


def _kv_check(case, num_splits=0, share_q=False, window=(-1, -1), workspace=None):
    out, lse, kc, vc = _kv_run(case, num_splits, share_q=share_q, window=window, workspace=workspace)
    ref, rlse, rkc, rvc = _kv_oracle(case, window)
    err = maxabs(out, ref)
    assert err <= TOL[case.dtype], "max abs err %.3e" % err
    assert _bits_equal(kc, rkc, case.dtype), "k_cache differs from the oracle"
    assert _bits_equal(vc, rvc, case.dtype), "v_cache differs from the oracle"
    l = lse.cpu().double().numpy()
    fin = np.isfinite(rlse)
    assert np.array_equal(fin, np.isfinite(l))
    assert np.max(np.abs(l[fin] - rlse[fin])) < LSE_TOL[case.dtype]
    return out, err


def test_workload_kvcache_empty():
    case = W.kvcache_empty()
    out, _ = _kv_check(case, share_q=True)
    # an empty cache with cache_seqlens=0 equals plain attention on the new tokens
    q = dev(case.q)
    plain = E().attn_fwd(q, q, q)
    torch.cuda.synchronize()
    diff = (plain.float() - out.float()).abs().max().item()
    assert diff <= 2 ** -11, diff       # at most one fp16 ulp of values below 1


def test_workload_decode_gqa():
    _kv_check(W.decode_gqa())


def test_workload_chunked_prefill():
    _kv_check(W.chunked_prefill())


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("dqk,dv", DIMS)
def test_kvcache_decode_nan_tail(dtype, dqk, dv):
    case = W.random_kvcache(3, 1, 8, 2, dqk, dv, 300, dtype, snew=1, seqlens=[0, 37, 298],
                            rotary_dim=dqk // 2, interleaved=dqk == 64, seed=dqk,
                            tail_fill=float("nan"))
    _kv_check(case)


@pytest.mark.parametrize("rot", [0, 64])
def test_kvcache_chunk_nan_tail(rot):
    case = W.random_kvcache(2, 70, 4, 4, 128, 128, 400, "bf16", snew=70, seqlens=[0, 201],
                            rotary_dim=rot, interleaved=True, seed=11, tail_fill=float("nan"))
    _kv_check(case)


@pytest.mark.parametrize("causal", [False, True])
def test_kvcache_decode_two_tokens_full_rows(causal):
    # Sq = 2 with 8 q heads per kv head: R = 16 rows, the decode path's maximum
    case = W.random_kvcache(2, 2, 16, 2, 64, 64, 256, "fp16", snew=2, seqlens=[5, 190],
                            rotary_dim=64, causal=causal, seed=13)
    _kv_check(case)


def test_kvcache_decode_many_splits():
    # capacity 131072 with one kv head per batch: the kernels size the splits
    # from the two lengths (160 keys), so the merge combines about 820 splits
    # per row of the first batch, 32 per memory round trip; the second batch
    # is half full
    case = W.random_kvcache(2, 1, 8, 1, 128, 128, 131072, "bf16", snew=1, seqlens=[131071, 70000],
                            rotary_dim=128, seed=73)
    _kv_check(case)


def test_kvcache_decode_more_than_64_batches():
    # 70 batches: the split sizing and the workgroup-to-batch search read the
    # lengths 64 at a time; empty, one-key and full caches mixed
    g = torch.Generator().manual_seed(91)
    lens = torch.randint(0, 255, (70,), generator=g).tolist()
    lens[0], lens[5], lens[69] = 0, 255, 1
    case = W.random_kvcache(70, 1, 8, 2, 64, 64, 256, "fp16", snew=1, seqlens=lens, rotary_dim=64, seed=92)
    _kv_check(case)
    _kv_check(case, num_splits=3)


@pytest.mark.parametrize("num_splits", [0, 9])
def test_kvcache_merge_ignores_stale_workspace(num_splits):
    # the merge requests its first 32 splits before it knows how many a row
    # has; a workspace full of NaN bits (left by nothing this call writes)
    # must not leak into rows with fewer splits: lengths from 0 to 3000
    case = W.random_kvcache(4, 1, 8, 2, 128, 128, 4096, "bf16", snew=1, seqlens=[3000, 40, 0, 700],
                            rotary_dim=64, seed=95)
    ws = torch.full((64 << 20,), 0xFF, dtype=torch.uint8, device="cuda")
    _kv_check(case, num_splits=num_splits, workspace=ws)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_kvcache_decode_large_scores(dtype):
    # q eight times the unit normal: scores of several hundred in log2 units,
    # so every step's row max must be the true one (a wrong max overflows the
    # exponentials); 16 query rows per kv head, several splits per row
    case = W.random_kvcache(2, 1, 16, 1, 128, 128, 1024, dtype, snew=1, seqlens=[1000, 300],
                            rotary_dim=128, seed=91)
    case.q = (case.q.float() * 8).to(case.q.dtype)
    _kv_check(case)
    _kv_check(case, num_splits=7)


def test_kvcache_scalar_and_tensor_seqlens_agree():
    a = W.random_kvcache(2, 1, 4, 1, 128, 128, 512, "bf16", snew=1, seqlens=[300, 300],
                         rotary_dim=128, seed=15)
    b = W.random_kvcache(2, 1, 4, 1, 128, 128, 512, "bf16", snew=1, seqlens=[300, 300],
                         rotary_dim=128, seed=15, seqlens_as_tensor=False)
    oa, _, ka, _ = _kv_run(a)
    ob, _, kb, _ = _kv_run(b)
    assert torch.equal(oa, ob) and torch.equal(ka, kb)
    _kv_check(b)


def test_kvcache_one_split_matches_auto():
    case = W.random_kvcache(2, 1, 8, 2, 128, 128, 2048, "bf16", snew=1, seqlens=[1500, 2000],
                            seed=17)
    o1, _, _, _ = _kv_run(case, num_splits=1)
    oa, _, _, _ = _kv_run(case, num_splits=0)
    assert (o1.float() - oa.float()).abs().max().item() <= 2 ** -6
    _kv_check(case, num_splits=1)
    _kv_check(case, num_splits=5)


def test_kvcache_gqa_equals_repeated_mha():
    case = W.random_kvcache(2, 1, 8, 2, 64, 64, 256, "fp16", snew=1, seqlens=[100, 200], seed=19)
    o_gqa, _, _, _ = _kv_run(case)
    rep = W.KVCacheCase("rep", "fp16", case.q, case.k_cache.repeat_interleave(4, dim=2),
                        case.v_cache.repeat_interleave(4, dim=2),
                        case.k_new.repeat_interleave(4, dim=2), case.v_new.repeat_interleave(4, dim=2),
                        case.cache_seqlens, causal=True)
    o_mha, _, _, _ = _kv_run(rep)
    assert (o_gqa.float() - o_mha.float()).abs().max().item() <= 2e-3


def test_kvcache_no_new_tokens():
    case = W.random_kvcache(2, 1, 4, 2, 128, 128, 128, "bf16", snew=0, seqlens=[1, 77],
                            rotary_dim=128, seed=21)
    _kv_check(case)


def test_kvcache_fused_rope_equals_unfused():
    case = W.random_kvcache(2, 40, 4, 2, 128, 128, 256, "bf16", snew=40, seqlens=[3, 150],
                            rotary_dim=64, interleaved=False, seed=23)
    out_f, _, kc_f, vc_f = _kv_run(case)
    mod = E()
    cs = dev(case.cache_seqlens)
    q_r = mod.rope_apply(dev(case.q), dev(case.rotary_cos), dev(case.rotary_sin), cs, False)
    k_r = mod.rope_apply(dev(case.k_new), dev(case.rotary_cos), dev(case.rotary_sin), cs, False)
    kc, vc = dev(case.k_cache), dev(case.v_cache)
    out_u = mod.attn_fwd_kvcache(q_r, kc, vc, k_r, dev(case.v_new), cache_seqlens=cs, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(kc_f, kc) and torch.equal(vc_f, vc)
    assert torch.equal(out_f, out_u)


@pytest.mark.parametrize("snew,rot", [(1, 128), (64, 64), (64, 0)])
def test_kvcache_fills_cache_exactly(snew, rot):
    # c_b + Snew == capacity: the appended rows are the last rows of the cache,
    # the rotary tables' last row is used, and nothing past the cache is touched
    cap = 320
    case = W.random_kvcache(3, snew, 8, 2, 128, 128, cap, "bf16", snew=snew, seqlens=[cap - snew, 0, 17],
                            rotary_dim=rot, interleaved=snew > 1, seed=47 + snew)
    _kv_check(case)
    _kv_check(case, num_splits=4)


def test_attn_check_rejects_lengths_that_do_not_fit(monkeypatch):
    # ATTN_CHECK=1: the call copies the device-side lengths to the host and
    # refuses them before anything is launched, so the caches stay untouched
    monkeypatch.setenv("ATTN_CHECK", "1")
    case = W.random_kvcache(2, 1, 4, 2, 64, 64, 64, "fp16", snew=1, seqlens=[10, 64], seed=49)
    kc, vc = dev(case.k_cache), dev(case.v_cache)
    with pytest.raises(E().AttnError) as ei:
        E().attn_fwd_kvcache(dev(case.q), kc, vc, dev(case.k_new), dev(case.v_new),
                             cache_seqlens=dev(case.cache_seqlens), causal=True)
    torch.cuda.synchronize()
    assert ei.value.code == -6
    assert torch.equal(kc.cpu(), case.k_cache) and torch.equal(vc.cpu(), case.v_cache)
    # lengths that fit pass the same check and give the oracle's result
    _kv_check(W.random_kvcache(2, 1, 4, 2, 64, 64, 64, "fp16", snew=1, seqlens=[10, 63], seed=49))
    # packed sequences: offsets that do not end at the packed row count are refused
    vc_case = W.random_varlen([5, 7], [5, 7], 2, 2, 64, 64, "fp16", False, seed=51)
    bad = vc_case.cu_seqlens_q.clone()
    bad[-1] = bad[-1] - 1
    with pytest.raises(E().AttnError) as ei:
        E().attn_fwd_varlen(dev(vc_case.q), dev(vc_case.k), dev(vc_case.v), dev(bad), dev(vc_case.cu_seqlens_k),
                            vc_case.max_seqlen_q)
    assert ei.value.code == -2


# ---------------------------------------------------------------- local window

WINDOWS = [(0, 0), (16, 0), (37, 5), (-1, 20), (100, -1), (3, 70)]


@pytest.mark.parametrize("window", WINDOWS)
@pytest.mark.parametrize("dqk,dv", [(64, 64), (128, 128), (192, 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_window(window, dqk, dv, causal):
    # 300 rows/keys: several query and key tiles, a ragged tail; the band of
    # each query tile starts and ends inside key tiles
    dtype = "fp16" if dqk == 64 else "bf16"
    case = W.random_fwd(2, 300, 300, 4, 2, dqk, dv, dtype, causal, seed=dqk + 3 * causal + window[0])
    _fwd_check(case, return_lse=True, window=window)


@pytest.mark.parametrize("window", [(0, 0), (50, 3), (-1, 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_window_sq_ne_sk(window, causal):
    # bottom-right positions: early rows of Sq > Sk have keys only inside the window
    for sq, sk in [(100, 333), (300, 77)]:
        case = W.random_fwd(1, sq, sk, 2, 1, 64, 64, "fp16", causal, seed=sq + sk)
        _fwd_check(case, return_lse=True, window=window)


@pytest.mark.parametrize("window", [(0, 0), (200, 0), (700, -1), (64, 16)])
@pytest.mark.parametrize("causal", [False, True])
def test_kvcache_decode_window(window, causal):
    # decode splits start at the window's first key; cache rows outside it are NaN-free noise
    case = W.random_kvcache(3, 1, 8, 2, 128, 128, 1024, "bf16", snew=1, seqlens=[700, 33, 1000],
                            rotary_dim=128, causal=causal, seed=29)
    _kv_check(case, window=window)
    _kv_check(case, window=window, num_splits=3)


@pytest.mark.parametrize("sq", [150, 64])
def test_kvcache_chunk_d64_longest_first_pairs(sq):
    # head size 64 with per-batch lengths: each workgroup takes the (batch,
    # query tile) group of its rank in key-tile order and then the group of the
    # mirrored rank; 3 batches of ceil(sq/64) tiles give an odd group count at
    # sq=150 (the middle group runs alone) and an even one at sq=64
    case = W.random_kvcache(3, sq, 8, 2, 64, 64, 1024, "fp16", snew=sq, seqlens=[0, 700, 333],
                            rotary_dim=64, interleaved=False, causal=True, seed=53 + sq)
    _kv_check(case)


@pytest.mark.parametrize("window", [(30, 0), (10, 10), (-1, 2)])
def test_kvcache_chunk_window(window):
    case = W.random_kvcache(2, 90, 4, 2, 128, 128, 512, "bf16", snew=90, seqlens=[0, 250],
                            rotary_dim=64, interleaved=True, causal=True, seed=31)
    _kv_check(case, window=window)


def test_window_wide_equals_no_window():
    # a window wider than the sequence is full attention; the two calls may
    # use different tile shapes (so a different summation order), hence the
    # fp16 bar rather than bit equality
    case = W.random_fwd(1, 200, 200, 2, 2, 64, 64, "fp16", True, seed=33)
    q, k, v = dev(case.q), dev(case.k), dev(case.v)
    a = E().attn_fwd(q, k, v, causal=True)
    b = E().attn_fwd(q, k, v, causal=True, window_size=(400, 400))
    torch.cuda.synchronize()
    ref, _ = attention_ref(to_f64(case.q), to_f64(case.k), to_f64(case.v), causal=True)
    assert maxabs(a, ref) <= TOL["fp16"] and maxabs(b, ref) <= TOL["fp16"]
    assert float((a.float() - b.float()).abs().max()) <= TOL["fp16"]


# ---------------------------------------------------------------- packed sequences

def _varlen_check(case, window=(-1, -1), max_seqlen_q=None):
    q, k, v = dev(case.q), dev(case.k), dev(case.v)
    cq, ck = dev(case.cu_seqlens_q), dev(case.cu_seqlens_k)
    tq, Hq, _ = q.shape
    buf, out = guarded_empty((tq, Hq, v.shape[2]), q.dtype)
    _, lse = E().attn_fwd_varlen(q, k, v, cq, ck, max_seqlen_q or case.max_seqlen_q, causal=case.causal,
                                 softmax_scale=case.softmax_scale, out=out, return_lse=True,
                                 window_size=window)
    torch.cuda.synchronize()
    assert canaries_intact(buf, out.numel())
    ref, rlse = attention_varlen_ref(to_f64(case.q), to_f64(case.k), to_f64(case.v),
                                     case.cu_seqlens_q.tolist(), case.cu_seqlens_k.tolist(),
                                     causal=case.causal, softmax_scale=case.softmax_scale, window=window)
    err = maxabs(out, ref)
    assert err <= TOL[case.dtype], "max abs err %.3e" % err
    l = lse.cpu().double().numpy()
    fin = np.isfinite(rlse)
    assert np.array_equal(fin, np.isfinite(l))
    assert np.max(np.abs(l[fin] - rlse[fin])) < LSE_TOL[case.dtype]
    return out


VARLEN_LENS = ([0, 1, 65, 200, 129, 7], [3, 1, 200, 65, 129, 0])


@pytest.mark.parametrize("dqk,dv,dtype", [(64, 64, "fp16"), (128, 128, "bf16"), (192, 128, "bf16"),
                                          (16, 16, "fp16")])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_ragged(dqk, dv, dtype, causal):
    # empty, one-row, multi-tile and ragged sequences; Sq != Sk per sequence; a sequence without keys
    case = W.random_varlen(*VARLEN_LENS, 4, 2, dqk, dv, dtype, causal, seed=dqk + causal)
    _varlen_check(case)


@pytest.mark.parametrize("window", [(0, 0), (37, 5), (-1, 16)])
def test_varlen_window(window):
    case = W.random_varlen(*VARLEN_LENS, 4, 2, 64, 64, "fp16", True, seed=41)
    _varlen_check(case, window=window)


def test_varlen_grid_larger_than_needed():
    # max_seqlen_q above the longest sequence: surplus query tiles do nothing
    case = W.random_varlen([100, 30], [100, 30], 2, 2, 64, 64, "fp16", True, seed=43)
    _varlen_check(case, max_seqlen_q=700)


@pytest.mark.parametrize("dqk,dv,dtype,causal", [(64, 64, "fp16", True), (128, 128, "bf16", True),
                                                 (64, 64, "fp16", False)])
def test_varlen_many_groups(dqk, dv, dtype, causal):
    # 12 sequences up to 611 rows: more than 64 (sequence, query tile) groups, so the
    # longest-first ranking runs through LDS instead of one wave's registers
    lens = [611, 3, 250, 0, 480, 77, 129, 600, 1, 333, 64, 500]
    case = W.random_varlen(lens, lens, 4, 2, dqk, dv, dtype, causal, seed=47 + dqk)
    _varlen_check(case)


def test_varlen_equal_lengths_bitwise_batched():
    # packed sequences of one length are the batched layout: same kernel, same bits
    B, S = 3, 300
    case = W.random_varlen([S] * B, [S] * B, 4, 2, 64, 64, "fp16", True, seed=45)
    out = _varlen_check(case)
    q, k, v = dev(case.q).view(B, S, 4, 64), dev(case.k).view(B, S, 2, 64), dev(case.v).view(B, S, 2, 64)
    ob = E().attn_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(ob.view(B * S, 4, 64), out)


# ---------------------------------------------------------------- gradients
# dq, dk, dv are sums over rows or keys, so their bar scales with their size:
# max-abs error <= TOL[dtype] * max(1, max |reference|)

def _bwd_check(case, window=(-1, -1), seed=0):
    q, k, v = dev(case.q), dev(case.k), dev(case.v)
    g = torch.Generator().manual_seed(seed + 1000)
    dout_c = torch.randn(q.shape[:3] + (v.shape[3],), generator=g).to(q.dtype)
    dout = dev(dout_c)
    out, lse = E().attn_fwd(q, k, v, causal=case.causal, softmax_scale=case.softmax_scale, return_lse=True,
                            window_size=window)
    dq, dk, dv = E().attn_bwd(dout, q, k, v, out, lse, causal=case.causal,
                              softmax_scale=case.softmax_scale, window_size=window)
    torch.cuda.synchronize()
    rq, rk, rv = attention_bwd_ref(to_f64(case.q), to_f64(case.k), to_f64(case.v), to_f64(dout_c),
                                   causal=case.causal, softmax_scale=case.softmax_scale, window=window)
    errs = []
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        err = maxabs(got, ref)
        bar = TOL[case.dtype] * max(1.0, float(np.max(np.abs(ref))))
        assert err <= bar, "%s max abs err %.3e > %.3e" % (name, err, bar)
        errs.append(err)
    return errs


@pytest.mark.parametrize("dqk,dv,dtype", [(64, 64, "fp16"), (128, 128, "bf16"), (192, 128, "bf16"),
                                          (64, 64, "bf16"), (128, 128, "fp16")])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_multi_tile_ragged(dqk, dv, dtype, causal):
    # 200 rows/keys: two 128-row tiles each way plus ragged tails; GQA 4:2
    case = W.random_fwd(2, 200, 200, 4, 2, dqk, dv, dtype, causal, seed=dqk + 5 * causal)
    _bwd_check(case, seed=dqk)


@pytest.mark.parametrize("causal", [False, True])
def test_workload_bwd_d64_full(causal):
    # every gradient element at the shape and launch configuration the benchmark times
    # (B=2, H=8, S=2048, D=64 fp16); the fp64 oracle takes a few seconds here
    _bwd_check(W.fwd_d64(causal), seed=11)


@pytest.mark.parametrize("sq,sk", [(100, 333), (333, 100), (1, 70), (70, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_sq_ne_sk(sq, sk, causal):
    case = W.random_fwd(1, sq, sk, 2, 1, 64, 64, "fp16", causal, seed=sq + sk)
    _bwd_check(case, seed=sq)


@pytest.mark.parametrize("window", [(0, 0), (37, 5), (-1, 20), (100, -1)])
def test_bwd_window(window):
    case = W.random_fwd(1, 300, 300, 4, 2, 128, 128, "bf16", True, seed=3 + window[0])
    _bwd_check(case, window=window, seed=7)


def test_bwd_gqa_group_of_eight():
    case = W.random_fwd(1, 150, 150, 8, 1, 64, 64, "fp16", True, seed=9)
    _bwd_check(case, seed=9)


def test_bwd_strided_views():
    # q, k, v, dO as transposed views of [B, H, S, D] memory; dq, dk, dv written
    # into transposed views as well (only their own elements)
    g = torch.Generator().manual_seed(71)
    B, S, Hq, Hkv, D = 2, 150, 4, 2, 128
    qm = torch.randn(B, Hq, S, D, generator=g).to(torch.bfloat16)
    km = torch.randn(B, Hkv, S, D, generator=g).to(torch.bfloat16)
    vm = torch.randn(B, Hkv, S, D, generator=g).to(torch.bfloat16)
    dom = torch.randn(B, Hq, S, D, generator=g).to(torch.bfloat16)
    q, k, v, do = (dev(t).transpose(1, 2) for t in (qm, km, vm, dom))
    assert not q.is_contiguous()
    out, lse = E().attn_fwd(q, k, v, causal=True, return_lse=True)
    dq = torch.full((B, Hq, S, D), 7.0, dtype=torch.bfloat16, device=DEV).transpose(1, 2)
    dk = torch.full((B, Hkv, S, D), 7.0, dtype=torch.bfloat16, device=DEV).transpose(1, 2)
    dv = torch.full((B, Hkv, S, D), 7.0, dtype=torch.bfloat16, device=DEV).transpose(1, 2)
    E().attn_bwd(do, q, k, v, out, lse, causal=True, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    rq, rk, rv = attention_bwd_ref(to_f64(qm.transpose(1, 2)), to_f64(km.transpose(1, 2)),
                                   to_f64(vm.transpose(1, 2)), to_f64(dom.transpose(1, 2)), causal=True)
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        err = maxabs(got, ref)
        bar = TOL["bf16"] * max(1.0, float(np.max(np.abs(ref))))
        assert err <= bar, "%s max abs err %.3e > %.3e" % (name, err, bar)


def test_bwd_no_keys_gives_zero_gradients():
    q = torch.randn(1, 5, 2, 64, device=DEV).half()
    k = torch.zeros(1, 0, 2, 64, device=DEV).half()
    out, lse = E().attn_fwd(q, k, k, return_lse=True)
    dq, dk, dv = E().attn_bwd(torch.randn_like(q), q, k, k, out, lse)
    torch.cuda.synchronize()
    assert (dq.float() == 0).all()


# ---------------------------------------------------------------- rope_apply

@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("interleaved", [False, True])
@pytest.mark.parametrize("D,rd", [(128, 32), (128, 40), (128, 128), (192, 96), (16, 16), (64, 48)])
def test_rope_apply_bit_exact(dtype, interleaved, D, rd):
    # rd % 16 == 0 takes the 16-byte-per-lane path (several rows per wave for
    # D < 512); rd = 40 takes the per-pair path
    tdt = W.DTYPES[dtype]
    g = torch.Generator().manual_seed(rd + interleaved + D)
    x = torch.randn(3, 50, 4, D, generator=g).to(tdt)
    cos, sin = W.rope_tables(512, rd, 10000.0, tdt)
    offs = torch.tensor([0, 17, 400], dtype=torch.int32)
    mod = E()
    for conj in (False, True):
        y = mod.rope_apply(dev(x), dev(cos), dev(sin), dev(offs), interleaved, conj)
        torch.cuda.synchronize()
        pos = offs.numpy()[:, None] + np.arange(50)[None, :]
        ref = rope_ref(to_f64(x), to_f64(cos), to_f64(sin), pos, rotary_dim=rd,
                       interleaved=interleaved, conjugate=conj, dtype=dtype)
        assert _bits_equal(y, ref, dtype)
    # in place, scalar offset
    xd = dev(x)
    mod.rope_apply(xd, dev(cos), dev(sin), 5, interleaved, inplace=True)
    torch.cuda.synchronize()
    ref = rope_ref(to_f64(x), to_f64(cos), to_f64(sin), 5 + np.tile(np.arange(50), (3, 1)),
                   rotary_dim=rd, interleaved=interleaved, dtype=dtype)
    assert _bits_equal(xd, ref, dtype)


# ---------------------------------------------------------------- FP8 inputs
# The skill page "Flash Attention - Fast Memory-Efficient Attention",
# Workflow 3: e4m3 q, k, v with per-tensor descales.  The output is bf16, so
# the bf16 bars apply (the weights P are rounded to bf16 for P V).

def _fp8_check(case, window=(-1, -1), sample_rows=None, views=False):
    q8, k8, v8 = dev(case.q), dev(case.k), dev(case.v)
    if views:   # [B, H, S, D] storage seen as [B, S, H, D] (strided views)
        q8, k8, v8 = (t.transpose(1, 2).contiguous().transpose(1, 2) for t in (q8, k8, v8))
    B, Sq, Hq, D = q8.shape
    buf, out = guarded_empty((B, Sq, Hq, D), torch.bfloat16)
    dq, dk, dvs = case.descale
    _, lse = E().attn_fwd_fp8(q8, k8, v8, causal=case.causal, softmax_scale=case.softmax_scale, out=out,
                              return_lse=True, window_size=window, descale_q=dq, descale_k=dk, descale_v=dvs)
    torch.cuda.synchronize()
    assert canaries_intact(buf, out.numel())
    qc, kc, vc = case.q.numpy(), case.k.numpy(), case.v.numpy()
    got, l = out, lse.cpu().double().numpy()
    if sample_rows is not None:
        rows = np.asarray(sample_rows)
        qc = qc[:, rows]
        got, l = out[:, torch.as_tensor(rows, device=DEV)], l[:, :, rows]
    kw = dict(descale_q=dq, descale_k=dk, descale_v=dvs, causal=case.causal, softmax_scale=case.softmax_scale,
              window=window)
    if sample_rows is None:
        ref, rlse = attention_fp8_ref(qc, kc, vc, **kw)
    else:   # the sampled rows keep their positions in the full sequence
        Sk = kc.shape[1]
        from oracle import e4m3_decode
        pos = np.tile(rows + Sk - Sq, (B, 1))
        ref, rlse = attention_ref(e4m3_decode(qc) * dq, e4m3_decode(kc) * dk, e4m3_decode(vc) * dvs,
                                  causal=case.causal, softmax_scale=case.softmax_scale, q_pos=pos, window=window)
    err = maxabs(got, ref)
    assert err <= TOL["bf16"], "max abs err %.3e" % err
    fin = np.isfinite(rlse)
    assert np.array_equal(fin, np.isfinite(l))
    if fin.any():
        assert np.max(np.abs(l[fin] - rlse[fin])) < LSE_TOL["bf16"]
    return err


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_multi_tile_ragged_gqa(d, causal):
    # 200 rows / 333 keys: several query and key tiles with ragged tails; GQA 4:2
    _fp8_check(W.random_fp8(2, 200, 333, 4, 2, d, causal, seed=d + causal))


@pytest.mark.parametrize("d", [64, 128])
def test_fp8_descales(d):
    _fp8_check(W.random_fp8(1, 130, 130, 2, 1, d, True, seed=5, descale=(0.5, 3.0, 1.5)))


@pytest.mark.parametrize("sq,sk", [(100, 300), (300, 77), (1, 129)])
def test_fp8_sq_ne_sk(sq, sk):
    _fp8_check(W.random_fp8(1, sq, sk, 4, 4, 64, True, seed=sq))


def test_fp8_window_and_scale():
    _fp8_check(W.random_fp8(1, 300, 300, 2, 2, 64, True, seed=9, softmax_scale=0.2), window=(64, 16))


def test_fp8_strided_views():
    _fp8_check(W.random_fp8(2, 96, 96, 4, 2, 128, False, seed=11), views=True)


def test_fp8_every_v_code_is_decoded_exactly():
    # one key with zero scores: every output row is v itself, so each of the 256
    # e4m3 codes placed in v must come out as its exact value (times descale_v,
    # a power of two here), NaN codes as NaN; the codes cover 4 heads x 64 dims
    from oracle import e4m3_decode
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(1, 1, 4, 64)
    zero = torch.zeros(1, 1, 4, 64, dtype=torch.uint8)
    for dv in (1.0, 0.5):
        out = E().attn_fwd_fp8(dev(zero), dev(zero), dev(codes), descale_v=dv)
        torch.cuda.synchronize()
        got = out.float().cpu().double().numpy()
        ref = e4m3_decode(codes.numpy()) * dv
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan)
        assert np.array_equal(got[~nan], ref[~nan])


def test_fp8_no_keys_gives_zero_rows():
    case = W.random_fp8(1, 5, 0, 2, 2, 64, False, seed=1)
    out, lse = E().attn_fwd_fp8(dev(case.q), dev(case.k), dev(case.v), return_lse=True)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


@pytest.mark.parametrize("causal", [False, True])
def test_workload_fwd_fp8_d64_full(causal):
    # the bench configuration: B=2, H=8, S=2048, D=64, every output row
    _fp8_check(W.fwd_fp8_d64(causal))


# ---------------------------------------------------------------- streams and graphs

def test_calls_follow_the_current_stream():
    # work is enqueued on torch's current stream: on a side stream the result
    # matches the default-stream call once that stream is synchronized
    case = W.random_fwd(2, 300, 300, 4, 2, 64, 64, "fp16", True, seed=61)
    q, k, v = dev(case.q), dev(case.k), dev(case.v)
    ref = E().attn_fwd(q, k, v, causal=True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        out = E().attn_fwd(q, k, v, causal=True)
    side.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_graph_capture_replays_match_eager():
    # the calls enqueue kernels only (no allocation inside the library, no
    # memset, no host synchronisation), so a HIP graph can hold them; every
    # replay, with eager work between replays, must give the eager bits
    mod = E()
    fc = W.random_fwd(2, 300, 300, 4, 2, 64, 64, "fp16", True, seed=63)
    q, k, v = dev(fc.q), dev(fc.k), dev(fc.v)
    kc = W.random_kvcache(3, 1, 8, 2, 128, 128, 512, "bf16", snew=1, seqlens=[0, 200, 511 - 1],
                          rotary_dim=128, seed=65)
    kq, kn, vn = dev(kc.q), dev(kc.k_new), dev(kc.v_new)
    kcache, vcache = dev(kc.k_cache), dev(kc.v_cache)
    cs, cos, sin = dev(kc.cache_seqlens), dev(kc.rotary_cos), dev(kc.rotary_sin)
    dout = torch.randn(q.shape, generator=torch.Generator().manual_seed(67)).to(q.dtype).to(DEV)

    fout = torch.empty_like(q)
    lse = torch.empty((2, 4, 300), dtype=torch.float32, device=DEV)
    kout = torch.empty((3, 1, 8, 128), dtype=kq.dtype, device=DEV)
    ws = torch.empty(1 << 22, dtype=torch.uint8, device=DEV)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

    def run():
        mod.attn_fwd(q, k, v, causal=True, out=fout, return_lse=False)
        o2, l2 = mod.attn_fwd(q, k, v, causal=True, return_lse=True)
        lse.copy_(l2)
        mod.attn_fwd_kvcache(kq, kcache, vcache, kn, vn, rotary_cos=cos, rotary_sin=sin, cache_seqlens=cs,
                             causal=True, rotary_interleaved=False, out=kout, workspace=ws)
        mod.attn_bwd(dout, q, k, v, fout, lse, causal=True, dq=dq, dk=dk, dv=dv)

    run()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (fout, lse, kout, kcache, vcache, dq, dk, dv)]

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()                                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (fout, lse, kout, dq, dk, dv):
            t.fill_(float("nan"))
        mod.attn_fwd(q, k, v, causal=False)     # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (fout, lse, kout, kcache, vcache, dq, dk, dv)
        for name, a, b in zip(("out", "lse", "kvcache out", "k_cache", "v_cache", "dq", "dk", "dv"), got, eager):
            assert torch.equal(a, b), "replay %d: %s differs from the eager call" % (rep, name)

