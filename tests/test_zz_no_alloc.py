"""attn_fwd_kvcache_noalloc: the kvcache entry point that allocates nothing.

It must give what attn_fwd_kvcache gives with a caller workspace -- the same
kernels run on the same plan, so outputs, lse and the appended cache rows are
compared bit for bit -- and both must match the fp64 oracle within the
bars (2e-3 fp16, 1.5e-2 bf16; caches bit-exact).  Each case makes two calls
in a row through the C ABI, the second with a smaller input, so the second
call reuses the device scratch the first one left behind.
"""
import ctypes

import numpy as np
import pytest
import torch

import workloads as W
from oracle import dtype_bits, kvcache_ref, to_f64

pytestmark = pytest.mark.gpu
TOL = {"fp16": 2e-3, "bf16": 1.5e-2}
DEV = "cuda"


def E():
    import exact_attention_qk_amd as mod
    return mod


def dev(t):
    return None if t is None else (t.to(DEV) if isinstance(t, torch.Tensor) else t)


def _call(case, noalloc):
    q, kn, vn = dev(case.q), dev(case.k_new), dev(case.v_new)
    kc, vc = dev(case.k_cache), dev(case.v_cache)
    cs = dev(case.cache_seqlens)
    B, Sq, Hq, _ = q.shape
    out = torch.full((B, Sq, Hq, vc.shape[3]), float("nan"), dtype=q.dtype, device=DEV)
    lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device=DEV)
    kw = dict(rotary_cos=dev(case.rotary_cos), rotary_sin=dev(case.rotary_sin), cache_seqlens=cs,
              causal=case.causal, softmax_scale=case.softmax_scale, rotary_interleaved=case.rotary_interleaved)
    if noalloc:
        E().attn_fwd_kvcache_noalloc(q, kc, vc, kn, vn, out=out, lse=lse, **kw)
    else:
        o, l = E().attn_fwd_kvcache(q, kc, vc, kn, vn, out=out, return_lse=True, **kw)
        lse.copy_(l)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu(), kc.cpu(), vc.cpu()


def _oracle_check(case, out, kc):
    B = case.q.shape[0]
    lens = W.seqlens_list(case.cache_seqlens, B)
    f = to_f64
    ref, _, rkc, _ = kvcache_ref(f(case.q), f(case.k_cache), f(case.v_cache), f(case.k_new), f(case.v_new),
                                 lens, dtype=case.dtype,
                                 rotary_cos=None if case.rotary_cos is None else f(case.rotary_cos),
                                 rotary_sin=None if case.rotary_sin is None else f(case.rotary_sin),
                                 rotary_interleaved=case.rotary_interleaved, causal=case.causal,
                                 softmax_scale=case.softmax_scale)
    err = float(np.max(np.abs(to_f64(out.float()) - ref)))
    assert err <= TOL[case.dtype], err
    assert np.array_equal(kc.view(torch.int16).numpy().view(np.uint16), dtype_bits(rkc, case.dtype))


def _pair(case):
    a = _call(case, noalloc=False)
    b = _call(case, noalloc=True)
    for name, x, y in zip(("out", "lse", "k_cache", "v_cache"), a, b):
        assert torch.equal(x.view(torch.int16) if x.dtype != torch.float32 else x.view(torch.int32),
                           y.view(torch.int16) if y.dtype != torch.float32 else y.view(torch.int32)), name
    _oracle_check(case, b[0], b[2])


def test_noalloc_decode_two_calls_second_smaller():
    # single-token decode (split partials in the scratch), then a smaller decode
    big = W.random_kvcache(4, 1, 16, 4, 128, 128, 2048, "bf16", snew=1, seqlens=[2000, 100, 1500, 7],
                           rotary_dim=128, seed=81)
    small = W.random_kvcache(2, 1, 8, 2, 64, 64, 512, "fp16", snew=1, seqlens=[300, 5], rotary_dim=64,
                             interleaved=True, seed=82)
    _pair(big)
    _pair(small)


def test_noalloc_rotated_copy_two_calls_second_smaller():
    # a rotary width that is not a multiple of 16: the rotated q copy lives in
    # the scratch too (chunk path, then a decode call with split partials)
    big = W.random_kvcache(2, 70, 4, 2, 128, 128, 400, "bf16", snew=70, seqlens=[0, 201], rotary_dim=40,
                           interleaved=True, seed=83)
    small = W.random_kvcache(2, 1, 4, 2, 128, 128, 256, "bf16", snew=1, seqlens=[100, 30], rotary_dim=40,
                             seed=84)
    _pair(big)
    _pair(small)


def test_noalloc_refuses_plans_beyond_the_scratch():
    # 16 query rows per kv head and 32 forced splits of 32 keys over 8 batches x
    # 8 kv heads need 16.8 MB of fp32 partials, above the 16 MiB scratch: refused
    # before anything is enqueued, the caches untouched
    case = W.random_kvcache(8, 1, 128, 8, 128, 128, 1024, "bf16", snew=1, seqlens=[10] * 8, seed=85)
    q, kn, vn = dev(case.q), dev(case.k_new), dev(case.v_new)
    kc, vc = dev(case.k_cache), dev(case.v_cache)
    out = torch.empty((8, 1, 128, 128), dtype=q.dtype, device=DEV)
    p = E().kvcache_params(q, kc, vc, kn, vn, None, None, dev(case.cache_seqlens), True, None, False, out,
                           None, None, 32)
    assert E().kvcache_workspace_size(p) > 16 << 20
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    code = E().lib().attn_fwd_kvcache_noalloc(ctypes.byref(p), stream)
    torch.cuda.synchronize()
    assert code == -5
    assert b"16777216" in E().lib().attn_last_error()
    assert torch.equal(kc.cpu(), case.k_cache)
