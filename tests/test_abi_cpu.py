"""Host-side tests of the C ABI (no GPU needed).

The library must load, export every function include/attn.h declares, share
torch's HIP runtime, and reject every malformed argument on the host before
anything is enqueued.  attn_validate_* make no HIP call, so CPU tensors'
addresses stand in for device pointers here (they are never dereferenced).
"""
import ctypes
import math
import os
import re

import pytest
import torch

import exact_attention_qk_amd as E
from exact_attention_qk_amd import AttnError

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                       src, flags=re.M)
    return sorted(set(names))


def test_header_functions_are_all_exported():
    names = _declared_functions()
    assert set(names) == set(E.EXPORTED), names
    lib = ctypes.CDLL(E.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert E.lib().attn_abi_version() == 3


def test_single_hip_runtime_in_process():
    maps = open("/proc/self/maps").read().splitlines()
    libs = {l.split()[-1] for l in maps if "libamdhip64" in l}
    assert len(libs) == 1, libs


def _t(shape, dtype=torch.float16):
    return torch.zeros(shape, dtype=dtype)


def _fwd(B=2, Sq=8, Sk=8, Hq=4, Hkv=2, Dqk=64, Dv=64, dtype=torch.float16, **kw):
    q, k, v = _t((B, Sq, Hq, Dqk), dtype), _t((B, Sk, Hkv, Dqk), dtype), _t((B, Sk, Hkv, Dv), dtype)
    out = _t((B, Sq, Hq, Dv), dtype)
    return E.fwd_params(q, k, v, out, **kw), (q, k, v, out)


def _code_fwd(p):
    return E.lib().attn_validate_fwd(ctypes.byref(p))


def test_validate_fwd_ok_and_errors():
    p, keep = _fwd()
    assert _code_fwd(p) == 0
    p, keep = _fwd(Hq=3, Hkv=2)
    assert _code_fwd(p) == -2
    assert b"multiple" in E.lib().attn_last_error()
    p, keep = _fwd(Dqk=96, Dv=96)
    assert _code_fwd(p) == -3
    p, keep = _fwd(Dqk=128, Dv=64)
    assert _code_fwd(p) == -3
    p, keep = _fwd()
    p.q.data = None
    assert _code_fwd(p) == -1
    p, keep = _fwd()
    p.k.data = p.k.data + 2
    assert _code_fwd(p) == -4
    p, keep = _fwd()
    p.v.stride_s = 100
    assert _code_fwd(p) == -4
    # key tiles use 32-bit byte offsets: the sequence stride stays below 2^24 elements
    p, keep = _fwd()
    p.k.stride_s = 1 << 24
    assert _code_fwd(p) == -3
    assert b"2^24" in E.lib().attn_last_error()
    p.k.stride_s = (1 << 24) - 8
    assert _code_fwd(p) == 0
    p, keep = _fwd()
    p.dtype = 7
    assert _code_fwd(p) == -3
    p, keep = _fwd()
    p.window_left = -2
    assert _code_fwd(p) == -2
    p, keep = _fwd()
    p.window_left, p.window_right = 0, 0
    assert _code_fwd(p) == 0
    # empty problems are valid no-ops
    p, keep = _fwd(Sq=0)
    assert _code_fwd(p) == 0
    p, keep = _fwd(Sk=0)
    p.k.data = None
    p.v.data = None
    assert _code_fwd(p) == 0


def test_validate_varlen():
    q = _t((10, 4, 64))
    k = _t((12, 2, 64))
    cu = torch.zeros(3, dtype=torch.int32)
    p = E.varlen_params(q, k, k, q, cu, cu, 8)
    assert E.lib().attn_validate_varlen(ctypes.byref(p)) == 0
    p.cu_seqlens_k = None
    assert E.lib().attn_validate_varlen(ctypes.byref(p)) == -1
    p = E.varlen_params(q, k, k, q, cu, cu, 8, window_size=(3, -4))
    assert E.lib().attn_validate_varlen(ctypes.byref(p)) == -2
    p = E.varlen_params(q, k, k, q, cu, cu, 8)
    p.Dqk = p.Dv = 96
    assert E.lib().attn_validate_varlen(ctypes.byref(p)) == -3


def test_validate_bwd():
    q = _t((2, 8, 4, 64))
    k = _t((2, 8, 2, 64))
    lse = torch.zeros(2, 4, 8)
    p = E.bwd_params(q, k, k, q, q, lse, q, k, k)
    assert E.lib().attn_validate_bwd(ctypes.byref(p)) == -5          # workspace missing
    need = E.lib().attn_bwd_workspace_size(ctypes.byref(p))
    assert need == ((2 * 4 * 8 * 8 + 255) // 256) * 256
    ws = torch.zeros(need + 512, dtype=torch.uint8)
    p.workspace, p.workspace_bytes = ws.data_ptr() + (-ws.data_ptr()) % 256, need
    assert E.lib().attn_validate_bwd(ctypes.byref(p)) == 0
    p.Dqk = p.Dv = 16
    assert E.lib().attn_validate_bwd(ctypes.byref(p)) == -3         # no backward at head size 16
    p = E.bwd_params(q, k, k, q, q, lse, q, k, k)
    p.workspace, p.workspace_bytes = ws.data_ptr() + (-ws.data_ptr()) % 256, need
    p.lse = None
    assert E.lib().attn_validate_bwd(ctypes.byref(p)) == -1


def test_validate_fp8():
    q8 = torch.zeros(2, 8, 4, 64, dtype=torch.uint8)
    k8 = torch.zeros(2, 8, 2, 64, dtype=torch.uint8)
    out = _t((2, 8, 4, 64), torch.bfloat16)
    p = E.fp8_params(q8, k8, k8, out)
    assert E.lib().attn_fwd_fp8_workspace_size(ctypes.byref(p)) == 0   # v is converted inside the kernel
    assert E.lib().attn_validate_fp8(ctypes.byref(p)) == 0           # no workspace needed
    p.D = 192
    assert E.lib().attn_validate_fp8(ctypes.byref(p)) == -3          # head sizes 64 and 128 only
    p.D = 64
    p.descale_v = float("inf")
    assert E.lib().attn_validate_fp8(ctypes.byref(p)) == -2
    p.descale_v = 1.0
    p.k.stride_s = 8                                                 # 1-byte rows: strides x16
    assert E.lib().attn_validate_fp8(ctypes.byref(p)) == -4
    with pytest.raises(AttnError):
        E.fp8_params(_t((2, 8, 4, 64)), k8, k8, out)                 # not e4m3 codes


def test_binding_rejects_other_dtypes_before_any_launch():
    q = torch.zeros(1, 4, 1, 64)
    with pytest.raises(AttnError):
        E.attn_fwd(q, q, q)


def test_binding_refuses_host_tensors_before_any_launch():
    # a host pointer handed to a kernel would be a GPU memory fault: the binding refuses it
    q = torch.zeros(1, 4, 1, 64, dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU"):
        E.attn_fwd(q, q, q)
    kc = torch.zeros(1, 8, 1, 64, dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU"):
        E.attn_fwd_kvcache(q[:, :1], kc, kc, cache_seqlens=0)
    cs = torch.zeros(8, 32, dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU"):
        E.rope_apply(q, cs, cs)
    with pytest.raises(ValueError, match="cu_seqlens"):
        E.attn_fwd_varlen(q[0], q[0], q[0], torch.zeros(2, dtype=torch.int64), torch.zeros(2, dtype=torch.int32), 4)


def _kv(B=2, Sq=1, Hq=8, Hkv=2, D=128, cap=64, snew=1, seqlens=5, rotary=0, dtype=torch.bfloat16,
        **kw):
    q = _t((B, Sq, Hq, D), dtype)
    kc, vc = _t((B, cap, Hkv, D), dtype), _t((B, cap, Hkv, D), dtype)
    kn = _t((B, snew, Hkv, D), dtype) if snew else None
    vn = _t((B, snew, Hkv, D), dtype) if snew else None
    cos = sin = None
    if rotary:
        cos, sin = _t((cap, rotary // 2), dtype), _t((cap, rotary // 2), dtype)
    out = _t((B, Sq, Hq, D), dtype)
    p = E.kvcache_params(q, kc, vc, kn, vn, cos, sin, seqlens, True, None, False, out, None, None,
                         kw.get("num_splits", 0))
    return p, (q, kc, vc, kn, vn, cos, sin, out)


def _code_kv(p):
    return E.lib().attn_validate_kvcache(ctypes.byref(p))


def test_validate_kvcache_workspace_and_overflow():
    p, keep = _kv()
    need = E.kvcache_workspace_size(p)
    assert need > 0                                     # decode path needs split partials
    assert _code_kv(p) == -5                            # no workspace given
    ws = torch.zeros(need + 512, dtype=torch.uint8)
    base = ws.data_ptr() + (-ws.data_ptr()) % 256
    p.workspace, p.workspace_bytes = base, need
    assert _code_kv(p) == 0
    p.workspace_bytes = need - 1
    assert _code_kv(p) == -5
    p.workspace, p.workspace_bytes = base + 16, need
    assert _code_kv(p) == -4
    p2, keep2 = _kv(seqlens=64)                          # 64 + 1 > capacity 64
    assert _code_kv(p2) == -6
    p3, keep3 = _kv(seqlens=-1)
    assert _code_kv(p3) == -2
    p4, keep4 = _kv(snew=0)
    p4.Snew = 1                                         # k_new NULL with Snew = 1
    p4.workspace, p4.workspace_bytes = base, need
    assert _code_kv(p4) == -1


def test_validate_kvcache_rotary_args():
    p, keep = _kv(rotary=64)
    assert p.rotary_dim == 64 and p.seqlen_ro == 64
    need = E.kvcache_workspace_size(p)
    ws = torch.zeros(need + 512, dtype=torch.uint8)
    p.workspace = ws.data_ptr() + (-ws.data_ptr()) % 256
    p.workspace_bytes = need
    assert _code_kv(p) == 0
    p.rotary_dim = 63
    assert _code_kv(p) == -2
    p.rotary_dim = 256
    assert _code_kv(p) == -2
    p.rotary_dim = 64
    p.rotary_sin = None
    assert _code_kv(p) == -1
    p, keep = _kv(rotary=64, seqlens=63)                 # position 63 + 1 token > 64 rows
    p.seqlen_ro = 63
    assert _code_kv(p) == -2


def _al(x):
    return (x + 255) // 256 * 256


def test_kvcache_workspace_plan():
    # decode path: partials for every (split, kv head, row), splits numbered
    # across batches; the rotation happens inside the decode kernel
    # (rd % 16 == 0).  The kernels size the splits from the device-side
    # lengths for at most 1408 (kv head, split) waves plus one split per
    # batch: 1408 // 8 + 8 + 1 = 185 splits (a 8192-row cache alone would
    # allow 8 * 256 splits of 32 keys)
    p, keep = _kv(B=8, Hq=32, Hkv=8, D=128, cap=8192, rotary=128)
    need = E.kvcache_workspace_size(p)
    nsp = 1408 // 8 + 8 + 1
    R = 4
    cnt = 0
    assert need == cnt + _al(nsp * 8 * R * 128 * 4) + _al(nsp * 8 * R * 2 * 4)
    # a short capacity bounds the splits instead: 8 batches x 2 splits of 32
    p2, keep2 = _kv(B=8, Hq=32, Hkv=8, D=128, cap=64, rotary=128)
    assert E.kvcache_workspace_size(p2) == _al(16 * 8 * R * 128 * 4) + _al(16 * 8 * R * 2 * 4)
    # forcing one split
    p.num_splits = 1
    assert E.kvcache_workspace_size(p) == cnt + _al(8 * 8 * 1 * R * 128 * 4) + _al(8 * 8 * R * 2 * 4)
    # a rotary width that is not a multiple of 16 takes the separate rotation
    # pass, whose rotated q copy comes first
    p, keep = _kv(B=8, Hq=32, Hkv=8, D=128, cap=8192, rotary=40)
    q_rot = 8 * 1 * 32 * 128 * 2
    assert E.kvcache_workspace_size(p) == cnt + _al(q_rot) + _al(nsp * 8 * R * 128 * 4) + \
        _al(nsp * 8 * R * 2 * 4)
    # chunked prefill (many query rows): q is rotated as the tiled kernel loads
    # it when the rotary width is a multiple of 16; otherwise a rotated copy
    p, keep = _kv(B=4, Sq=512, Hq=16, Hkv=16, D=128, cap=4096, snew=512, rotary=64)
    assert E.kvcache_workspace_size(p) == 0
    p, keep = _kv(B=4, Sq=512, Hq=16, Hkv=16, D=128, cap=4096, snew=512, rotary=40)
    assert E.kvcache_workspace_size(p) == 4 * 512 * 16 * 128 * 2
    p, keep = _kv(B=4, Sq=512, Hq=16, Hkv=16, D=128, cap=4096, snew=512)
    assert E.kvcache_workspace_size(p) == 0


def test_validate_rope():
    x = _t((2, 5, 3, 64))
    cos, sin = _t((16, 16)), _t((16, 16))
    p = E.rope_params(x, cos, sin, 3, False, False, x)
    assert E.lib().attn_validate_rope(ctypes.byref(p)) == 0
    p = E.rope_params(x, cos, sin, 12, False, False, x)      # 12 + 5 > 16 rows
    assert E.lib().attn_validate_rope(ctypes.byref(p)) == -2
    p = E.rope_params(x, cos, sin, 0, False, False, x)
    p.rotary_dim = 65
    assert E.lib().attn_validate_rope(ctypes.byref(p)) == -2
    p = E.rope_params(x, cos, sin, 0, False, False, x)
    p.cos = None
    assert E.lib().attn_validate_rope(ctypes.byref(p)) == -1


def test_kvcache_binding_requires_explicit_interleave_flag():
    q = torch.zeros(1, 1, 2, 64, dtype=torch.float16)
    cos = torch.zeros(4, 32, dtype=torch.float16)
    with pytest.raises(ValueError):
        E.attn_fwd_kvcache(q, q, q, rotary_cos=cos, rotary_sin=cos)


# ---------------------------------------------------------------- binding shape checks
# A tensor whose shape disagrees with the others would make a kernel read or
# write outside it (a GPU fault, not an error code): the binding refuses it
# while building the parameter block, before any pointer reaches the library.

def test_fwd_params_refuse_mismatched_tensors():
    q, k, v, out = _t((2, 8, 4, 64)), _t((2, 8, 2, 64)), _t((2, 8, 2, 64)), _t((2, 8, 4, 64))
    E.fwd_params(q, k, v, out)
    for bad_k in (_t((1, 8, 2, 64)), _t((2, 8, 2, 32)), _t((2, 8, 2, 64), torch.bfloat16)):
        with pytest.raises(ValueError):
            E.fwd_params(q, bad_k, v, out)
    with pytest.raises(ValueError):
        E.fwd_params(q, k, _t((2, 9, 2, 64)), out)           # v length differs from k
    with pytest.raises(ValueError):
        E.fwd_params(q, k, _t((2, 8, 1, 64)), out)           # v heads differ from k
    with pytest.raises(ValueError):
        E.fwd_params(q, k, v, _t((2, 8, 4, 32)))             # out head_dim != Dv
    with pytest.raises(ValueError):
        E.fwd_params(q, k, v, out, lse=torch.zeros(2, 4, 7))  # lse shape
    with pytest.raises(ValueError):
        E.fwd_params(q, k, v, out, lse=torch.zeros(2, 4, 8, dtype=torch.float16))
    with pytest.raises(ValueError):
        E.fwd_params(q[0], k, v, out)                        # not 4-d


def test_bwd_params_refuse_mismatched_tensors():
    q, k = _t((2, 8, 4, 64)), _t((2, 8, 2, 64))
    lse = torch.zeros(2, 4, 8)
    E.bwd_params(q, k, k, q, q, lse, q, k, k)
    with pytest.raises(ValueError):
        E.bwd_params(q, k, k, q, _t((2, 7, 4, 64)), lse, q, k, k)     # dout
    with pytest.raises(ValueError):
        E.bwd_params(q, k, k, q, q, lse, _t((2, 8, 4, 32)), k, k)     # dq
    with pytest.raises(ValueError):
        E.bwd_params(q, k, k, q, q, lse, q, _t((2, 8, 4, 64)), k)     # dk heads
    with pytest.raises(ValueError):
        E.bwd_params(q, k, k, q, q, lse, q, k, _t((2, 9, 2, 64)))     # dv length
    with pytest.raises(ValueError):
        E.bwd_params(q, k, k, q, q, torch.zeros(2, 4, 9), q, k, k)    # lse


def test_fp8_params_refuse_mismatched_tensors():
    q8 = torch.zeros(2, 8, 4, 64, dtype=torch.uint8)
    k8 = torch.zeros(2, 8, 2, 64, dtype=torch.uint8)
    out = _t((2, 8, 4, 64), torch.bfloat16)
    E.fp8_params(q8, k8, k8, out)
    with pytest.raises(ValueError):
        E.fp8_params(q8, k8, torch.zeros(2, 6, 2, 64, dtype=torch.uint8), out)
    with pytest.raises(ValueError):
        E.fp8_params(q8, k8, k8, _t((2, 8, 4, 64)))          # output must be bf16
    with pytest.raises(ValueError):
        E.fp8_params(q8, k8, k8, _t((2, 8, 2, 64), torch.bfloat16))


def test_varlen_params_refuse_mismatched_tensors():
    q, k, out = _t((10, 4, 64)), _t((12, 2, 64)), _t((10, 4, 64))
    cu = torch.zeros(3, dtype=torch.int32)
    E.varlen_params(q, k, k, out, cu, cu, 8)
    with pytest.raises(ValueError):
        E.varlen_params(q, k, _t((11, 2, 64)), out, cu, cu, 8)
    with pytest.raises(ValueError):
        E.varlen_params(q, k, k, _t((10, 4, 32)), cu, cu, 8)
    with pytest.raises(ValueError):
        E.varlen_params(q, k, k, out, cu, torch.zeros(4, dtype=torch.int32), 8)
    with pytest.raises(ValueError):
        E.varlen_params(q, k, k, out, cu, cu, 8, lse=torch.zeros(4, 9))


def test_kvcache_params_refuse_mismatched_tensors():
    B, cap, D = 2, 64, 128
    q = _t((B, 1, 8, D), torch.bfloat16)
    kc = _t((B, cap, 2, D), torch.bfloat16)
    kn = _t((B, 1, 2, D), torch.bfloat16)
    out = _t((B, 1, 8, D), torch.bfloat16)
    cs = torch.zeros(B, dtype=torch.int32)
    cos = _t((cap, 64), torch.bfloat16)
    E.kvcache_params(q, kc, kc, kn, kn, cos, cos, cs, True, None, False, out)
    bad = [
        dict(v_cache=_t((B, cap - 1, 2, D), torch.bfloat16)),     # capacities differ
        dict(v_cache=_t((B, cap, 1, D), torch.bfloat16)),         # kv heads differ
        dict(k=_t((B, 2, 2, D), torch.bfloat16)),                 # k_new / v_new lengths differ
        dict(v=_t((B, 1, 2, 64), torch.bfloat16)),                # v_new head_dim != Dv
        dict(out=_t((B, 1, 8, 64), torch.bfloat16)),
        dict(k_cache=_t((B, cap, 2, D), torch.float16)),          # dtype differs from q
        dict(cache_seqlens=torch.zeros(B - 1, dtype=torch.int32)),
        dict(cache_seqlens=torch.zeros(B, dtype=torch.int64)),
        dict(rotary_cos=_t((cap, 64)), rotary_sin=_t((cap, 64))),  # fp32 tables
        dict(rotary_cos=_t((cap, 128), torch.bfloat16)[:, :64],    # sliced (strided) table rows
             rotary_sin=_t((cap, 128), torch.bfloat16)[:, :64]),
        dict(rotary_sin=_t((cap, 32), torch.bfloat16)),           # cos and sin differ
        dict(rotary_cos=_t((cap, 72), torch.bfloat16), rotary_sin=_t((cap, 72), torch.bfloat16)),  # 144 > D
        dict(v=None),                                             # k without v
    ]
    for kw in bad:
        args = dict(q=q, k_cache=kc, v_cache=kc, k=kn, v=kn, rotary_cos=cos, rotary_sin=cos,
                    cache_seqlens=cs, causal=True, softmax_scale=None, rotary_interleaved=False, out=out)
        args.update(kw)
        with pytest.raises(ValueError):
            E.kvcache_params(**args)


def test_rope_params_refuse_mismatched_tensors():
    x = _t((2, 5, 3, 64))
    cos = _t((16, 16))
    E.rope_params(x, cos, cos, 0, False, False, x)
    with pytest.raises(ValueError):
        E.rope_params(x, cos, cos, 0, False, False, _t((2, 5, 3, 32)))
    with pytest.raises(ValueError):
        E.rope_params(x, _t((16, 16), torch.bfloat16), _t((16, 16), torch.bfloat16), 0, False, False, x)
    with pytest.raises(ValueError):
        E.rope_params(x, cos, _t((16, 8)), 0, False, False, x)
    with pytest.raises(ValueError):
        E.rope_params(x, cos, cos, torch.zeros(1, dtype=torch.int32), False, False, x)


def test_abi_refuses_zero_sequence_stride():
    # an expanded view (stride 0 along the sequence) would make the tiled
    # kernel's K/V buffer resources empty: the library refuses it
    p, keep = _fwd()
    p.k.stride_s = 0
    assert _code_fwd(p) == -3
    assert b"stride 0" in E.lib().attn_last_error()
    p, keep = _fwd(Sk=1)
    p.k.stride_s = p.v.stride_s = 0                  # one row: no stride is ever applied
    assert _code_fwd(p) == 0
    p, keep = _kv()
    p.k_cache.stride_s = 0
    assert _code_kv(p) == -3
    x = _t((2, 5, 3, 64))
    cos = _t((16, 16))
    pr = E.rope_params(x, cos, cos, 0, False, False, x)
    pr.x.stride_s = 0
    assert E.lib().attn_validate_rope(ctypes.byref(pr)) == -3
