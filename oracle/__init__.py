"""fp64 CPU oracle for exact attention and its KV-cache decode variant.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call it.  It shares no code with the HIP library
(no kernels, headers, helpers, tables or constants); the only thing both sides
consume is the seeded input module ``workloads.py``, which holds no attention
arithmetic.

What it computes, and where each function's definition comes from:

* ``attention_ref`` -- the plain definition softmax(scale * Q K^T + mask) V,
  with the S x S score matrix materialised, one (batch, head) at a time, in
  fp64.  Source: the skill page "Flash Attention - Fast Memory-Efficient
  Attention", Workflow 1 Step 2 ("standard attention") and Step 4 (accuracy
  check against standard attention); the tiled online-softmax method reaches
  the same value up to rounding, so the oracle is that definition written out.
* ``rope_ref`` -- rotary position embedding by 2-D pair rotation, pairs
  (j, j + rd/2) (the rotate_half form of flash-attention issue #1402, second
  script) or (2j, 2j+1) when interleaved (flag named in ROCm/flash-attention
  PR #99), angle from a given cos/sin table row chosen by absolute position
  (PR #99, rotary kernel argument review), with a stated rounding contract.
* ``kvcache_ref`` -- append rotated new keys and raw new values into the cache
  at ``cache_seqlens`` and attend the rotated query over the cache prefix
  (issue #1402, both scripts; PR #99 test parametrisation).
* ``attention_bwd_ref`` -- the gradients dQ, dK, dV (flash-attention PR #1604).
* ``e4m3_decode``, ``attention_fp8_ref`` -- FP8 e4m3 inputs with per-tensor
  descale factors (the skill page, Workflow 3).

Pins (tests/test_oracle_pins.py) tie every function to closed forms, library
routines, invariants the pages state, and brute force on tiny shapes.
"""
from .numerics import round_to_dtype, dtype_bits, bits_to_f64, to_f64, f32_to_bf16_rne_bits
from .attention import attention_ref, attention_varlen_ref
from .rope import rope_ref
from .backward import attention_bwd_ref
from .kvcache import kvcache_ref
from .fp8 import e4m3_decode, attention_fp8_ref

__all__ = [
    "attention_ref", "attention_varlen_ref", "attention_bwd_ref", "e4m3_decode", "attention_fp8_ref", "rope_ref", "kvcache_ref", "round_to_dtype", "dtype_bits",
    "bits_to_f64", "to_f64", "f32_to_bf16_rne_bits",
]
