// Host-side entry points of the kernel translation units.
#pragma once
#include <hip/hip_runtime.h>
#include "attn_args.hpp"

namespace attn {
hipError_t run_tile_attn(const AttnArgs& a, int dtype_bf16, int dqk, int dv, bool causal,
                         hipStream_t st);
// q, k, v: e4m3 codes (byte strides); output bf16.  d in {64, 128}.
hipError_t run_tile_attn_fp8(const AttnArgs& a, int d, bool causal, hipStream_t st);
hipError_t run_decode_attn(const AttnArgs& a, int dtype_bf16, int dqk, int dv, bool causal,
                           hipStream_t st);
hipError_t run_rope_rows(const RowSet* sets, int nsets, int dtype_bf16, hipStream_t st);
hipError_t run_attn_bwd(const BwdArgs& a, int dtype_bf16, int dqk, int dv, hipStream_t st);
hipError_t run_zero_rows(void* data, int64_t sb, int64_t ss, int64_t sh, int B, int S, int H, int D,
                         hipStream_t st);
}  // namespace attn
