// Split-KV attention for few query rows per kv head (single-token decode and
// short appends), and the log-sum-exp merge of the splits.
//
// Method: the decode-time variant of exact attention (flash-attention issue
// #1402, flash_attn_with_kvcache): queries attend the cache prefix of their
// batch.  With one new token per step there are only (Hq/Hkv) * Sq query rows
// per kv head, so the key range of each (batch, kv head) is cut into splits
// that run in parallel; each split keeps its own running max, sum and
// unnormalised output, and a second kernel combines them exactly:
//   M = max_s m_s,  l = sum_s l_s 2^(m_s - M),  O = sum_s O_s 2^(m_s - M) / l.
// A (batch, kv head) whose keys fit in one split writes its output directly.
//
// Fused append (when the rotary width is 0 or a multiple of 16): queries are
// rotated as they are loaded; the split whose key range holds the new
// positions [c_b, c_b + Snew) writes the rotated new keys (same rounding as
// rope_apply) and the new values into the cache before it streams its keys,
// and is the only workgroup that reads those rows.
//
// One wave per (kv head, split, batch).  The R <= 16 query rows of a kv head
// are the 16 columns of v_mfma_f32_16x16x32 (unused columns are zero):
//  * S^T = K Q^T with K read straight from HBM into the A operand (16 keys x
//    32 dims per MFMA, 16 contiguous bytes per lane);
//  * the V rows of a 32-key step go global -> LDS (row-major, swizzled) by
//    DMA and come back as the transposed A operand of O^T += V^T P^T through
//    ds_read_b64_tr_b16;
//  * two steps' loads are in flight while a step computes.
// The grid is sized from the cache capacity, so the host never reads the
// device-side cache lengths; workgroups past the total work exit at once.
#include "device_common.hpp"
#include "attn_args.hpp"
#include "launchers.hpp"

namespace attn {

// vmcnt(n) with the other counters left alone (gfx9 encoding: vmcnt in bits 3:0 and 15:14)
#define VMCNT_WAIT(n) __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14)) | 0x0F70)

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m);
  return x;
}

// Keys of a batch that any of its query rows can see: [kbeg, kend), with
// the query at position p seeing p - wl <= j <= p + wr (wr capped at 0 when
// causal).  Splits tile [kbeg, kend).
struct SeqInfo {
  int L, off, kbeg, kend, wl, wr;   // key length, position of query token 0, key range, window
};
__device__ __forceinline__ SeqInfo seq_info(const AttnArgs& a, int b, bool causal) {
  SeqInfo s;
  if (a.kvcache) {
    const int cb = a.seqlens ? a.seqlens[b] : a.seqlen_scalar;
    s.L = cb + a.Snew;
    s.off = cb;
  } else {
    s.L = a.Sk;
    s.off = a.Sk - a.Sq;
  }
  s.wl = a.wl;
  s.wr = causal ? min(a.wr, 0) : a.wr;
  s.kend = max(0, min(s.L, s.off + a.Sq + s.wr));
  s.kbeg = min(s.kend, max(0, s.off - s.wl));
  return s;
}
__device__ __forceinline__ int split_count(const AttnArgs& a, const SeqInfo& s) {
  return min(a.num_splits, (s.kend - s.kbeg + a.split_len - 1) / a.split_len);
}

// Combine the nvalid splits of query row r of (b, hkv) (one wave).  A lane
// owns output columns lane and lane + 64.  The partial outputs of the first
// 32 splits are requested together with the splits' maxima, so the common
// case needs one round trip to memory; split weights are broadcast with
// cross-lane reads.
template <class T>
__device__ void merge_row(const AttnArgs& a, int b, int hkv, int r, int R, int nvalid, int DV) {
  constexpr int C = 32;
  const int lane = threadIdx.x;
  const int dv0 = min(lane, DV - 1), dv1 = min(lane + 64, DV - 1);   // clamped: loads never branch
  const int tok = r / a.group;
  const int hq = hkv * a.group + (r - tok * a.group);
  const int64_t slot0 = ((int64_t)b * a.Hkv + hkv) * a.num_splits * R + r;
  auto orow_of = [&](int sp) { return a.ws_o + (slot0 + (int64_t)sp * R) * DV; };
  float v0[C], v1[C];
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const float* os = orow_of(min(j, nvalid - 1));
    v0[j] = os[dv0];
    v1[j] = os[dv1];
  }
  float M = -__builtin_inff();
  for (int sp = lane; sp < nvalid; sp += 64) M = fmaxf(M, a.ws_ml[(slot0 + (int64_t)sp * R) * 2]);
  M = wave_max(M);
  const float Ms = (M == -__builtin_inff()) ? 0.f : M;
  float lpart = 0.f, acc0 = 0.f, acc1 = 0.f;
  for (int s0 = 0; s0 < nvalid; s0 += 64) {
    // weight of split s0 + lane
    const int sp = s0 + lane;
    float w = 0.f;
    if (sp < nvalid) {
      const float ms = a.ws_ml[(slot0 + (int64_t)sp * R) * 2];
      w = (ms == -__builtin_inff()) ? 0.f : fast_exp2(ms - Ms);
      lpart += w * a.ws_ml[(slot0 + (int64_t)sp * R) * 2 + 1];
    }
    const int n = min(64, nvalid - s0);
    for (int j0 = 0; j0 < n; j0 += C) {
      if (s0 + j0 > 0) {
#pragma unroll
        for (int j = 0; j < C; ++j) {
          const float* os = orow_of(s0 + min(j0 + j, n - 1));
          v0[j] = os[dv0];
          v1[j] = os[dv1];
        }
      }
#pragma unroll
      for (int j = 0; j < C; ++j) {
        const float wj = __shfl(w, j0 + j);
        if (j0 + j < n) {
          acc0 += wj * v0[j];
          acc1 += wj * v1[j];
        }
      }
    }
  }
  const float lsum = wave_sum(lpart);
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  uint16_t* orow = a.out + (int64_t)b * a.o_sb + (int64_t)tok * a.o_ss + (int64_t)hq * a.o_sh;
  if (lane < DV) orow[lane] = T::from_f32(acc0 * inv);
  if (lane + 64 < DV) orow[lane + 64] = T::from_f32(acc1 * inv);
  if (a.lse && lane == 0)
    a.lse[((int64_t)b * a.Hq + hq) * a.Sq + tok] =
        lsum > 0.f ? (M + __log2f(lsum)) * 0.69314718055994531f : -__builtin_inff();
}

// One wave per (batch, kv head, query row).  A (batch, kv head) whose keys
// fit in one split (or that has no key) was finished by the attention kernel.
template <class T>
__global__ __launch_bounds__(64) void split_merge_kernel(AttnArgs a, int DV) {
  const int R = a.group * a.Sq;
  int idx = blockIdx.x;
  const int r = idx % R;
  idx /= R;
  const int hkv = idx % a.Hkv;
  const int b = idx / a.Hkv;
  const SeqInfo si = seq_info(a, b, a.causal != 0);
  const int nvalid = split_count(a, si);
  if (nvalid <= 1) return;
  merge_row<T>(a, b, hkv, r, R, nvalid, DV);
}

template <class T, int DQK, int DV, bool CAUSAL, bool FUSED>
__global__ __launch_bounds__(64, (DQK > 128 ? 1 : 2)) void decode_attn_kernel(AttnArgs a) {
  constexpr int QS = (DQK + 31) / 32;          // 32-dim k-steps of S
  constexpr int CK = DQK / 8;                  // chunks per K row
  constexpr int CV = DV / 8;                   // chunks per V row
  constexpr int VPL = (32 * CV) / 64;          // V DMA instructions per 32-key step
  constexpr int DVB = DV / 16;                 // 16-wide output blocks
  constexpr int NK = 2 * QS;                   // K loads per lane per step
  static_assert((32 * CV) % 64 == 0, "V step must be whole DMA instructions");
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[3 * 32 * DV];

  const int lane = threadIdx.x;
  // Workgroup i takes the i-th (batch, split, kv head) that has keys, in that
  // order, so the busy workgroups are the first ones dispatched and spread
  // evenly over the CUs whatever the cache lengths; kv heads vary fastest, so
  // the heads of one split (whose rows share cache lines and DRAM pages) are
  // fetched at about the same time.  Batches without keys get one workgroup
  // per kv head (split 0) that writes zeros.
  int item = blockIdx.x;
  int b = 0, nsp_b = 0;
  for (; b < a.B; ++b) {
    const SeqInfo sb = seq_info(a, b, CAUSAL);
    nsp_b = max(1, split_count(a, sb));
    if (item < nsp_b * a.Hkv) break;
    item -= nsp_b * a.Hkv;
  }
  if (b >= a.B) return;   // surplus workgroup
  const int split = item / a.Hkv, hkv = item - split * a.Hkv;
  const SeqInfo si = seq_info(a, b, CAUSAL);
  const int L = si.L, off = si.off, kend_all = si.kend, wlft = si.wl, wrgt = si.wr;
  const int R = a.group * a.Sq;
  const int r = lane & 15, kg = lane >> 4;
  const int tok = r / a.group;
  const int hq = hkv * a.group + (r - tok * a.group);
  const bool row_ok = r < R;
  const int qpos = off + tok;

  const int k_begin = si.kbeg + split * a.split_len;
  if (k_begin >= kend_all) {
    if (kend_all == si.kbeg && split == 0 && row_ok) {
      // no keys at all: the output rows are zero and the lse is -inf
      uint16_t* orow = a.out + (int64_t)b * a.o_sb + (int64_t)tok * a.o_ss + (int64_t)hq * a.o_sh;
#pragma unroll
      for (int i = 0; i < DVB; ++i) *reinterpret_cast<u32x2*>(orow + i * 16 + 4 * kg) = (u32x2){0u, 0u};
      if (a.lse && kg == 0) a.lse[((int64_t)b * a.Hq + hq) * a.Sq + tok] = -__builtin_inff();
    }
    return;
  }
  const int k_end = min(kend_all, k_begin + a.split_len);
  const int nvalid = split_count(a, si);

  u32x4 qf[QS];
  {
    const int tq = min(tok, a.Sq - 1);
    const uint16_t* qrow = a.q + (int64_t)b * a.q_sb + (int64_t)tq * a.q_ss + (int64_t)min(hq, a.Hq - 1) * a.q_sh;
#pragma unroll
    for (int st = 0; st < QS; ++st) {
      const int d = min(32 * st + 8 * kg, DQK - 8);
      if (FUSED)
        qf[st] = rope_chunk<T>(qrow, d, a.rcos, a.rsin, (int64_t)off + tq, a.rd, a.rinter, false);
      else
        qf[st] = ldg16(qrow + d);
      if (!row_ok || 32 * st + 8 * kg >= DQK) qf[st] = (u32x4){0, 0, 0, 0};
    }
  }

  const uint16_t* kbase = a.k + (int64_t)b * a.k_sb + (int64_t)hkv * a.k_sh;
  const uint16_t* vbase = a.v + (int64_t)b * a.v_sb + (int64_t)hkv * a.v_sh;
  const uint16_t* knbase = FUSED ? a.kn + (int64_t)b * a.kn_sb + (int64_t)hkv * a.kn_sh : nullptr;
  const uint16_t* vnbase = FUSED ? a.vn + (int64_t)b * a.vn_sb + (int64_t)hkv * a.vn_sh : nullptr;

  // One 32-key step: K straight into MFMA A operands (registers), V into an
  // LDS stage by DMA.  Rows past the split end are fetched from its last row
  // and masked, so every load is unconditional.
  struct KBuf {
    u32x4 k[2][QS];
  };
  auto load = [&](int kk, KBuf& B, int stage) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int key = min(kk + 16 * blk + r, k_end - 1);
#pragma unroll
      for (int st = 0; st < QS; ++st) {
        const int d = min(32 * st + 8 * kg, DQK - 8);
        B.k[blk][st] = ldg16(kbase + (int64_t)key * a.k_ss + d);
      }
    }
    uint16_t* vd = lds_v + stage * 32 * DV;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int P = j * 64 + lane;
      const int row = P / CV, pos = P % CV;
      const int ch = pos ^ swz_v<CV>(row);
      const int key = min(kk + row, k_end - 1);
      __builtin_amdgcn_global_load_lds((const void*)(vbase + (int64_t)key * a.v_ss + ch * 8),
                                       (LDS_AS void*)(vd + j * 512), 16, 0, 0);
    }
  };

  f32x4 o[DVB];
#pragma unroll
  for (int i = 0; i < DVB; ++i) o[i] = (f32x4){0, 0, 0, 0};
  float m_run = -__builtin_inff(), l_run = 0.f;
  const float c = a.c;
  const int tr_t = (lane & 15) >> 2, tr_q = lane & 3;

  auto step = [&](int kk, const KBuf& B, int stage, int later_steps) {
    // this step's V DMA has landed once at most the later steps' loads are pending
    if (later_steps >= 2) VMCNT_WAIT(2 * (NK + VPL));
    else if (later_steps == 1) VMCNT_WAIT(NK + VPL);
    else VMCNT_WAIT(0);
    const uint16_t* vt = lds_v + stage * 32 * DV;
    f32x4 sa = (f32x4){0, 0, 0, 0}, sb = (f32x4){0, 0, 0, 0};
#pragma unroll
    for (int st = 0; st < QS; ++st) {
      u32x4 ka = B.k[0][st], kb = B.k[1][st];
      if (32 * st + 8 * kg >= DQK) ka = kb = (u32x4){0, 0, 0, 0};
      sa = T::mfma16(ka, qf[st], sa);
      sb = T::mfma16(kb, qf[st], sb);
    }
    float x[8];
    float mx = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key = kk + (i < 4 ? 4 * kg + i : 16 + 4 * kg + i - 4);
      const float v = (i < 4 ? sa[i] : sb[i - 4]) * c;
      const bool ok = key < k_end && key <= qpos + wrgt && key >= qpos - wlft;
      x[i] = ok ? v : -__builtin_inff();
      mx = fmaxf(mx, x[i]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = xhalf_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const bool grow = m_new > m_run;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float alpha = grow ? fast_exp2(m_run - m_new) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DVB; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) o[i][e] *= alpha;
    }
    m_run = m_new;
    const float msub = (m_new == -__builtin_inff()) ? 0.f : m_new;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[i] = fast_exp2(x[i] - msub);
      l_run += x[i];
    }
    const u32x4 pf = (u32x4){T::pack2(x[0], x[1]), T::pack2(x[2], x[3]), T::pack2(x[4], x[5]),
                             T::pack2(x[6], x[7])};
    const int rowa = 4 * kg + tr_t, rowb = 16 + 4 * kg + tr_t;
#pragma unroll
    for (int i = 0; i < DVB; ++i) {
      const int col = i * 16 + 4 * tr_q;
      const int ch = col >> 3, within = col & 7;
      const u32x2 lo = lds_read_tr16(vt + rowa * DV + ((ch ^ swz_v<CV>(rowa)) << 3) + within);
      const u32x2 hi = lds_read_tr16(vt + rowb * DV + ((ch ^ swz_v<CV>(rowb)) << 3) + within);
      o[i] = T::mfma16((u32x4){lo[0], lo[1], hi[0], hi[1]}, pf, o[i]);
    }
  };

  // fused append: the split whose range holds positions [c_b, L) first writes
  // the rotated keys and the values of those rows into the cache, then reads
  // them back like any other row (no other split reads them)
  if (FUSED) {
    const int n0 = max(off, k_begin), n1 = min(L, k_end);
    if (n0 < n1) {
      uint16_t* kc = const_cast<uint16_t*>(kbase);
      uint16_t* vc = const_cast<uint16_t*>(vbase);
      for (int id = lane; id < (n1 - n0) * CK; id += 64) {
        const int key = n0 + id / CK, d = (id % CK) * 8;
        stg16(kc + (int64_t)key * a.k_ss + d,
              rope_chunk<T>(knbase + (int64_t)(key - off) * a.kn_ss, d, a.rcos, a.rsin, key, a.rd, a.rinter, false));
      }
      for (int id = lane; id < (n1 - n0) * CV; id += 64) {
        const int key = n0 + id / CV, d = (id % CV) * 8;
        stg16(vc + (int64_t)key * a.v_ss + d, ldg16(vnbase + (int64_t)(key - off) * a.vn_ss + d));
      }
      __syncthreads();   // stores complete and visible to the whole (single-wave) workgroup
    }
  }

  // three-deep pipeline: K registers A/B/C and LDS stages 0/1/2; two steps'
  // loads are in flight while the current step computes
  KBuf A, B, C;
  load(k_begin, A, 0);
  if (k_begin + 32 < k_end) load(k_begin + 32, B, 1);
  for (int kk = k_begin;;) {
    if (kk + 64 < k_end) load(kk + 64, C, 2);
    step(kk, A, 0, (kk + 32 < k_end) + (kk + 64 < k_end));
    kk += 32;
    if (kk >= k_end) break;
    if (kk + 64 < k_end) load(kk + 64, A, 0);
    step(kk, B, 1, (kk + 32 < k_end) + (kk + 64 < k_end));
    kk += 32;
    if (kk >= k_end) break;
    if (kk + 64 < k_end) load(kk + 64, B, 1);
    step(kk, C, 2, (kk + 32 < k_end) + (kk + 64 < k_end));
    kk += 32;
    if (kk >= k_end) break;
  }

  float lt = l_run + __shfl_xor(l_run, 16);
  lt = xhalf_sum(lt);
  if (nvalid == 1) {
    // the only split of this (batch, kv head): normalise and store
    if (row_ok) {
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      uint16_t* orow = a.out + (int64_t)b * a.o_sb + (int64_t)tok * a.o_ss + (int64_t)hq * a.o_sh;
#pragma unroll
      for (int i = 0; i < DVB; ++i)
        *reinterpret_cast<u32x2*>(orow + i * 16 + 4 * kg) =
            (u32x2){T::pack2(o[i][0] * inv, o[i][1] * inv), T::pack2(o[i][2] * inv, o[i][3] * inv)};
      if (a.lse && kg == 0)
        a.lse[((int64_t)b * a.Hq + hq) * a.Sq + tok] =
            lt > 0.f ? (m_run + __log2f(lt)) * 0.69314718055994531f : -__builtin_inff();
    }
    return;
  }
  if (row_ok) {
    const int64_t slot = (((int64_t)b * a.Hkv + hkv) * a.num_splits + split) * R + r;
    float* wo = a.ws_o + slot * DV;
#pragma unroll
    for (int i = 0; i < DVB; ++i)
      *reinterpret_cast<f32x4*>(wo + i * 16 + 4 * kg) = o[i];
    if (kg == 0) {
      a.ws_ml[slot * 2 + 0] = m_run;
      a.ws_ml[slot * 2 + 1] = lt;
    }
  }
}

// ---------------------------------------------------------------- launchers
template <class T, int DQK, int DV>
static hipError_t launch_decode(const AttnArgs& a, bool causal, hipStream_t st) {
  const dim3 grid((unsigned)(a.Hkv * a.num_splits * a.B));
  if (a.fused) {
    if (causal)
      hipLaunchKernelGGL((decode_attn_kernel<T, DQK, DV, true, true>), grid, dim3(64), 0, st, a);
    else
      hipLaunchKernelGGL((decode_attn_kernel<T, DQK, DV, false, true>), grid, dim3(64), 0, st, a);
  } else {
    if (causal)
      hipLaunchKernelGGL((decode_attn_kernel<T, DQK, DV, true, false>), grid, dim3(64), 0, st, a);
    else
      hipLaunchKernelGGL((decode_attn_kernel<T, DQK, DV, false, false>), grid, dim3(64), 0, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.num_splits <= 1) return e;
  const int64_t rows = (int64_t)a.B * a.Hkv * a.group * a.Sq;
  hipLaunchKernelGGL((split_merge_kernel<T>), dim3((unsigned)rows), dim3(64), 0, st, a, DV);
  return hipGetLastError();
}

template <class T>
static hipError_t launch_decode_t(const AttnArgs& a, int dqk, int dv, bool causal, hipStream_t st) {
  if (dqk == 16 && dv == 16) return launch_decode<T, 16, 16>(a, causal, st);
  if (dqk == 64 && dv == 64) return launch_decode<T, 64, 64>(a, causal, st);
  if (dqk == 128 && dv == 128) return launch_decode<T, 128, 128>(a, causal, st);
  if (dqk == 192 && dv == 128) return launch_decode<T, 192, 128>(a, causal, st);
  return hipErrorInvalidValue;
}

hipError_t run_decode_attn(const AttnArgs& a, int dtype_bf16, int dqk, int dv, bool causal,
                           hipStream_t st) {
  return dtype_bf16 ? launch_decode_t<BF16>(a, dqk, dv, causal, st)
                    : launch_decode_t<F16>(a, dqk, dv, causal, st);
}

}  // namespace attn
