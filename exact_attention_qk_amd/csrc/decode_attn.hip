// Split-KV attention for few query rows per kv head (single-token decode and
// short appends), plus the log-sum-exp merge of the splits.
//
// Method: the decode-time variant of exact attention (flash-attention issue
// #1402, flash_attn_with_kvcache): queries attend the cache prefix of their
// batch.  With one new token per step there are only (Hq/Hkv) * Sq query rows
// per kv head, so the key range of each (batch, kv head) is cut into splits
// that run in parallel; each split keeps its own running max, sum and
// unnormalised output, and a second kernel combines the splits exactly:
//   M = max_s m_s,  l = sum_s l_s 2^(m_s - M),  O = sum_s O_s 2^(m_s - M) / l.
//
// One wave per (split, kv head, batch).  The R <= 16 query rows of a kv head
// are the 16 columns of v_mfma_f32_16x16x32 (unused columns are zero):
//  * S^T = K Q^T with K read straight from HBM into the A operand (16 keys x
//    32 dims per MFMA, 16 contiguous bytes per lane);
//  * the V rows of a 32-key step go global -> registers -> LDS (row-major,
//    swizzled) and come back as the transposed A operand of O^T += V^T P^T
//    through ds_read_b64_tr_b16;
//  * the next step's K and V loads are issued before the current step's math.
// The grid is sized from the cache capacity, so the host never reads the
// device-side cache lengths; splits past a batch's length exit at once.
#include "device_common.hpp"
#include "attn_args.hpp"
#include "launchers.hpp"

namespace attn {

template <class T, int DQK, int DV, bool CAUSAL>
__global__ __launch_bounds__(64) void decode_attn_kernel(AttnArgs a) {
  constexpr int QS = (DQK + 31) / 32;          // 32-dim k-steps of S
  constexpr int CV = DV / 8;                   // chunks per V row
  constexpr int VPL = (32 * CV + 63) / 64;     // V chunks per lane per 32-key step
  constexpr int DVB = DV / 16;                 // 16-wide output blocks
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[32 * DV];

  const int lane = threadIdx.x;
  const int split = blockIdx.x, hkv = blockIdx.y, b = blockIdx.z;
  int L, off;
  if (a.kvcache) {
    int cb = a.seqlens ? a.seqlens[b] : a.seqlen_scalar;
    L = cb + a.Snew;
    off = cb;
  } else {
    L = a.Sk;
    off = a.Sk - a.Sq;
  }
  const int kend_all = CAUSAL ? max(0, min(L, off + a.Sq)) : L;
  const int k_begin = split * a.split_len;
  if (k_begin >= kend_all) return;
  const int k_end = min(kend_all, k_begin + a.split_len);

  const int R = a.group * a.Sq;
  const int r = lane & 15, kg = lane >> 4;
  const int tok = r / a.group;
  const int hq = hkv * a.group + (r - tok * a.group);
  const bool row_ok = r < R;
  const int qpos = off + tok;

  u32x4 qf[QS];
#pragma unroll
  for (int st = 0; st < QS; ++st) {
    const int d = 32 * st + 8 * kg;
    qf[st] = (u32x4){0, 0, 0, 0};
    if (row_ok && d < DQK)
      qf[st] = ldg16(a.q + (int64_t)b * a.q_sb + (int64_t)tok * a.q_ss + (int64_t)hq * a.q_sh + d);
  }

  const uint16_t* kbase = a.k + (int64_t)b * a.k_sb + (int64_t)hkv * a.k_sh;
  const uint16_t* vbase = a.v + (int64_t)b * a.v_sb + (int64_t)hkv * a.v_sh;

  auto load = [&](int kk, u32x4 (&kr)[2][QS], u32x4 (&vr)[VPL]) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int key = kk + 16 * blk + r;
#pragma unroll
      for (int st = 0; st < QS; ++st) {
        const int d = 32 * st + 8 * kg;
        kr[blk][st] = (u32x4){0, 0, 0, 0};
        if (key < k_end && d < DQK) kr[blk][st] = ldg16(kbase + (int64_t)key * a.k_ss + d);
      }
    }
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int id = i * 64 + lane;
      const int row = id / CV, ch = id - (id / CV) * CV;
      const int key = kk + row;
      vr[i] = (u32x4){0, 0, 0, 0};
      if (id < 32 * CV && key < k_end) vr[i] = ldg16(vbase + (int64_t)key * a.v_ss + ch * 8);
    }
  };

  f32x4 o[DVB];
#pragma unroll
  for (int i = 0; i < DVB; ++i) o[i] = (f32x4){0, 0, 0, 0};
  float m_run = -__builtin_inff(), l_run = 0.f;
  const float c = a.c;
  const int tr_t = (lane & 15) >> 2, tr_q = lane & 3;

  u32x4 kc[2][QS], vc[VPL];
  load(k_begin, kc, vc);
  for (int kk = k_begin; kk < k_end; kk += 32) {
    u32x4 kn[2][QS], vn[VPL];
    const bool more = kk + 32 < k_end;
    if (more) load(kk + 32, kn, vn);

    __syncthreads();
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int id = i * 64 + lane;
      const int row = id / CV, ch = id - (id / CV) * CV;
      if (id < 32 * CV)
        *reinterpret_cast<u32x4*>(lds_v + row * DV + ((ch ^ swz_v<CV>(row)) << 3)) = vc[i];
    }
    __syncthreads();

    f32x4 sa = (f32x4){0, 0, 0, 0}, sb = (f32x4){0, 0, 0, 0};
#pragma unroll
    for (int st = 0; st < QS; ++st) {
      sa = T::mfma16(kc[0][st], qf[st], sa);
      sb = T::mfma16(kc[1][st], qf[st], sb);
    }
    float x[8];
    float mx = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key = kk + (i < 4 ? 4 * kg + i : 16 + 4 * kg + i - 4);
      float v = (i < 4 ? sa[i] : sb[i - 4]) * c;
      const bool ok = key < k_end && (!CAUSAL || key <= qpos);
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
      u32x2 lo = lds_read_tr16(lds_v + rowa * DV + ((ch ^ swz_v<CV>(rowa)) << 3) + within);
      u32x2 hi = lds_read_tr16(lds_v + rowb * DV + ((ch ^ swz_v<CV>(rowb)) << 3) + within);
      o[i] = T::mfma16((u32x4){lo[0], lo[1], hi[0], hi[1]}, pf, o[i]);
    }
    if (more) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int st = 0; st < QS; ++st) kc[blk][st] = kn[blk][st];
#pragma unroll
      for (int i = 0; i < VPL; ++i) vc[i] = vn[i];
    }
  }

  float lt = l_run + __shfl_xor(l_run, 16);
  lt = xhalf_sum(lt);
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

// One 64-thread block per (batch, kv head, query row of that kv head).
template <class T>
__global__ __launch_bounds__(64) void split_merge_kernel(AttnArgs a, int DV) {
  const int R = a.group * a.Sq;
  int idx = blockIdx.x;
  const int r = idx % R;
  idx /= R;
  const int hkv = idx % a.Hkv;
  const int b = idx / a.Hkv;
  int L, off;
  if (a.kvcache) {
    int cb = a.seqlens ? a.seqlens[b] : a.seqlen_scalar;
    L = cb + a.Snew;
    off = cb;
  } else {
    L = a.Sk;
    off = a.Sk - a.Sq;
  }
  const int kend_all = a.causal ? max(0, min(L, off + a.Sq)) : L;
  const int nvalid = min(a.num_splits, (kend_all + a.split_len - 1) / a.split_len);
  const int tok = r / a.group;
  const int hq = hkv * a.group + (r - tok * a.group);
  const int64_t slot0 = ((int64_t)b * a.Hkv + hkv) * a.num_splits * R + r;

  float M = -__builtin_inff();
  for (int s = 0; s < nvalid; ++s) M = fmaxf(M, a.ws_ml[(slot0 + (int64_t)s * R) * 2]);
  float lsum = 0.f;
  if (M != -__builtin_inff()) {
    for (int s = 0; s < nvalid; ++s) {
      const float ms = a.ws_ml[(slot0 + (int64_t)s * R) * 2];
      const float ls = a.ws_ml[(slot0 + (int64_t)s * R) * 2 + 1];
      if (ms != -__builtin_inff()) lsum += ls * fast_exp2(ms - M);
    }
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  uint16_t* orow = a.out + (int64_t)b * a.o_sb + (int64_t)tok * a.o_ss + (int64_t)hq * a.o_sh;
  for (int dv = threadIdx.x; dv < DV; dv += 64) {
    float acc = 0.f;
    if (lsum > 0.f) {
      for (int s = 0; s < nvalid; ++s) {
        const float ms = a.ws_ml[(slot0 + (int64_t)s * R) * 2];
        if (ms == -__builtin_inff()) continue;
        acc += a.ws_o[(slot0 + (int64_t)s * R) * DV + dv] * fast_exp2(ms - M);
      }
    }
    orow[dv] = T::from_f32(acc * inv);
  }
  if (a.lse && threadIdx.x == 0)
    a.lse[((int64_t)b * a.Hq + hq) * a.Sq + tok] =
        lsum > 0.f ? (M + __log2f(lsum)) * 0.69314718055994531f : -__builtin_inff();
}

// ---------------------------------------------------------------- launchers
template <class T, int DQK, int DV>
static hipError_t launch_decode(const AttnArgs& a0, bool causal, hipStream_t st) {
  AttnArgs a = a0;
  dim3 grid((unsigned)a.num_splits, (unsigned)a.Hkv, (unsigned)a.B);
  if (causal)
    hipLaunchKernelGGL((decode_attn_kernel<T, DQK, DV, true>), grid, dim3(64), 0, st, a);
  else
    hipLaunchKernelGGL((decode_attn_kernel<T, DQK, DV, false>), grid, dim3(64), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
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
