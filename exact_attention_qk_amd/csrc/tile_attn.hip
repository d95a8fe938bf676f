// Tiled exact attention with an online softmax for gfx950 (prefill and
// chunked prefill over a KV cache).
//
// Method: exact attention softmax(scale * Q K^T + mask) V computed tile by tile
// with a running row max and row sum, so the score matrix never leaves
// registers (skill page "Flash Attention - Fast Memory-Efficient Attention":
// Quick start on IO-aware tiling; Workflow 1 Step 2 for the definition it
// must equal).
//
// Work decomposition (one workgroup = NW waves of 64 lanes):
//  * a workgroup owns BM = 32*NW query rows of one (batch, q head); each wave
//    owns 32 rows and keeps their Q fragment in registers for the whole pass;
//  * K/V tiles of BN = 64 keys are staged global -> registers -> LDS, the next
//    tile's global loads in flight while the current tile is consumed;
//  * S^T = K Q^T on v_mfma_f32_32x32x16 (K from LDS, Q from registers), so a
//    lane owns one query row: the row max needs a single lane^32 exchange and
//    the row sum none until the end;
//  * the K rows fed to the MFMA are permuted so that each lane's 8-score
//    groups cover 8 consecutive keys; those scores, rounded to the input type,
//    are directly the B operand of O^T += V^T P^T, whose A operand V^T is read
//    from the row-major V tile with ds_read_b64_tr_b16;
//  * causal: each wave skips 32-key blocks that lie entirely above its rows'
//    diagonal and masks only blocks that cross it; key rows past the key
//    length are never loaded (zero-filled) and masked;
//  * epilogue: O / l rounded to the output type, staged through LDS so each
//    lane stores 16 contiguous bytes of an output row.
#include "device_common.hpp"
#include "attn_args.hpp"
#include "launchers.hpp"

namespace attn {

constexpr int BN = 64;

// MFMA row m of a 32-key block -> key offset inside the block (see header).
__device__ __forceinline__ int key_perm(int m) {
  int a = m >> 3, hh = (m >> 2) & 1, b = m & 3;
  return 16 * (a >> 1) + 8 * hh + 4 * (a & 1) + b;
}

template <class T, int DQK, int DV, bool CAUSAL, int NW>
__global__ __launch_bounds__(64 * NW, 2) void tile_attn_kernel(AttnArgs a) {
  constexpr int NT = 64 * NW;
  constexpr int BM = 32 * NW;
  constexpr int CK = DQK / 8;             // 16-byte chunks per K row
  constexpr int CV = DV / 8;              // 16-byte chunks per V row
  constexpr int KSTEPS = DQK / 16;        // MFMA k-steps for S
  constexpr int DVB = (DV + 31) / 32;     // 32-wide output blocks
  constexpr int KPT = (BN * CK + NT - 1) / NT;
  constexpr int VPT = (BN * CV + NT - 1) / NT;
  constexpr int OSTR = DV + 8;            // padded row stride of the output staging tile
  constexpr int LDS_KV = BN * (DQK + DV);
  constexpr int LDS_O = NW * 32 * OSTR;
  constexpr int LDS_ELEMS = LDS_KV > LDS_O ? LDS_KV : LDS_O;
  __shared__ __attribute__((aligned(16))) uint16_t lds[LDS_ELEMS];
  uint16_t* lds_k = lds;
  uint16_t* lds_v = lds + BN * DQK;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int hh = lane >> 5;

  // ---- which (batch, q head, q tile) this workgroup owns
  int u = blockIdx.x;
  const int total = gridDim.x;
  if (a.xcd_remap) {  // consecutive units on one XCD so their K/V stay in its L2
    int per = total >> 3;
    u = (u & 7) * per + (u >> 3);
  }
  const int nqt = a.num_qtiles;
  const int bh = u / nqt;
  int qt = u - bh * nqt;
  if (CAUSAL) qt = nqt - 1 - qt;  // heavy tiles first within a (batch, head)
  const int b = bh / a.Hq;
  const int hq = bh - b * a.Hq;
  const int hkv = hq / a.group;

  int L, off;
  if (a.kvcache) {
    int cb = a.seqlens ? a.seqlens[b] : a.seqlen_scalar;
    L = cb + a.Snew;
    off = cb;
  } else {
    L = a.Sk;
    off = a.Sk - a.Sq;
  }
  const int q0 = qt * BM;
  const int rows_end = min(q0 + BM, a.Sq);
  int kend = L;
  if (CAUSAL) kend = max(0, min(L, off + rows_end));
  const int ntiles = (kend + BN - 1) / BN;

  // per-wave row range
  const int wr0 = q0 + 32 * w;
  const int wr1 = min(wr0 + 32, a.Sq);        // exclusive
  const bool wave_active = wr0 < a.Sq;
  const int pmin = off + wr0;                  // smallest query position of the wave
  const int pmax = off + wr1 - 1;              // largest
  int wkend = L;
  if (CAUSAL) wkend = max(0, min(L, pmax + 1));

  const uint16_t* qbase = a.q + (int64_t)b * a.q_sb + (int64_t)hq * a.q_sh;
  const uint16_t* kbase = a.k + (int64_t)b * a.k_sb + (int64_t)hkv * a.k_sh;
  const uint16_t* vbase = a.v + (int64_t)b * a.v_sb + (int64_t)hkv * a.v_sh;

  // ---- Q fragment (B operand of S^T = K Q^T): row l%32, dims 16s + 8h .. +7
  const int qrow = wr0 + (lane & 31);
  u32x4 qf[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    qf[s] = (u32x4){0, 0, 0, 0};
    if (qrow < a.Sq) qf[s] = ldg16(qbase + (int64_t)qrow * a.q_ss + 16 * s + 8 * hh);
  }

  f32x16 o[DVB];
#pragma unroll
  for (int i = 0; i < DVB; ++i) o[i] = (f32x16){};
  float m_run = -__builtin_inff();
  float l_run = 0.f;
  const float c = a.c;
  const int qpos = off + qrow;

  // ---- tile loader (global -> registers -> LDS)
  u32x4 kreg[KPT], vreg[VPT];
  auto load_tile = [&](int t) {
    const int key0 = t * BN;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      int id = i * NT + tid;
      int row = id / CK, ch = id - (id / CK) * CK;
      int key = key0 + row;
      kreg[i] = (u32x4){0, 0, 0, 0};
      if (id < BN * CK && key < L) kreg[i] = ldg16(kbase + (int64_t)key * a.k_ss + ch * 8);
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      int id = i * NT + tid;
      int row = id / CV, ch = id - (id / CV) * CV;
      int key = key0 + row;
      vreg[i] = (u32x4){0, 0, 0, 0};
      if (id < BN * CV && key < L) vreg[i] = ldg16(vbase + (int64_t)key * a.v_ss + ch * 8);
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      int id = i * NT + tid;
      int row = id / CK, ch = id - (id / CK) * CK;
      if (id < BN * CK)
        *reinterpret_cast<u32x4*>(lds_k + row * DQK + ((ch ^ swz_k<CK>(row)) << 3)) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      int id = i * NT + tid;
      int row = id / CV, ch = id - (id / CV) * CV;
      if (id < BN * CV)
        *reinterpret_cast<u32x4*>(lds_v + row * DV + ((ch ^ swz_v<CV>(row)) << 3)) = vreg[i];
    }
  };

  if (ntiles > 0) load_tile(0);

  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (t + 1 < ntiles) load_tile(t + 1);

    const int key0 = t * BN;
    if (!wave_active || key0 >= wkend) continue;   // whole tile above this wave's diagonal

    // ---- S^T for the two 32-key blocks
    f32x16 sc[2];
    bool blk_on[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      blk_on[kb] = key0 + kb * 32 < wkend;
      sc[kb] = (f32x16){};
      if (blk_on[kb]) {
        const int krow = kb * 32 + key_perm(lane & 31);
        const uint16_t* kr = lds_k + krow * DQK;
        const int sw = swz_k<CK>(krow);
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
          u32x4 af = *reinterpret_cast<const u32x4*>(kr + (((2 * s + hh) ^ sw) << 3));
          sc[kb] = T::mfma32(af, qf[s], sc[kb]);
        }
      }
    }

    // ---- scale, mask, row max
    const bool need_mask = (key0 + BN > L) || (CAUSAL && key0 + BN - 1 > pmin);
    float mx = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = sc[kb][r] * c;
        if (need_mask) {
          int key = key0 + kb * 32 + 16 * (r >> 3) + 8 * hh + (r & 7);
          bool ok = blk_on[kb] && key < L && (!CAUSAL || key <= qpos);
          x = ok ? x : -__builtin_inff();
        } else if (!blk_on[kb]) {
          x = -__builtin_inff();
        }
        sc[kb][r] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = xhalf_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const bool grow = m_new > m_run;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float alpha = grow ? fast_exp2(m_run - m_new) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DVB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
    }
    m_run = m_new;
    const float msub = (m_new == -__builtin_inff()) ? 0.f : m_new;

    // ---- P = exp2(x - m), row-sum, pack to the input type
    u32x4 pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = fast_exp2(sc[kb][r] - msub);
        sc[kb][r] = p;
        l_run += p;
      }
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        pf[kb][t2] = (u32x4){T::pack2(sc[kb][8 * t2 + 0], sc[kb][8 * t2 + 1]),
                             T::pack2(sc[kb][8 * t2 + 2], sc[kb][8 * t2 + 3]),
                             T::pack2(sc[kb][8 * t2 + 4], sc[kb][8 * t2 + 5]),
                             T::pack2(sc[kb][8 * t2 + 6], sc[kb][8 * t2 + 7])};
      }
    }

    // ---- O^T += V^T P^T
    const int grp = lane >> 4;
    const int tr_t = (lane & 15) >> 2;
    const int tr_q = lane & 3;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (!blk_on[kb]) continue;
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const int rowa = kb * 32 + 16 * t2 + 8 * hh + tr_t;   // keys for slots 0..3
        const int rowb = rowa + 4;                              // keys for slots 4..7
#pragma unroll
        for (int i = 0; i < DVB; ++i) {
          int col = i * 32 + 16 * (grp & 1) + 4 * tr_q;
          const bool dead = (DV < 32) && (grp & 1);            // padding lanes of a 16-wide V
          if (dead) col = 4 * tr_q;
          const int ch = col >> 3, within = col & 7;
          u32x2 lo = lds_read_tr16(lds_v + rowa * DV + ((ch ^ swz_v<CV>(rowa)) << 3) + within);
          u32x2 hi = lds_read_tr16(lds_v + rowb * DV + ((ch ^ swz_v<CV>(rowb)) << 3) + within);
          u32x4 af = (u32x4){lo[0], lo[1], hi[0], hi[1]};
          if (dead) af = (u32x4){0, 0, 0, 0};
          o[i] = T::mfma32(af, pf[kb][t2], o[i]);
        }
      }
    }
  }

  // ---- epilogue
  const float lsum = xhalf_sum(l_run);
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  __syncthreads();
  uint16_t* lds_o = lds + w * 32 * OSTR;
#pragma unroll
  for (int i = 0; i < DVB; ++i) {
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int dv = i * 32 + 8 * a4 + 4 * hh;
      if (dv < DV) {
        u32x2 pk = (u32x2){T::pack2(o[i][4 * a4 + 0] * inv, o[i][4 * a4 + 1] * inv),
                           T::pack2(o[i][4 * a4 + 2] * inv, o[i][4 * a4 + 3] * inv)};
        *reinterpret_cast<u32x2*>(lds_o + (lane & 31) * OSTR + dv) = pk;
      }
    }
  }
  __syncthreads();
  if (wave_active) {
    uint16_t* obase = a.out + (int64_t)b * a.o_sb + (int64_t)hq * a.o_sh;
    constexpr int OCH = 32 * CV;
#pragma unroll
    for (int i = 0; i < (OCH + 63) / 64; ++i) {
      int id = i * 64 + lane;
      int row = id / CV, ch = id - (id / CV) * CV;
      if (id < OCH && wr0 + row < a.Sq) {
        u32x4 val = *reinterpret_cast<const u32x4*>(lds_o + row * OSTR + ch * 8);
        stg16(obase + (int64_t)(wr0 + row) * a.o_ss + ch * 8, val);
      }
    }
    if (a.lse && hh == 0 && qrow < a.Sq) {
      a.lse[((int64_t)b * a.Hq + hq) * a.Sq + qrow] =
          lsum > 0.f ? (m_run + __log2f(lsum)) * 0.69314718055994531f : -__builtin_inff();
    }
  }
}

// ---------------------------------------------------------------- launchers
template <class T, int DQK, int DV, bool CAUSAL>
static hipError_t launch_tile(const AttnArgs& a0, hipStream_t st) {
  constexpr int NW = 4;
  AttnArgs a = a0;
  a.num_qtiles = (a.Sq + 32 * NW - 1) / (32 * NW);
  const int64_t units = (int64_t)a.B * a.Hq * a.num_qtiles;
  if (units <= 0) return hipSuccess;
  a.xcd_remap = (units % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL((tile_attn_kernel<T, DQK, DV, CAUSAL, NW>), dim3((unsigned)units), dim3(64 * NW),
                     0, st, a);
  return hipGetLastError();
}

template <class T, int DQK, int DV>
static hipError_t launch_tile_c(const AttnArgs& a, bool causal, hipStream_t st) {
  return causal ? launch_tile<T, DQK, DV, true>(a, st) : launch_tile<T, DQK, DV, false>(a, st);
}

template <class T>
static hipError_t launch_tile_t(const AttnArgs& a, int dqk, int dv, bool causal, hipStream_t st) {
  if (dqk == 16 && dv == 16) return launch_tile_c<T, 16, 16>(a, causal, st);
  if (dqk == 64 && dv == 64) return launch_tile_c<T, 64, 64>(a, causal, st);
  if (dqk == 128 && dv == 128) return launch_tile_c<T, 128, 128>(a, causal, st);
  if (dqk == 192 && dv == 128) return launch_tile_c<T, 192, 128>(a, causal, st);
  return hipErrorInvalidValue;
}

hipError_t run_tile_attn(const AttnArgs& a, int dtype_bf16, int dqk, int dv, bool causal,
                         hipStream_t st) {
  return dtype_bf16 ? launch_tile_t<BF16>(a, dqk, dv, causal, st)
                    : launch_tile_t<F16>(a, dqk, dv, causal, st);
}

}  // namespace attn
