// Gradients of exact attention for gfx950: dQ, dK, dV for a given dO, with
// head_dim_qk != head_dim_v allowed (flash-attention PR #1604 "Support
// hdimQK != hdimV backward": the backward pass with differing head sizes; the
// kernels here tile K and V at their own widths, the option that PR names as
// the better one).
//
// With P = exp(scale * Q K^T - lse) recomputed from the forward pass's row
// log-sum-exp, and D = rowsum(dO * O):
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
//
// Two launches:
//  * bwd_dq_kernel: a wave owns 32 query rows of one (batch, q head) (their Q
//    and dO fragments in registers), first computes each row's lse * log2(e)
//    and D = rowsum(dO * O) (stored in the workspace for the next kernel),
//    then streams 32-key K/V tiles through LDS, like the forward kernel:
//    S^T = K Q^T and
//    dP^T = V dO^T leave each lane with one query row, so P and dS need no
//    cross-lane work; dQ^T += K^T dS^T reads K^T with ds_read_b64_tr_b16;
//  * bwd_dkdv_kernel: the same with the roles of queries and keys swapped: a
//    wave owns 32 keys of one (batch, kv head) (K, V fragments in registers)
//    and streams 32-row Q / dO / (lse, D) tiles of every q head that reads
//    this kv head, accumulating dK^T += Q^T dS and dV^T += dO^T P; summing
//    over the group in registers needs no atomics.
// Inside a workgroup, key-split (dQ) or row-split (dK/dV) groups of waves
// walk disjoint tiles and add their partial sums through LDS at the end;
// causal launches dispatch the longest tiles of every head first, so the
// short ones fill the tail (a complementary-pair mode remains in the kernels).
// Both stream through double-buffered LDS stages filled by buffer loads whose
// resource ends at the last valid row (rows past it read as zero and are
// masked).  Masks: key length, causal (bottom-right), local window.
#include "device_common.hpp"
#include "attn_args.hpp"
#include "launchers.hpp"

namespace attn {
namespace {

__device__ __forceinline__ int perm32(int m) {   // the K-row order of the forward kernel
  const int a = m >> 3, hh = (m >> 2) & 1, b = m & 3;
  return 16 * (a >> 1) + 8 * hh + 4 * (a & 1) + b;
}

template <class T>
__device__ __forceinline__ uint32_t packw(float a, float b) { return T::pack2(a, b); }

// Row-major tile of 32 rows x D elements in LDS, 16-byte chunks swizzled by
// row (SK: the K-side swizzle, else the V-side one).
template <int D, bool SK>
__device__ __forceinline__ int swz(int r) {
  return SK ? swz_k<D / 8>(r) : swz_v<D / 8>(r);
}
// 16 bytes of row `row`, chunk `chunk` (the A operand of a row-major product)
template <int D, bool SK>
__device__ __forceinline__ u32x4 row_frag(const uint16_t* tile, int row, int chunk) {
  return *reinterpret_cast<const u32x4*>(tile + row * D + ((chunk ^ swz<D, SK>(row)) << 3));
}
// transposed operand: elements (rowa..rowa+3, rowa+4..rowa+7) of column col
template <int D, bool SK>
__device__ __forceinline__ u32x4 tr_frag(const uint16_t* tile, int rowa, int col) {
  const int ch = col >> 3, within = col & 7;
  const u32x2 lo = lds_read_tr16(tile + rowa * D + ((ch ^ swz<D, SK>(rowa)) << 3) + within);
  const u32x2 hi = lds_read_tr16(tile + (rowa + 4) * D + ((ch ^ swz<D, SK>(rowa + 4)) << 3) + within);
  return (u32x4){lo[0], lo[1], hi[0], hi[1]};
}
// byte offset of this lane's 16-B piece of DMA instruction i of a 32 x D tile
template <int D, bool SK>
__device__ __forceinline__ int dma_off(int i, int lane, int64_t row_stride) {
  constexpr int C = D / 8;
  const int P = i * 64 + lane, row = P / C, pos = P % C;
  return (int)(row * row_stride * 2) + ((pos ^ swz<D, SK>(row)) << 4);
}

}  // namespace

// ---------------------------------------------------------------- dQ
// A workgroup is NS key-split groups of NR waves; a wave owns 32 query rows,
// the groups walk disjoint key tiles (tile t to group t % NS) through their
// own double-buffered LDS stages, and their dQ partial sums are added through
// LDS at the end.  PAIR (causal): a unit is the query-tile pair (n-1-p, p).
template <class T, int DQK, int DV, bool CAUSAL, bool WIN, int NR, int NS, bool PAIR, int MINW>
__global__ __launch_bounds__(64 * NR * NS, MINW) void bwd_dq_kernel(BwdArgs a) {
  constexpr int KS = DQK / 16, VS = DV / 16, QB = DQK / 32;
  constexpr int BM = 32 * NR;
  constexpr int KT = 32 * DQK, VT = 32 * DV, STAGE = KT + VT;
  constexpr int NIK = DQK / 16, NIV = DV / 16;                 // 1 KiB DMA instructions per tile
  constexpr int JK = (NIK + NR - 1) / NR, JV = (NIV + NR - 1) / NR;
  constexpr int OSTR = DQK + 8;
  constexpr int LDS_KV = NS * 2 * STAGE * 2;
  constexpr int MERGE = (NS - 1) * NR * QB * 16 * 64 * 4;
  constexpr int LDS_O = BM * OSTR * 2;
  constexpr int LDS_A = LDS_KV > MERGE ? LDS_KV : MERGE;
  constexpr int LDS_BYTES = LDS_A > LDS_O ? LDS_A : LDS_O;
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_BYTES];
  uint16_t* lds16 = reinterpret_cast<uint16_t*>(smem);
  const uint32_t smem_addr = (uint32_t)reinterpret_cast<uintptr_t>((LDS_AS void*)smem);

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = w / NR, rw = w - g * NR;
  const int hh = lane >> 5;
  const int nt = a.num_tiles;
  const int nub = PAIR ? (nt + 1) / 2 : nt;
  const int BH = a.B * a.Hq;
  int bh, pu;
  if (PAIR) {
    int u = blockIdx.x;
    if (a.xcd_remap) {
      const int per = gridDim.x >> 3;
      u = (u & 7) * per + (u >> 3);
    }
    bh = u / nub;
    pu = u - bh * nub;
  } else {   // tile rank major: the longest tiles are dispatched first; a head stays on one XCD when BH % 8 == 0
    pu = blockIdx.x / BH;
    bh = blockIdx.x - pu * BH;
  }
  const int b = bh / a.Hq, hq = bh - b * a.Hq, hkv = hq / a.group;
  const int nslots = (PAIR && nt - 1 - pu != pu) ? 2 : 1;
  const int L = a.Sk, off = a.Sk - a.Sq;
  const int wrgt = WIN ? (CAUSAL ? min(a.wr, 0) : a.wr) : 0;
  const int wlft = WIN ? a.wl : 0;
  const uint16_t* kbase = a.k + (int64_t)b * a.k_sb + (int64_t)hkv * a.k_sh;
  const uint16_t* vbase = a.v + (int64_t)b * a.v_sb + (int64_t)hkv * a.v_sh;
  const int grp = lane >> 4, tr_t = (lane & 15) >> 2, tr_q = lane & 3;
  const float c = a.c;

  int koff[JK], voff[JV];
#pragma unroll
  for (int j = 0; j < JK; ++j) koff[j] = dma_off<DQK, true>(min(rw + NR * j, NIK - 1), lane, a.k_ss);
#pragma unroll
  for (int j = 0; j < JV; ++j) voff[j] = dma_off<DV, false>(min(rw + NR * j, NIV - 1), lane, a.v_ss);

#pragma clang loop unroll(disable)
  for (int slot = 0; slot < nslots; ++slot) {
    int qt = pu;
    if (CAUSAL) qt = (PAIR && slot == 1) ? pu : nt - 1 - pu;   // the longer key range first
    const int q0 = qt * BM;
    const int rows_end = min(q0 + BM, a.Sq);
    int kend = L, kbeg = 0;
    if (WIN || CAUSAL) kend = max(0, min(L, off + rows_end + wrgt));
    if (WIN) kbeg = min(kend, max(0, off + q0 - wlft));
    const int t_lo = kbeg / 32;
    const int ntiles = max(0, (kend + 31) / 32 - t_lo);
    const int nit = (ntiles + NS - 1) / NS;

    const int wr0 = q0 + rw * 32;
    const int wr1 = min(wr0 + 32, a.Sq);
    const bool wave_active = wr0 < a.Sq;
    int wkend = L, wkbeg = 0;
    if (WIN || CAUSAL) wkend = max(0, min(L, off + wr1 + wrgt));
    if (WIN) wkbeg = max(0, off + wr0 - wlft);
    const int row = wr0 + (lane & 31);             // this lane's query row
    const bool row_ok = row < a.Sq;
    const int rc = min(row, a.Sq - 1);
    const int qpos = off + row;

    u32x4 qf[KS], dof[VS];
    {
      const uint16_t* qr = a.q + (int64_t)b * a.q_sb + (int64_t)rc * a.q_ss + (int64_t)hq * a.q_sh;
      const uint16_t* dr = a.dout + (int64_t)b * a.do_sb + (int64_t)rc * a.do_ss + (int64_t)hq * a.do_sh;
#pragma unroll
      for (int st = 0; st < KS; ++st) qf[st] = ldg16(qr + 16 * st + 8 * hh);
#pragma unroll
      for (int st = 0; st < VS; ++st) dof[st] = ldg16(dr + 16 * st + 8 * hh);
    }
    // this row's lse * log2(e) and D = rowsum(dO * O) (lanes l and l ^ 32 hold
    // the two halves of every 16 dims); group 0 also stores them for the dK/dV
    // kernel, which runs after this one
    const int64_t lrow = ((int64_t)b * a.Hq + hq) * a.Sq + rc;
    float Dp = 0.f;
    {
      const uint16_t* orow = a.o + (int64_t)b * a.o_sb + (int64_t)rc * a.o_ss + (int64_t)hq * a.o_sh;
#pragma unroll
      for (int st = 0; st < VS; ++st) {
        const u32x4 ov = ldg16(orow + 16 * st + 8 * hh);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          Dp += T::to_f32((uint16_t)(dof[st][e] & 0xFFFFu)) * T::to_f32((uint16_t)(ov[e] & 0xFFFFu));
          Dp += T::to_f32((uint16_t)(dof[st][e] >> 16)) * T::to_f32((uint16_t)(ov[e] >> 16));
        }
      }
    }
    const float Drow = xhalf_sum(Dp);
    const float lse2 = a.lse[lrow] * 1.4426950408889634f;
    if (g == 0 && hh == 0 && row_ok) {
      a.ld[2 * lrow] = lse2;
      a.ld[2 * lrow + 1] = Drow;
    }

    auto issue = [&](int t, int s) {
      const int key0 = t * 32, rows = min(32, L - key0);
      const i32x4 rk = make_rsrc(kbase + (int64_t)key0 * a.k_ss, rows * (int)a.k_ss * 2);
      const i32x4 rv = make_rsrc(vbase + (int64_t)key0 * a.v_ss, rows * (int)a.v_ss * 2);
      const uint32_t kd = smem_addr + (uint32_t)((g * 2 + s) * STAGE) * 2, vd = kd + KT * 2;
#pragma unroll
      for (int j = 0; j < JK; ++j)
        if (NIK % NR == 0 || rw + NR * j < NIK) dma_b128(rk, kd + (rw + NR * j) * 1024, koff[j]);
#pragma unroll
      for (int j = 0; j < JV; ++j)
        if (NIV % NR == 0 || rw + NR * j < NIV) dma_b128(rv, vd + (rw + NR * j) * 1024, voff[j]);
    };

    f32x16 dq[QB];
#pragma unroll
    for (int i = 0; i < QB; ++i) dq[i] = (f32x16){};

    if (g < ntiles) issue(t_lo + g, 0);
    // two tiles per trip, the inner loop unrolled: each copy's LDS stage s is a
    // constant, so its LDS reads take immediate offsets
    for (int it0 = 0; it0 < nit; it0 += 2) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int it = it0 + s;
        if (it >= nit) break;
        const int tr = it * NS + g;                 // this group's tile, relative to t_lo
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this lane's part of the tile landed
        __syncthreads();                      // ... every lane's; stage s^1 is free again
        if (tr + NS < ntiles) issue(t_lo + tr + NS, s ^ 1);
        const int key0 = (t_lo + tr) * 32;
        if (tr >= ntiles || !wave_active || key0 >= wkend || (WIN && key0 + 32 <= wkbeg)) continue;
        const uint16_t* kt = lds16 + (g * 2 + s) * STAGE;
        const uint16_t* vt = kt + KT;
        // S^T = K Q^T and dP^T = V dO^T, keys in the forward kernel's order
        const int prow = perm32(lane & 31);
        f32x16 sc = (f32x16){}, dp = (f32x16){};
  #pragma unroll
        for (int st = 0; st < KS; ++st) sc = T::mfma32(row_frag<DQK, true>(kt, prow, 2 * st + hh), qf[st], sc);
  #pragma unroll
        for (int st = 0; st < VS; ++st) dp = T::mfma32(row_frag<DV, false>(vt, prow, 2 * st + hh), dof[st], dp);
        u32x4 dsf[2];
  #pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          float d[8];
  #pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int r = 8 * t2 + e;
            const int key = key0 + 16 * t2 + 8 * hh + e;
            bool ok = row_ok && key < L;
            if (WIN || CAUSAL) ok = ok && key <= qpos + wrgt;
            if (WIN) ok = ok && key >= qpos - wlft;
            const float p = ok ? fast_exp2(__builtin_fmaf(sc[r], c, -lse2)) : 0.f;
            d[e] = p * (dp[r] - Drow);
          }
          dsf[t2] = (u32x4){packw<T>(d[0], d[1]), packw<T>(d[2], d[3]), packw<T>(d[4], d[5]), packw<T>(d[6], d[7])};
        }
        // dQ^T += K^T dS^T
  #pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          const int rowa = 16 * t2 + 8 * hh + tr_t;
  #pragma unroll
          for (int i = 0; i < QB; ++i)
            dq[i] = T::mfma32(tr_frag<DQK, true>(kt, rowa, i * 32 + 16 * (grp & 1) + 4 * tr_q), dsf[t2], dq[i]);
        }
      }
    }

    __syncthreads();
    if constexpr (NS > 1) {   // add the key-split groups' partial sums into group 0
      float* mo = reinterpret_cast<float*>(smem);
      if (g > 0) {
#pragma unroll
        for (int i = 0; i < QB; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) mo[((((g - 1) * NR + rw) * QB + i) * 16 + r) * 64 + lane] = dq[i][r];
      }
      __syncthreads();
      if (g == 0) {
        for (int gg = 1; gg < NS; ++gg)
#pragma unroll
          for (int i = 0; i < QB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) dq[i][r] += mo[((((gg - 1) * NR + rw) * QB + i) * 16 + r) * 64 + lane];
      }
      __syncthreads();
    }

    // epilogue (group 0): scale, round, stage through LDS, 16-byte stores of whole rows
    if (g == 0 && wave_active) {
      uint16_t* st_o = lds16 + rw * 32 * OSTR;
#pragma unroll
      for (int i = 0; i < QB; ++i)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const int d = i * 32 + 8 * a4 + 4 * hh;
          *reinterpret_cast<u32x2*>(st_o + (lane & 31) * OSTR + d) =
              (u32x2){T::pack2(dq[i][4 * a4 + 0] * a.scale, dq[i][4 * a4 + 1] * a.scale),
                      T::pack2(dq[i][4 * a4 + 2] * a.scale, dq[i][4 * a4 + 3] * a.scale)};
        }
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
      __builtin_amdgcn_wave_barrier();
      constexpr int CH = DQK / 8;
      for (int id = lane; id < 32 * CH; id += 64) {
        const int r = id / CH, ch = id - r * CH;
        const int qrow = wr0 + r;
        if (qrow < a.Sq)
          stg16(a.dq + (int64_t)b * a.dq_sb + (int64_t)qrow * a.dq_ss + (int64_t)hq * a.dq_sh + ch * 8,
                *reinterpret_cast<const u32x4*>(st_o + r * OSTR + ch * 8));
      }
    }
    __syncthreads();   // the next slot refills LDS
  }
}

// ---------------------------------------------------------------- dK, dV
// The same split with the roles of queries and keys swapped: a wave owns 32
// keys, the NS groups walk disjoint (q head, 32-row block) steps, and their
// dK/dV partial sums are added through LDS.  PAIR (causal): key tiles (p, n-1-p).
// KVL: K and V stay in LDS (a 32-key tile per wave column, shared by the
// groups) instead of registers, which leaves room for two waves per SIMD at
// the larger head sizes.
template <class T, int DQK, int DV, bool CAUSAL, bool WIN, int NR, int NS, bool PAIR, int MINW, bool KVL>
__global__ __launch_bounds__(64 * NR * NS, MINW) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int KS = DQK / 16, VS = DV / 16, KB = DQK / 32, VB = DV / 32;
  constexpr int BK = 32 * NR;
  constexpr int QT = 32 * DQK, OT = 32 * DV, LT = 32 * 2 * 2;     // elements: Q, dO, (lse, D) tiles
  constexpr int STAGE = QT + OT + LT;
  constexpr int NIQ = DQK / 16, NIO = DV / 16;
  constexpr int JQ = (NIQ + NR - 1) / NR, JO = (NIO + NR - 1) / NR;
  constexpr int OSTR = (DQK > DV ? DQK : DV) + 8;
  constexpr int RES = KVL ? NR * 32 * (DQK + DV) : 0;            // elements of resident K/V tiles
  constexpr int LDS_KV = RES * 2 + NS * 2 * STAGE * 2;
  constexpr int MERGE = (NS - 1) * NR * (KB + VB) * 16 * 64 * 4;
  constexpr int LDS_O = BK * OSTR * 2;
  constexpr int LDS_A = LDS_KV > MERGE ? LDS_KV : MERGE;
  constexpr int LDS_BYTES = LDS_A > LDS_O ? LDS_A : LDS_O;
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_BYTES];
  uint16_t* lds16 = reinterpret_cast<uint16_t*>(smem);
  const uint32_t smem_addr = (uint32_t)reinterpret_cast<uintptr_t>((LDS_AS void*)smem);

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = w / NR, rw = w - g * NR;
  const int hh = lane >> 5;
  const int nt = a.num_tiles;
  const int nub = PAIR ? (nt + 1) / 2 : nt;
  const int BH = a.B * a.Hkv;
  int bh, pu;
  if (PAIR) {
    int u = blockIdx.x;
    if (a.xcd_remap) {
      const int per = gridDim.x >> 3;
      u = (u & 7) * per + (u >> 3);
    }
    bh = u / nub;
    pu = u - bh * nub;
  } else {   // tile rank major, as in the dQ kernel
    pu = blockIdx.x / BH;
    bh = blockIdx.x - pu * BH;
  }
  const int b = bh / a.Hkv, hkv = bh - b * a.Hkv;
  const int nslots = (PAIR && nt - 1 - pu != pu) ? 2 : 1;
  const int L = a.Sk, off = a.Sk - a.Sq;
  const int wrgt = WIN ? (CAUSAL ? min(a.wr, 0) : a.wr) : 0;
  const int wlft = WIN ? a.wl : 0;
  const int grp = lane >> 4, tr_t = (lane & 15) >> 2, tr_q = lane & 3;
  const float c = a.c;

  int qoff[JQ], ooff[JO];
#pragma unroll
  for (int j = 0; j < JQ; ++j) qoff[j] = dma_off<DQK, true>(min(rw + NR * j, NIQ - 1), lane, a.q_ss);
#pragma unroll
  for (int j = 0; j < JO; ++j) ooff[j] = dma_off<DV, false>(min(rw + NR * j, NIO - 1), lane, a.do_ss);

#pragma clang loop unroll(disable)
  for (int slot = 0; slot < nslots; ++slot) {
    const int kt_i = (PAIR && slot == 1) ? nt - 1 - pu : pu;
    const int k0 = kt_i * BK;
    const int k1 = min(k0 + BK, L);
    // query rows that see any key of [k0, k1): position p with k0 - wrgt <= p <= k1 - 1 + wlft
    int r_lo = 0, r_hi = a.Sq;
    if (WIN || CAUSAL) r_lo = min(a.Sq, max(0, k0 - wrgt - off));
    if (WIN) r_hi = max(r_lo, min(a.Sq, k1 - 1 + wlft - off + 1));
    const int rb_lo = r_lo / 32;
    const int nrb = max(0, (r_hi + 31) / 32 - rb_lo);   // row blocks per q head
    const int nsteps = nrb * a.group;
    const int nit = (nsteps + NS - 1) / NS;

    const int wk0 = k0 + rw * 32;
    const int key = wk0 + (lane & 31);                  // this lane's key
    const bool key_ok = key < L;
    const int kc = min(key, L - 1);
    u32x4 kf[KVL ? 1 : KS], vf[KVL ? 1 : VS];
    const uint16_t* kres = lds16 + rw * 32 * (DQK + DV);
    const uint16_t* vres = kres + 32 * DQK;
    if constexpr (KVL) {
      // this wave column's K and V tiles; the NS waves that share it split the copies
      if (wk0 < L) {
        const int rows = min(32, L - wk0);
        const i32x4 rk = make_rsrc(a.k + (int64_t)b * a.k_sb + (int64_t)wk0 * a.k_ss + (int64_t)hkv * a.k_sh,
                                   rows * (int)a.k_ss * 2);
        const i32x4 rv = make_rsrc(a.v + (int64_t)b * a.v_sb + (int64_t)wk0 * a.v_ss + (int64_t)hkv * a.v_sh,
                                   rows * (int)a.v_ss * 2);
        const uint32_t kd = smem_addr + (uint32_t)(rw * 32 * (DQK + DV)) * 2, vd = kd + 32 * DQK * 2;
        for (int i = g; i < NIQ; i += NS) dma_b128(rk, kd + i * 1024, dma_off<DQK, true>(i, lane, a.k_ss));
        for (int i = g; i < NIO; i += NS) dma_b128(rv, vd + i * 1024, dma_off<DV, true>(i, lane, a.v_ss));
      }
    } else {
      const uint16_t* kr = a.k + (int64_t)b * a.k_sb + (int64_t)kc * a.k_ss + (int64_t)hkv * a.k_sh;
      const uint16_t* vr = a.v + (int64_t)b * a.v_sb + (int64_t)kc * a.v_ss + (int64_t)hkv * a.v_sh;
#pragma unroll
      for (int st = 0; st < KS; ++st) kf[st] = ldg16(kr + 16 * st + 8 * hh);
#pragma unroll
      for (int st = 0; st < VS; ++st) vf[st] = ldg16(vr + 16 * st + 8 * hh);
    }

    // step n: q head hkv * group + n / nrb, row block rb_lo + n % nrb
    auto issue = [&](int n, int s) {
      const int h = hkv * a.group + n / nrb;
      const int r0 = (rb_lo + n % nrb) * 32, rows = min(32, a.Sq - r0);
      const i32x4 rq = make_rsrc(a.q + (int64_t)b * a.q_sb + (int64_t)r0 * a.q_ss + (int64_t)h * a.q_sh,
                                 rows * (int)a.q_ss * 2);
      const i32x4 ro = make_rsrc(a.dout + (int64_t)b * a.do_sb + (int64_t)r0 * a.do_ss + (int64_t)h * a.do_sh,
                                 rows * (int)a.do_ss * 2);
      const uint32_t qd = smem_addr + (uint32_t)(RES + (g * 2 + s) * STAGE) * 2, od = qd + QT * 2, ldd = od + OT * 2;
#pragma unroll
      for (int j = 0; j < JQ; ++j)
        if (NIQ % NR == 0 || rw + NR * j < NIQ) dma_b128(rq, qd + (rw + NR * j) * 1024, qoff[j]);
#pragma unroll
      for (int j = 0; j < JO; ++j)
        if (NIO % NR == 0 || rw + NR * j < NIO) dma_b128(ro, od + (rw + NR * j) * 1024, ooff[j]);
      if (rw == 0 && lane < 16) {   // 32 rows of (lse2, D): 256 bytes
        const i32x4 rl = make_rsrc(a.ld + 2 * (((int64_t)b * a.Hq + h) * a.Sq + r0), rows * 8);
        dma_b128(rl, ldd, lane * 16);
      }
    };

    f32x16 dk[KB], dv[VB];
#pragma unroll
    for (int i = 0; i < KB; ++i) dk[i] = (f32x16){};
#pragma unroll
    for (int i = 0; i < VB; ++i) dv[i] = (f32x16){};

    if (g < nsteps) issue(g, 0);
    // two tiles per trip, the inner loop unrolled: each copy's LDS stage s is a
    // constant, so its LDS reads take immediate offsets
    for (int it0 = 0; it0 < nit; it0 += 2) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int it = it0 + s;
        if (it >= nit) break;
        const int n = it * NS + g;
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
        if (n + NS < nsteps) issue(n + NS, s ^ 1);
        if (n >= nsteps || wk0 >= L) continue;
        const int r0 = (rb_lo + n % nrb) * 32;
        // this wave's keys [wk0, wk0 + 32) against the block's band of rows
        if ((WIN || CAUSAL) && wk0 > off + r0 + 31 + wrgt) continue;
        if (WIN && wk0 + 31 < off + r0 - wlft) continue;
        const uint16_t* qt = lds16 + RES + (g * 2 + s) * STAGE;
        const uint16_t* ot = qt + QT;
        const float* lt = reinterpret_cast<const float*>(ot + OT);
        // S = Q K^T and dP = dO V^T: a lane owns a key; its registers cover rows
        // r0 + 16 (r >> 3) + 8 hh + (r & 7)
        const int prow = perm32(lane & 31);
        f32x16 sc = (f32x16){}, dp = (f32x16){};
  #pragma unroll
        for (int st = 0; st < KS; ++st)
          sc = T::mfma32(row_frag<DQK, true>(qt, prow, 2 * st + hh),
                         KVL ? row_frag<DQK, true>(kres, lane & 31, 2 * st + hh) : kf[KVL ? 0 : st], sc);
  #pragma unroll
        for (int st = 0; st < VS; ++st)
          dp = T::mfma32(row_frag<DV, false>(ot, prow, 2 * st + hh),
                         KVL ? row_frag<DV, true>(vres, lane & 31, 2 * st + hh) : vf[KVL ? 0 : st], dp);
        u32x4 pf[2], dsf[2];
  #pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          const f32x4 l0 = *reinterpret_cast<const f32x4*>(lt + 2 * (16 * t2 + 8 * hh));
          const f32x4 l1 = *reinterpret_cast<const f32x4*>(lt + 2 * (16 * t2 + 8 * hh) + 4);
          const f32x4 l2 = *reinterpret_cast<const f32x4*>(lt + 2 * (16 * t2 + 8 * hh) + 8);
          const f32x4 l3 = *reinterpret_cast<const f32x4*>(lt + 2 * (16 * t2 + 8 * hh) + 12);
          const float lsev[8] = {l0[0], l0[2], l1[0], l1[2], l2[0], l2[2], l3[0], l3[2]};
          const float dv8[8] = {l0[1], l0[3], l1[1], l1[3], l2[1], l2[3], l3[1], l3[3]};
          float p[8], d[8];
  #pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int r = 8 * t2 + e;
            const int qrow = r0 + 16 * t2 + 8 * hh + e;
            const int qpos = off + qrow;
            bool ok = key_ok && qrow < a.Sq;
            if (WIN || CAUSAL) ok = ok && key <= qpos + wrgt;
            if (WIN) ok = ok && key >= qpos - wlft;
            p[e] = ok ? fast_exp2(__builtin_fmaf(sc[r], c, -lsev[e])) : 0.f;
            d[e] = p[e] * (dp[r] - dv8[e]);
          }
          pf[t2] = (u32x4){packw<T>(p[0], p[1]), packw<T>(p[2], p[3]), packw<T>(p[4], p[5]), packw<T>(p[6], p[7])};
          dsf[t2] = (u32x4){packw<T>(d[0], d[1]), packw<T>(d[2], d[3]), packw<T>(d[4], d[5]), packw<T>(d[6], d[7])};
        }
        // dV^T += dO^T P and dK^T += Q^T dS
  #pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          const int rowa = 16 * t2 + 8 * hh + tr_t;
  #pragma unroll
          for (int i = 0; i < VB; ++i)
            dv[i] = T::mfma32(tr_frag<DV, false>(ot, rowa, i * 32 + 16 * (grp & 1) + 4 * tr_q), pf[t2], dv[i]);
  #pragma unroll
          for (int i = 0; i < KB; ++i)
            dk[i] = T::mfma32(tr_frag<DQK, true>(qt, rowa, i * 32 + 16 * (grp & 1) + 4 * tr_q), dsf[t2], dk[i]);
        }
      }
    }

    if constexpr (KVL) __builtin_amdgcn_s_waitcnt(0x0F70);   // resident copies landed before LDS is reused
    __syncthreads();
    if constexpr (NS > 1) {   // add the row-split groups' partial sums into group 0
      float* mo = reinterpret_cast<float*>(smem);
      if (g > 0) {
        float* mb = mo + ((g - 1) * NR + rw) * (KB + VB) * 16 * 64;
#pragma unroll
        for (int i = 0; i < KB; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) mb[(i * 16 + r) * 64 + lane] = dk[i][r];
#pragma unroll
        for (int i = 0; i < VB; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) mb[((KB + i) * 16 + r) * 64 + lane] = dv[i][r];
      }
      __syncthreads();
      if (g == 0) {
        for (int gg = 1; gg < NS; ++gg) {
          const float* mb = mo + ((gg - 1) * NR + rw) * (KB + VB) * 16 * 64;
#pragma unroll
          for (int i = 0; i < KB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) dk[i][r] += mb[(i * 16 + r) * 64 + lane];
#pragma unroll
          for (int i = 0; i < VB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) dv[i][r] += mb[((KB + i) * 16 + r) * 64 + lane];
        }
      }
      __syncthreads();
    }

    // epilogue (group 0): dK = scale (dK^T)^T, dV = (dV^T)^T, staged through LDS per wave
    if (g == 0 && wk0 < L) {
      uint16_t* st_o = lds16 + rw * 32 * OSTR;
      auto store = [&](const f32x16* acc, int NB, int D, float mul, uint16_t* gbase, int64_t g_ss) {
        for (int i = 0; i < NB; ++i)
#pragma unroll
          for (int a4 = 0; a4 < 4; ++a4) {
            const int d = i * 32 + 8 * a4 + 4 * hh;
            *reinterpret_cast<u32x2*>(st_o + (lane & 31) * OSTR + d) =
                (u32x2){T::pack2(acc[i][4 * a4 + 0] * mul, acc[i][4 * a4 + 1] * mul),
                        T::pack2(acc[i][4 * a4 + 2] * mul, acc[i][4 * a4 + 3] * mul)};
          }
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_wave_barrier();
        const int CH = D / 8;
        for (int id = lane; id < 32 * CH; id += 64) {
          const int r = id / CH, ch = id - r * CH;
          const int kk = wk0 + r;
          if (kk < L)
            stg16(gbase + (int64_t)kk * g_ss + ch * 8, *reinterpret_cast<const u32x4*>(st_o + r * OSTR + ch * 8));
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_wave_barrier();
      };
      store(dk, KB, DQK, a.scale, a.dk + (int64_t)b * a.dk_sb + (int64_t)hkv * a.dk_sh, a.dk_ss);
      store(dv, VB, DV, 1.f, a.dv + (int64_t)b * a.dv_sb + (int64_t)hkv * a.dv_sh, a.dv_ss);
    }
    __syncthreads();   // the next slot refills LDS
  }
}

// ---------------------------------------------------------------- launchers
template <class T, int DQK, int DV, bool CAUSAL, bool WIN, int NR, int NS, bool PAIR, int MINW>
static hipError_t launch_dq(BwdArgs a, hipStream_t st) {
  a.num_tiles = (a.Sq + 32 * NR - 1) / (32 * NR);
  const int64_t units = (int64_t)a.B * a.Hq * (PAIR ? (a.num_tiles + 1) / 2 : a.num_tiles);
  a.xcd_remap = PAIR && units % 8 == 0;
  hipLaunchKernelGGL((bwd_dq_kernel<T, DQK, DV, CAUSAL, WIN, NR, NS, PAIR, MINW>), dim3((unsigned)units),
                     dim3(64 * NR * NS), 0, st, a);
  return hipGetLastError();
}
template <class T, int DQK, int DV, bool CAUSAL, bool WIN, int NR, int NS, bool PAIR, int MINW, bool KVL = false>
static hipError_t launch_dkdv(BwdArgs a, hipStream_t st) {
  a.num_tiles = (a.Sk + 32 * NR - 1) / (32 * NR);
  const int64_t units = (int64_t)a.B * a.Hkv * (PAIR ? (a.num_tiles + 1) / 2 : a.num_tiles);
  a.xcd_remap = PAIR && units % 8 == 0;
  hipLaunchKernelGGL((bwd_dkdv_kernel<T, DQK, DV, CAUSAL, WIN, NR, NS, PAIR, MINW, KVL>), dim3((unsigned)units),
                     dim3(64 * NR * NS), 0, st, a);
  return hipGetLastError();
}

// Shapes per head size: eight-wave workgroups (two waves per SIMD) where the
// registers allow it; causal launches take the longest tiles first over all
// heads (measured at B2 H8 S2048 D64: 68.8 -> 67.4 us against complementary
// tile pairs).
template <class T, int DQK, int DV, bool CAUSAL, bool WIN>
static hipError_t launch_bwd(const BwdArgs& a, hipStream_t st) {
  hipError_t e;
  if constexpr (DQK <= 64) {
    if constexpr (CAUSAL) e = launch_dq<T, DQK, DV, CAUSAL, WIN, 2, 4, false, 2>(a, st);
    else e = launch_dq<T, DQK, DV, CAUSAL, WIN, 4, 2, false, 2>(a, st);
  } else if constexpr (DQK <= 128) {
    if constexpr (CAUSAL) e = launch_dq<T, DQK, DV, CAUSAL, WIN, 2, 4, false, 2>(a, st);
    else e = launch_dq<T, DQK, DV, CAUSAL, WIN, 4, 2, false, 2>(a, st);
  } else {
    e = launch_dq<T, DQK, DV, CAUSAL, WIN, 4, 1, false, 1>(a, st);
  }
  if (e != hipSuccess) return e;
  if constexpr (DQK <= 64) {
    if constexpr (CAUSAL) return launch_dkdv<T, DQK, DV, CAUSAL, WIN, 2, 4, false, 2>(a, st);
    else return launch_dkdv<T, DQK, DV, CAUSAL, WIN, 4, 2, false, 2>(a, st);
  } else if constexpr (DQK <= 128) {
    return launch_dkdv<T, DQK, DV, CAUSAL, WIN, 4, 2, false, 2, true>(a, st);
  } else {
    return launch_dkdv<T, DQK, DV, CAUSAL, WIN, 4, 1, false, 1>(a, st);
  }
}

template <class T, int DQK, int DV>
static hipError_t launch_bwd_c(const BwdArgs& a, hipStream_t st) {
  const bool win = a.wl < kNoWindow || a.wr < kNoWindow;
  if (win) return a.causal ? launch_bwd<T, DQK, DV, true, true>(a, st) : launch_bwd<T, DQK, DV, false, true>(a, st);
  return a.causal ? launch_bwd<T, DQK, DV, true, false>(a, st) : launch_bwd<T, DQK, DV, false, false>(a, st);
}

template <class T>
static hipError_t launch_bwd_t(const BwdArgs& a, int dqk, int dv, hipStream_t st) {
  if (dqk == 64 && dv == 64) return launch_bwd_c<T, 64, 64>(a, st);
  if (dqk == 128 && dv == 128) return launch_bwd_c<T, 128, 128>(a, st);
  if (dqk == 192 && dv == 128) return launch_bwd_c<T, 192, 128>(a, st);
  return hipErrorInvalidValue;
}

// zero a [B, S, H, D] 16-bit tensor with element strides (16 bytes per thread)
__global__ __launch_bounds__(256) void zero_rows_kernel(uint16_t* p, int64_t sb, int64_t ss, int64_t sh, int B,
                                                        int S, int H, int D) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int CH = D / 8;
  const int64_t total = (int64_t)B * S * H * CH;
  if (i >= total) return;
  const int ch = (int)(i % CH);
  const int64_t r = i / CH;
  const int h = (int)(r % H), s = (int)((r / H) % S), b = (int)(r / ((int64_t)H * S));
  stg16(p + (int64_t)b * sb + (int64_t)s * ss + (int64_t)h * sh + ch * 8, (u32x4){0u, 0u, 0u, 0u});
}

hipError_t run_zero_rows(void* data, int64_t sb, int64_t ss, int64_t sh, int B, int S, int H, int D,
                         hipStream_t st) {
  const int64_t total = (int64_t)B * S * H * (D / 8);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_rows_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st,
                     static_cast<uint16_t*>(data), sb, ss, sh, B, S, H, D);
  return hipGetLastError();
}

hipError_t run_attn_bwd(const BwdArgs& a, int dtype_bf16, int dqk, int dv, hipStream_t st) {
  if (a.B == 0 || a.Hq == 0) return hipSuccess;
  return dtype_bf16 ? launch_bwd_t<BF16>(a, dqk, dv, st) : launch_bwd_t<F16>(a, dqk, dv, st);
}

}  // namespace attn
