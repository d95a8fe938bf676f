// Tiled exact attention with an online softmax for gfx950 (prefill and
// chunked prefill over a KV cache).
//
// Method: exact attention softmax(scale * Q K^T + mask) V computed tile by tile
// with a running row max and row sum, so the score matrix never leaves
// registers (skill page "Flash Attention - Fast Memory-Efficient Attention":
// Quick start on IO-aware tiling; Workflow 1 Step 2 for the definition it
// must equal).
//
// Work decomposition.  A workgroup owns BM = NR * 32 * RB query rows of one
// (batch, q head) and is made of NS key-split groups of NR waves:
//  * every wave owns 32*RB query rows (RB MFMA row blocks) and keeps their Q
//    fragments in registers; the NS groups hold the same rows and walk
//    disjoint key tiles (tile t goes to group t % NS), which multiplies the
//    waves per CU on small problems; the groups' partial results are merged
//    exactly through LDS at the end;
//  * each group double-buffers its 64-key K/V tiles in LDS with direct
//    global->LDS loads (global_load_lds_dwordx4): the next tile streams in
//    while the current one is consumed, without staging registers.  Rows past
//    the key length are outside the tile's buffer resource and read as zero
//    (stale or NaN cache content is never read); their scores are masked;
//  * S^T = K Q^T on v_mfma_f32_32x32x16: one K fragment read from LDS feeds RB
//    MFMAs, and a lane owns one query row, so the row max needs one lane^32
//    exchange and the row sum none until the end;
//  * the K rows fed to the MFMA are permuted so each lane's 8-score groups
//    cover 8 consecutive keys; rounded to the input type those scores are
//    directly the B operand of O^T += V^T P^T, whose A operand V^T comes from
//    the row-major V tile through ds_read_b64_tr_b16;
//  * online softmax: P = exp2(s*c - m*c) with one FMA per score (c = scale *
//    log2 e); the running max used as reference is only raised when a row's
//    max exceeds it by more than 2^8, so the O rescale is rare and P stays
//    below 256; the row sum is accumulated from the packed P with v_dot2, so
//    numerator and denominator use the same rounded weights;
//  * causal and local windows: a unit walks only the key tiles its rows can
//    see, waves skip 32-key blocks outside their rows' band and mask only
//    blocks that cross a band edge;
//  * epilogue: O / l rounded to the output type, staged through LDS so each
//    lane stores 16 contiguous bytes of an output row.
#include <type_traits>

#include "device_common.hpp"
#include "attn_args.hpp"
#include "launchers.hpp"

namespace attn {

constexpr float kLazyRescale = 8.0f;  // log2 units: P may grow to 2^8 before a rescale

__device__ __forceinline__ int key_perm(int m) {
  int a = m >> 3, hh = (m >> 2) & 1, b = m & 3;
  return 16 * (a >> 1) + 8 * hh + 4 * (a & 1) + b;
}

constexpr int cmax(int a, int b) { return a > b ? a : b; }

// Query rows, key length and query-0 position of batch b (packed sequences,
// KV cache or plain), and the number of BN-key tiles that query tile qt of
// BM rows walks under the causal / window bounds.
struct UnitGeom {
  int Sqb, qst, kst, L, off;
};
__device__ __forceinline__ UnitGeom unit_geom(const AttnArgs& a, int b) {
  UnitGeom u;
  u.Sqb = a.Sq; u.qst = 0; u.kst = 0;
  if (a.varlen) {
    u.qst = a.cu_q[b];
    u.Sqb = a.cu_q[b + 1] - u.qst;
    u.kst = a.cu_k[b];
    u.L = a.cu_k[b + 1] - u.kst;
    u.off = u.L - u.Sqb;
  } else if (a.kvcache) {
    const int cb = a.seqlens ? a.seqlens[b] : a.seqlen_scalar;
    u.L = cb + a.Snew;
    u.off = cb;
  } else {
    u.L = a.Sk;
    u.off = a.Sk - a.Sq;
  }
  return u;
}
template <bool CAUSAL, bool WIN, int BM, int BN>
__device__ __forceinline__ int unit_tiles(const AttnArgs& a, const UnitGeom& u, int qt) {
  const int wrgt = WIN ? (CAUSAL ? min(a.wr, 0) : a.wr) : 0;
  const int q0 = qt * BM;
  if (q0 >= u.Sqb) return 0;
  const int rows_end = min(q0 + BM, u.Sqb);
  int kend = u.L, kbeg = 0;
  if (WIN || CAUSAL) kend = max(0, min(u.L, u.off + rows_end + wrgt));
  if (WIN) kbeg = min(kend, max(0, u.off + q0 - a.wl));
  return max(0, (kend + BN - 1) / BN - (WIN ? kbeg / BN : 0));
}

template <class T>
__device__ __forceinline__ uint32_t pack_p(float a, float b);
template <>
__device__ __forceinline__ uint32_t pack_p<F16>(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}
template <>
__device__ __forceinline__ uint32_t pack_p<BF16>(float a, float b) {
  return BF16::pack2(a, b);
}
template <class T>
__device__ __forceinline__ float dot2_sum(uint32_t p, float acc);
template <>
__device__ __forceinline__ float dot2_sum<F16>(uint32_t p, float acc) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, p), (f16x2){(_Float16)1.f, (_Float16)1.f},
                                acc, false);
}
template <>
__device__ __forceinline__ float dot2_sum<BF16>(uint32_t p, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p),
                                         (bf16x2){(__bf16)1.f, (__bf16)1.f}, acc, false);
}

// F8: q and k hold e4m3 codes (1 byte per element, strides in bytes) and S^T
// runs on the 32x32x64 fp8 MFMA; V, P and the output stay 16-bit (T).
template <class T, int DQK, int DV, bool CAUSAL, bool WIN, int RB, int NR, int NS, int BN, bool PAIR,
          bool FASTC, int MINW, bool F8, bool ROTQ>
__global__ __launch_bounds__(64 * NR * NS, MINW) void tile_attn_kernel(AttnArgs a) {
  constexpr int NKB = BN / 32;                           // 32-key MFMA blocks per tile
  constexpr int RW = 32 * RB;
  constexpr int BM = NR * RW;
  constexpr int EK = F8 ? 1 : 2;                         // bytes per q / k element
  constexpr int CK = DQK * EK / 16;                      // 16-byte chunks per K row
  constexpr int CV = DV / 8;
  constexpr int KSTEPS = DQK / 16;
  constexpr int K8 = DQK / 64;                           // fp8 MFMA steps of S
  static_assert(!F8 || DQK % 64 == 0, "fp8 head size");
  constexpr int DVB = (DV + 31) / 32;
  constexpr int KT = BN * DQK * EK / 2;                  // K tile, in 16-bit LDS words
  constexpr int VT = BN * DV;
  constexpr int STAGE = KT + VT;                          // elements
  constexpr int LDS_KV = NS * 2 * STAGE * 2;              // bytes
  constexpr int MERGE_O = (NS - 1) * NR * RB * DVB * 16 * 64;   // floats
  constexpr int MERGE_B = (MERGE_O + (NS - 1) * NR * RB * 2 * 64) * 4;
  constexpr int OSTR = DV + 8;
  constexpr int LDS_O = BM * OSTR * 2;
  constexpr int LDS_BYTES = cmax(LDS_KV, cmax(MERGE_B, LDS_O));
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_BYTES];
  uint16_t* lds16 = reinterpret_cast<uint16_t*>(smem);
  const uint32_t smem_addr = (uint32_t)reinterpret_cast<uintptr_t>((LDS_AS void*)smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int g = w / NR;          // key-split group
  const int rw = w - g * NR;     // row wave inside the group
  const int hh = lane >> 5;

  // ---- work unit
  const int nqt = a.num_qtiles;
  int b, hq, pu;
  if (!PAIR && a.lpt) {
    // Longest first across batches (per-batch lengths: KV caches, packed
    // sequences): every workgroup ranks the (batch, query tile) groups by
    // their key-tile count, computed from the device-side lengths, and takes
    // the group of its rank.  With Hq a multiple of 8 each XCD owns Hq/8
    // heads of every group (blockIdx % 8 is the XCD), so a head's K/V stay
    // in one L2.  The ranking needs B * nqt <= workgroup size (host-checked).
    const int ng = a.B * nqt;
    int* rk = reinterpret_cast<int*>(smem);
    if (tid < ng) rk[tid] = unit_tiles<CAUSAL, WIN, BM, BN>(a, unit_geom(a, tid / nqt), tid % nqt);
    __syncthreads();
    int rank, h;
    const int bid = blockIdx.x;
    if (a.xcd_remap) {
      const int hpx = a.Hq >> 3;
      const int j = bid >> 3;
      rank = j / hpx;
      h = (bid & 7) * hpx + (j - rank * hpx);
    } else {
      rank = bid / a.Hq;
      h = bid - rank * a.Hq;
    }
    int mine = 0;
    if (tid < ng) {
      const int wt = rk[tid];
      int r = 0;
      for (int j = 0; j < ng; ++j) {
        const int wj = rk[j];
        r += (wj > wt || (wj == wt && j < tid)) ? 1 : 0;
      }
      mine = (r == rank) ? tid + 1 : 0;
    }
    __syncthreads();
    if (mine) rk[0] = mine - 1;
    __syncthreads();
    const int gsel = min(max(rk[0], 0), ng - 1);   // (exactly one lane matched)
    __syncthreads();   // the first tile's DMA reuses this LDS
    b = gsel / nqt;
    hq = h;
    pu = gsel - b * nqt;   // the query tile itself (no heavy-first flip below)
  } else {
    int u = blockIdx.x;
    if (!PAIR && a.qmajor) {
      // causal, equal lengths: every head's last query tile first, then the
      // one before, ...  Workgroups are dispatched in index order as CUs free
      // up, so the long units start first and the short ones fill the tail.
      // (batch, head) is the fastest index: with B * Hq a multiple of 8 an XCD
      // keeps the same heads (blockIdx % 8) throughout.
      const int nbh = a.B * a.Hq;
      const int pq = u / nbh;
      u = (u - pq * nbh) * nqt + pq;
    } else if (a.xcd_remap) {
      const int per = gridDim.x >> 3;
      u = (u & 7) * per + (u >> 3);
    }
    // PAIR (causal): a unit is the query-tile pair (nqt-1-p, p), processed one
    // after the other, so every workgroup gets the same number of key tiles.
    const int nub = PAIR ? (nqt + 1) / 2 : nqt;   // units per (batch, head)
    const int bh = u / nub;
    pu = u - bh * nub;
    b = bh / a.Hq;
    hq = bh - b * a.Hq;
  }
  const int hkv = hq / a.group;
  const int nslots = (PAIR && nqt - 1 - pu != pu) ? 2 : 1;
  // packed variable-length batches: sequence b owns query rows [qst, qst + Sqb)
  // and key rows from kst on; the grid covers the longest query sequence
  const UnitGeom ug = unit_geom(a, b);
  const int Sqb = ug.Sqb, qst = ug.qst, kst = ug.kst, L = ug.L, off = ug.off;
  for (int slot = 0; slot < nslots; ++slot) {
  int qt = pu;
  // heavy tiles first; a pair at head size 64 takes its light tile first
  // (measured on the paired B2 H8 S2048 causal launch: 20.9 -> 20.4 us; at
  // 192/128 the light-first order is 4 % slower)
  if (CAUSAL && !a.lpt) qt = PAIR ? ((slot == 0) == (DQK <= 64) ? pu : nqt - 1 - pu) : nqt - 1 - pu;
  // key j is allowed for the query at position p iff p - wlft <= j <= p + wrgt
  // (causal caps wrgt at 0; without a window the bounds are compile-time
  // constants and the unbounded sides drop out)
  const int wrgt = WIN ? (CAUSAL ? min(a.wr, 0) : a.wr) : 0;
  const int wlft = WIN ? a.wl : 0;
  const int q0 = qt * BM;
  if (q0 >= Sqb) continue;   // a query tile past this sequence's end (uniform)
  const int rows_end = min(q0 + BM, Sqb);
  int kend = L, kbeg = 0;
  if (WIN || CAUSAL) kend = max(0, min(L, off + rows_end + wrgt));
  if (WIN) kbeg = min(kend, max(0, off + q0 - wlft));
  const int t_lo = WIN ? kbeg / BN : 0;              // first key tile of the unit
  const int ntiles = max(0, (kend + BN - 1) / BN - t_lo);
  const int nit = (ntiles + NS - 1) / NS;

  const int wr0 = q0 + rw * RW;
  const int wr1 = min(wr0 + RW, Sqb);
  const bool wave_active = wr0 < Sqb;
  const int pmin = off + wr0;
  const int pmax = off + wr1 - 1;
  int wkend = L, wkbeg = 0;
  if (WIN || CAUSAL) wkend = max(0, min(L, pmax + wrgt + 1));
  if (WIN) wkbeg = max(0, pmin - wlft);

  const uint16_t* qbase = a.q + (int64_t)b * a.q_sb + (int64_t)qst * a.q_ss + (int64_t)hq * a.q_sh;
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k) +
                         ((int64_t)b * a.k_sb + (int64_t)kst * a.k_ss + (int64_t)hkv * a.k_sh) * EK;
  const int64_t kss = a.k_ss * EK;                       // bytes between key rows
  const uint16_t* vbase = a.v + (int64_t)b * a.v_sb + (int64_t)kst * a.v_ss + (int64_t)hkv * a.v_sh;
  // F8: v holds e4m3 codes too (strides in bytes); each tile is loaded into
  // registers, converted exactly to the 16-bit type and written to the V stage
  const uint8_t* vbase8 = reinterpret_cast<const uint8_t*>(a.v) +
                          ((int64_t)b * a.v_sb + (int64_t)kst * a.v_ss + (int64_t)hkv * a.v_sh);

  // ---- tile DMA: tile t of this group into stage s.  Each lane's source row
  // and chunk inside a tile do not depend on the tile, so their byte offsets
  // are computed once.  A tile is read through a buffer resource that starts
  // at its first key row and ends after its last valid one: rows past the key
  // length read as zero (and are masked), without per-lane clamping.
  constexpr int NIK = NKB * CK / 2;                 // DMA instructions per K tile
  constexpr int NIV = NKB * CV / 2;
  constexpr int JK = (NIK + NR - 1) / NR;           // ... per wave
  constexpr int JV = (NIV + NR - 1) / NR;
  int koff_j[JK], voff_j[JV];
#pragma unroll
  for (int j = 0; j < JK; ++j) {
    const int P = (rw + j * NR) * 64 + lane;
    const int row = P / CK, pos = P % CK;
    koff_j[j] = row * kss + ((pos ^ swz_k<CK>(row)) << 4);
  }
#pragma unroll
  for (int j = 0; j < JV; ++j) {
    const int P = (rw + j * NR) * 64 + lane;
    const int row = P / CV, pos = P % CV;
    voff_j[j] = row * a.v_ss * 2 + ((pos ^ swz_vt<CV>(row)) << 4);
  }
  // F8 V: lane part of each 16-byte load (global byte offset inside the tile,
  // and the two LDS chunks its 16 converted elements land in)
  constexpr int JV8 = F8 ? (BN * DV) / (NR * 64 * 16) : 1;
  static_assert(!F8 || (BN * DV) % (NR * 64 * 16) == 0, "fp8 V tile split");
  int v8off[JV8], v8lds0[JV8], v8lds1[JV8];
  i32x4 v8raw[JV8];
#pragma unroll
  for (int j = 0; j < JV8; ++j) {
    const int P = (rw + j * NR) * 64 + lane;
    const int row = (P * 16) / DV, c0 = (P * 16) % DV;   // 16 elements: chunks c0/8 and c0/8 + 1
    v8off[j] = row * (int)a.v_ss + c0;
    v8lds0[j] = row * DV + (((c0 >> 3) ^ swz_vt<CV>(row)) << 3);
    v8lds1[j] = row * DV + ((((c0 >> 3) + 1) ^ swz_vt<CV>(row)) << 3);
  }
  auto issue = [&](int t, int s) {
    const uint32_t kd = smem_addr + (uint32_t)((g * 2 + s) * STAGE) * 2;
    const uint32_t vd = kd + KT * 2;
    const int key0 = t * BN;
    const int rows = min(BN, L - key0);
    const i32x4 rk = make_rsrc(kbase + (int64_t)key0 * kss, rows * kss);
#pragma unroll
    for (int j = 0; j < JK; ++j) {
      const int I = rw + j * NR;
      if (NIK % NR == 0 || I < NIK)
        dma_b128(rk, kd + I * 1024, koff_j[j]);
    }
    if constexpr (F8) {
      // rows past the key length read as zero (bounded resource), like the DMA
      const __amdgpu_buffer_rsrc_t rv8 = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(vbase8 + (int64_t)key0 * a.v_ss), (short)0, rows * (int)a.v_ss, 0x00020000);
#pragma unroll
      for (int j = 0; j < JV8; ++j) v8raw[j] = __builtin_amdgcn_raw_buffer_load_b128(rv8, v8off[j], 0, 0);
    } else {
      const i32x4 rv = make_rsrc(vbase + (int64_t)key0 * a.v_ss, rows * a.v_ss * 2);
#pragma unroll
      for (int j = 0; j < JV; ++j) {
        const int I = rw + j * NR;
        if (NIV % NR == 0 || I < NIV)
          dma_b128(rv, vd + I * 1024, voff_j[j]);
      }
    }
  };
  // F8: the e4m3 V tile loaded by the last issue() goes to stage s as 16-bit
  // values (the hardware pair conversion is exact for every code, NaN included)
  auto v8_store = [&](int s) {
    if constexpr (F8) {
      uint16_t* vdst = lds16 + (g * 2 + s) * STAGE + KT;
#pragma unroll
      for (int j = 0; j < JV8; ++j) {
        uint32_t cv[8];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t w = (uint32_t)v8raw[j][d];
          cv[2 * d] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
          cv[2 * d + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
        }
        *reinterpret_cast<u32x4*>(vdst + v8lds0[j]) = (u32x4){cv[0], cv[1], cv[2], cv[3]};
        *reinterpret_cast<u32x4*>(vdst + v8lds1[j]) = (u32x4){cv[4], cv[5], cv[6], cv[7]};
      }
    }
  };

  // ---- Q fragments (B operand of S^T = K Q^T); fp8: 32 bytes per lane and
  // 64 dims, the same dims as the lane's K fragment (any order works as long
  // as both operands use it)
  u32x4 qf[RB][F8 ? 1 : KSTEPS];
  i32x8 q8[RB][F8 ? K8 : 1];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int qrow = wr0 + rb * 32 + (lane & 31);
    const int qr = min(qrow, Sqb - 1);
    if constexpr (F8) {
      const uint8_t* qb = reinterpret_cast<const uint8_t*>(a.q) + (int64_t)b * a.q_sb + (int64_t)(qst + qr) * a.q_ss +
                          (int64_t)hq * a.q_sh;
#pragma unroll
      for (int s = 0; s < K8; ++s) {
        const u32x4 lo = ldg16(qb + 64 * s + 32 * hh), hi = ldg16(qb + 64 * s + 32 * hh + 16);
        q8[rb][s] = (i32x8){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                            (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
    } else if constexpr (ROTQ) {   // rotary embedding at the query's absolute position, as rope_apply rounds it
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s)
        qf[rb][s] = rope_chunk<T>(qbase + (int64_t)qr * a.q_ss, 16 * s + 8 * hh, a.rcos, a.rsin, (int64_t)off + qr,
                                  a.rd, a.rinter != 0, false);
    } else {
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) qf[rb][s] = ldg16(qbase + (int64_t)qr * a.q_ss + 16 * s + 8 * hh);
    }
  }

  f32x16 o[RB][DVB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int i = 0; i < DVB; ++i) o[rb][i] = (f32x16){};
  float m_use[RB], l_run[RB];   // m_use in log2 units (score * c)
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_use[rb] = -__builtin_inff();
    l_run[rb] = 0.f;
  }
  const float c = FASTC ? a.c : 1.f;
  const float cpre = a.c;   // general path: scores are multiplied by c first

  if (nit > 0 && g < ntiles) issue(t_lo + g, 0);

  const int grp = lane >> 4;
  const int tr_t = (lane & 15) >> 2;
  const int tr_q = lane & 3;

  // LDS read offsets (elements) that depend on the lane only; every other
  // part of a K or V fragment address is a compile-time constant, so the
  // reads use instruction offsets instead of per-read address arithmetic.
  //  * K (S^T = K Q^T): row key_perm(lane) of each 32-key block; the chunk
  //    swizzle depends on the row modulo 32 only.  When it flips fewer than
  //    4 chunk bits, chunk 2*st + hh sits at base[st % 4] + 8*(st / 4) chunks.
  //  * V (O^T += V^T P^T): rows 8*hh + tr_t (+4, +16 t2, +32 kb) share one
  //    swizzle value; column block i needs its own base.
  constexpr int NKO = (CK % 16 == 0) ? KSTEPS : (KSTEPS < 4 ? KSTEPS : 4);
  int koffl[NKO];
  {
    const int krow = key_perm(lane & 31);
    const int sw = swz_k<CK>(krow);
#pragma unroll
    for (int j = 0; j < NKO; ++j) koffl[j] = krow * DQK + (((2 * j + hh) ^ sw) << 3);
  }
  int voffl[DVB];
  {
    const int vrow = 8 * hh + tr_t;
    const int sv = swz_vt<CV>(vrow);
#pragma unroll
    for (int i = 0; i < DVB; ++i) {
      int col = i * 32 + 16 * (grp & 1) + 4 * tr_q;
      if (DV < 32 && (grp & 1)) col = 4 * tr_q;   // lanes past a 16-wide V read a valid spot and are zeroed
      voffl[i] = vrow * DV + (((col >> 3) ^ sv) << 3) + (col & 7);
    }
  }

  // One key tile per call; the loop makes two calls per trip so that each
  // call's LDS stage is a constant (its addresses become instruction offsets
  // of loop-invariant registers).
  auto iter = [&](const int it, auto SC) {
    constexpr int s = decltype(SC)::value;   // LDS stage of this iteration
    const int tr = it * NS + g;                  // tile index inside the unit
    const int t = t_lo + tr;
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this lane's DMA for stage s landed
    if (F8 && tr < ntiles) v8_store(s);   // (stage s has been free since the previous barrier)
    __syncthreads();                      // ... and every lane's; stage s^1 is free again
    if (it + 1 < nit && tr + NS < ntiles) issue(t + NS, s ^ 1);

    const int key0 = t * BN;
    if (tr >= ntiles || !wave_active || key0 >= wkend || (WIN && key0 + BN <= wkbeg)) return;
    const uint16_t* kt = lds16 + (g * 2 + s) * STAGE;
    const uint16_t* vt = kt + KT;

    // Wave priorities at head size >= 128 with one key group (the two waves
    // of a SIMD then come from different workgroups and drift freely): at
    // 192/128 the MFMA phases run at priority 2, at 128 the softmax at 3
    // (measured on four boxes: 192/128 S=4096 causal -2..-3 %, 128 S=4096
    // causal -3.5..-5 %; no gain or a loss at head size 64 and with two key
    // groups, so those stay at the default)
    constexpr bool PRIO = DQK >= 128 && NS == 1 && !F8;
    constexpr int PRIO_MFMA = DQK >= 192 ? 2 : 0, PRIO_SOFT = DQK >= 192 ? 0 : 3;
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(PRIO_MFMA);
    // ---- S^T = K Q^T for two 32-key blocks
    f32x16 sc[RB][NKB];
    bool blk_on[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) blk_on[kb] = key0 + kb * 32 < wkend && (!WIN || key0 + kb * 32 + 32 > wkbeg);
    // K fragment kb, k-step st of this stage (16 bytes per lane)
    auto kfrag = [&](int kb, int st) -> u32x4 {
      const int o = (CK % 16 == 0) ? koffl[st] : koffl[st % 4] + 64 * (st / 4);
      return *reinterpret_cast<const u32x4*>(kt + kb * 32 * DQK + o);
    };
    bool all_on = true;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) all_on = all_on && blk_on[kb];
    bool s_done = false;
    if constexpr (!F8) {
      if (all_on) {
        // every block is in the band (the common case): the blocks' MFMA
        // chains are independent and interleave
        // fragment f = (st, kb) in MFMA order, read SPD fragments ahead: each
        // read is issued before the MFMA SPD places earlier, so the LDS
        // latency overlaps the MFMA pipe instead of sitting before each MFMA
        // (the compiler alone read each fragment into one register right
        // before its MFMA at head size 192; measured: 192/128 S=4096 causal
        // 169 -> 166 us, chunked prefill 53.8 -> 52.3 us; 3 or 4 ahead no better)
        constexpr int NF = KSTEPS * NKB;
        constexpr int SPD = 2 < NF ? 2 : NF;
        u32x4 fr[SPD];
#pragma unroll
        for (int p = 0; p < SPD; ++p) fr[p] = kfrag(p % NKB, p / NKB);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const int st = f / NKB, kb = f % NKB;
          const u32x4 af = fr[f % SPD];
          if (f + SPD < NF) fr[f % SPD] = kfrag((f + SPD) % NKB, (f + SPD) / NKB);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            sc[rb][kb] = T::mfma32(af, qf[rb][st], st == 0 ? (f32x16){} : sc[rb][kb]);
        }
        s_done = true;
      }
    }
    if (!s_done)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      if (blk_on[kb]) {
        const int krow = kb * 32 + key_perm(lane & 31);
        const int sw = swz_k<CK>(krow);
        if constexpr (F8) {
          const uint8_t* kr = reinterpret_cast<const uint8_t*>(kt) + krow * DQK;
#pragma unroll
          for (int st = 0; st < K8; ++st) {
            const int c0 = 4 * st + 2 * hh;
            const u32x4 lo = *reinterpret_cast<const u32x4*>(kr + ((c0 ^ sw) << 4));
            const u32x4 hi = *reinterpret_cast<const u32x4*>(kr + (((c0 + 1) ^ sw) << 4));
            const i32x8 af = (i32x8){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                     (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
              sc[rb][kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  af, q8[rb][st], st == 0 ? (f32x16){} : sc[rb][kb], 0, 0, 0, 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int st = 0; st < KSTEPS; ++st) {
            const u32x4 af = kfrag(kb, st);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
              sc[rb][kb] = T::mfma32(af, qf[rb][st], st == 0 ? (f32x16){} : sc[rb][kb]);
          }
        }
      } else {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) sc[rb][kb] = (f32x16){};
      }
    }

    if constexpr (PRIO) __builtin_amdgcn_s_setprio(PRIO_SOFT);
    // ---- mask, row max, lazy rescale, P
    const bool need_mask = (key0 + BN > L) || ((WIN || CAUSAL) && key0 + BN - 1 > pmin + wrgt) ||
                           (WIN && key0 < pmax - wlft) || (WIN && !blk_on[0]) || !blk_on[NKB - 1];
    u32x4 pf[RB][NKB][2];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int qpos = off + wr0 + rb * 32 + (lane & 31);
      if (!FASTC) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sc[rb][kb][r] *= cpre;
      }
      if (need_mask) {
        asm volatile("" ::: "memory");   // keep this a branch: only edge tiles pay for masking
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + kb * 32 + 16 * (r >> 3) + 8 * hh + (r & 7);
            const bool ok = blk_on[kb] && key < L && (!(WIN || CAUSAL) || key <= qpos + wrgt) &&
                            (!WIN || key >= qpos - wlft);
            sc[rb][kb][r] = ok ? sc[rb][kb][r] : -__builtin_inff();
          }
      }
      float mx = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[rb][kb][r]);
      mx = xhalf_max(mx) * c;                   // log2 units
      const bool grow = mx > m_use[rb] + kLazyRescale;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        asm volatile("" ::: "memory");   // rare: keep the O rescale out of the common path
        const float alpha = grow ? fast_exp2(m_use[rb] - mx) : 1.f;
        if (grow) m_use[rb] = mx;
        l_run[rb] *= alpha;
#pragma unroll
        for (int i = 0; i < DVB; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[rb][i][r] *= alpha;
      }
      const float msub = (m_use[rb] == -__builtin_inff()) ? 0.f : m_use[rb];
      float lsum = l_run[rb];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) p[r] = fast_exp2(__builtin_fmaf(sc[rb][kb][r], c, -msub));
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          u32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[e] = pack_p<T>(p[8 * t2 + 2 * e], p[8 * t2 + 2 * e + 1]);
            lsum = dot2_sum<T>(v[e], lsum);
          }
          pf[rb][kb][t2] = v;
        }
      }
      l_run[rb] = lsum;
    }

    if constexpr (PRIO) __builtin_amdgcn_s_setprio(PRIO_MFMA);
    // ---- O^T += V^T P^T
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      if (!blk_on[kb]) continue;
      // V^T fragment f = (t2, i), read VPD fragments ahead of its MFMA
      // (one ahead: two were no better)
      constexpr int NM = 2 * DVB;
      constexpr int VPD = 1 < NM ? 1 : NM;
      auto vfrag = [&](int f) -> u32x4 {
        const int t2 = f / DVB, i = f % DVB;
        const uint16_t* vp = vt + (kb * 32 + 16 * t2) * DV + voffl[i];
        const u32x2 lo = lds_read_tr16(vp);
        const u32x2 hi = lds_read_tr16(vp + 4 * DV);
        u32x4 af = (u32x4){lo[0], lo[1], hi[0], hi[1]};
        if ((DV < 32) && (grp & 1)) af = (u32x4){0, 0, 0, 0};
        return af;
      };
      u32x4 vr[VPD];
#pragma unroll
      for (int p = 0; p < VPD; ++p) vr[p] = vfrag(p);
#pragma unroll
      for (int f = 0; f < NM; ++f) {
        const int t2 = f / DVB, i = f % DVB;
        const u32x4 af = vr[f % VPD];
        if (f + VPD < NM) vr[f % VPD] = vfrag(f + VPD);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) o[rb][i] = T::mfma32(af, pf[rb][kb][t2], o[rb][i]);
      }
    }
  };
  for (int it = 0; it < nit; it += 2) {
    iter(it, std::integral_constant<int, 0>{});
    if (it + 1 < nit) iter(it + 1, std::integral_constant<int, 1>{});
  }

  // ---- merge the key-split groups (exact log-sum-exp combination)
  __syncthreads();
  if constexpr (NS > 1) {
    float* mo = reinterpret_cast<float*>(smem);
    float* mml = mo + MERGE_O;
    if (g > 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int i = 0; i < DVB; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            mo[((((g - 1) * NR + rw) * RB + rb) * DVB * 16 + i * 16 + r) * 64 + lane] = o[rb][i][r];
        mml[((((g - 1) * NR + rw) * RB + rb) * 2 + 0) * 64 + lane] = m_use[rb];
        mml[((((g - 1) * NR + rw) * RB + rb) * 2 + 1) * 64 + lane] = l_run[rb];
      }
    }
    __syncthreads();
    if (g == 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        float M = m_use[rb];
        for (int gg = 1; gg < NS; ++gg)
          M = fmaxf(M, mml[((((gg - 1) * NR + rw) * RB + rb) * 2 + 0) * 64 + lane]);
        const float Ms = (M == -__builtin_inff()) ? 0.f : M;
        const float a0 = fast_exp2(m_use[rb] - Ms);
        float lt = l_run[rb] * a0;
#pragma unroll
        for (int i = 0; i < DVB; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[rb][i][r] *= a0;
        for (int gg = 1; gg < NS; ++gg) {
          const int base = ((gg - 1) * NR + rw) * RB + rb;
          const float ag = fast_exp2(mml[(base * 2 + 0) * 64 + lane] - Ms);
          lt += mml[(base * 2 + 1) * 64 + lane] * ag;
#pragma unroll
          for (int i = 0; i < DVB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[rb][i][r] += ag * mo[(base * DVB * 16 + i * 16 + r) * 64 + lane];
        }
        m_use[rb] = M;
        l_run[rb] = lt;
      }
    }
    __syncthreads();
  }

  // ---- epilogue (group 0): O / l -> output type -> LDS -> coalesced stores
  if (g == 0) {
    float lsum[RB], inv[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      lsum[rb] = xhalf_sum(l_run[rb]);
      inv[rb] = lsum[rb] > 0.f ? 1.f / lsum[rb] : 0.f;
      if constexpr (F8) inv[rb] *= a.oscale;
    }
    uint16_t* lds_o = lds16 + rw * RW * OSTR;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < DVB; ++i)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const int dv = i * 32 + 8 * a4 + 4 * hh;
          if (dv < DV) {
            const u32x2 pk = (u32x2){T::pack2(o[rb][i][4 * a4 + 0] * inv[rb], o[rb][i][4 * a4 + 1] * inv[rb]),
                                     T::pack2(o[rb][i][4 * a4 + 2] * inv[rb], o[rb][i][4 * a4 + 3] * inv[rb])};
            *reinterpret_cast<u32x2*>(lds_o + (rb * 32 + (lane & 31)) * OSTR + dv) = pk;
          }
        }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
    if (wave_active) {
      uint16_t* obase = a.out + (int64_t)b * a.o_sb + (int64_t)qst * a.o_ss + (int64_t)hq * a.o_sh;
      constexpr int OCH = RW * CV;
#pragma unroll
      for (int i = 0; i < (OCH + 63) / 64; ++i) {
        const int id = i * 64 + lane;
        const int row = id / CV, ch = id - (id / CV) * CV;
        if (id < OCH && wr0 + row < Sqb) {
          const u32x4 val = *reinterpret_cast<const u32x4*>(lds_o + row * OSTR + ch * 8);
          stg16(obase + (int64_t)(wr0 + row) * a.o_ss + ch * 8, val);
        }
      }
      if (a.lse && hh == 0) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const int qrow = wr0 + rb * 32 + lane;
          if (qrow < Sqb)
            a.lse[(int64_t)b * a.lse_sb + (int64_t)hq * a.lse_sh + qst + qrow] =
                lsum[rb] > 0.f ? (m_use[rb] + __log2f(lsum[rb])) * 0.69314718055994531f
                               : -__builtin_inff();
        }
      }
    }
  }
  __syncthreads();   // the staging tile is reused by the next slot
  }   // slot
}

// ---------------------------------------------------------------- launchers
template <class T, int DQK, int DV, bool CAUSAL, bool WIN, int RB, int NR, int NS, int BN, bool PAIR, int MINW,
          bool F8, bool ROTQ>
static hipError_t launch_cfg(const AttnArgs& a0, bool fastc, hipStream_t st) {
  AttnArgs a = a0;
  constexpr int BM = NR * 32 * RB;
  a.num_qtiles = (a.Sq + BM - 1) / BM;
  const int64_t units = (int64_t)a.B * a.Hq * (PAIR ? (a.num_qtiles + 1) / 2 : a.num_qtiles);
  if (units <= 0) return hipSuccess;
  // longest-first order across batches when their lengths differ (per-batch
  // cache lengths, packed sequences) and the ranking fits one workgroup
  a.lpt = (!PAIR && (a.varlen || (a.kvcache && a.seqlens)) &&
           (int64_t)a.B * a.num_qtiles <= 64 * NR * NS) ? 1 : 0;
  a.xcd_remap = a.lpt ? (a.Hq % 8 == 0 && units % 8 == 0) : (units % 8 == 0);
  const dim3 grid((unsigned)units), block(64 * NR * NS);
  if (fastc)
    hipLaunchKernelGGL((tile_attn_kernel<T, DQK, DV, CAUSAL, WIN, RB, NR, NS, BN, PAIR, true, MINW, F8, ROTQ>), grid,
                       block, 0, st, a);
  else
    hipLaunchKernelGGL((tile_attn_kernel<T, DQK, DV, CAUSAL, WIN, RB, NR, NS, BN, PAIR, false, MINW, F8, ROTQ>), grid,
                       block, 0, st, a);
  return hipGetLastError();
}

// Rows per workgroup and key splits per head dimension: small problems get
// key-split groups so that every CU runs several waves.
template <class T, int DQK, int DV, bool CAUSAL, bool WIN, bool F8 = false, bool ROTQ = false>
static hipError_t launch_dims(const AttnArgs& a, bool fastc, hipStream_t st) {
  const int64_t rows = (int64_t)a.B * a.Hq * a.Sq;
  if constexpr (DQK <= 16) {
    return launch_cfg<T, DQK, DV, CAUSAL, WIN, 1, 4, 1, 64, false, 2, F8, ROTQ>(a, fastc, st);
  } else if constexpr (DQK <= 64) {
    // causal, no window, at most 65536 rows: 64-row units of 32-key tiles.
    //  * equal lengths: no pairing, heaviest query tiles of every head first;
    //    two workgroups fit a CU (64 KB of LDS each), so a CU runs 16 waves
    //    and the dispatcher balances the tail (measured: B2 H8 S2048 causal
    //    20.1 -> 18.6 us against complementary tile pairs);
    //  * packed sequences size the grid by the longest one, so pairs would
    //    mostly meet tiles past a shorter sequence's end: longest first from
    //    the device-side lengths (7 packed sequences: 21.3 -> 19.6 us);
    //  * KV caches: complementary tile pairs (every workgroup the same work).
    // A causal band (window) gives every tile about the same work already,
    // and larger causal problems balance by dispatching the longest tiles
    // first (measured: window (256, 256) 14.4 -> 11.2 us, B4 H16 S8192 causal
    // 781 -> 700 us).
    if constexpr (CAUSAL && !WIN) {
      if (rows <= 256 * 256 && a.varlen)
        return launch_cfg<T, DQK, DV, CAUSAL, WIN, 1, 2, 4, 32, false, 2, F8, ROTQ>(a, fastc, st);
      if (rows <= 256 * 256 && !a.kvcache) {
        AttnArgs aq = a;
        aq.qmajor = 1;
        return launch_cfg<T, DQK, DV, CAUSAL, WIN, 1, 2, 4, 32, false, 2, F8, ROTQ>(aq, fastc, st);
      }
      if (rows <= 256 * 256)
        return launch_cfg<T, DQK, DV, CAUSAL, WIN, 1, 2, 4, 32, true, 2, F8, ROTQ>(a, fastc, st);
    }
    return launch_cfg<T, DQK, DV, CAUSAL, WIN, 1, 4, 2, 64, false, 2, F8, ROTQ>(a, fastc, st);
  } else {
    // one query block per wave keeps two waves per SIMD at these head sizes
    // (two row blocks per wave need ~300 VGPRs, one wave per SIMD: 1.9x slower
    // at B2 H16 S4096 D192/128 causal).
    // causal prefill without a window: complementary query-tile pairs, so that
    // every workgroup walks the same number of key tiles (measured at B2 H16
    // S4096 causal: D192/128 197 -> 169 us, D128 167 -> 142 us; the longest-
    // first order per (batch, head) left a tail of heavy tiles started late)
    // small head-128 problems also split the keys in two, so that a launch of
    // a few hundred workgroups still has two waves per SIMD (measured: D=128
    // B2 H8 S2048 49.8 -> 42.3 us, chunked prefill 66.4 -> 58.4 us)
    if (DQK <= 128 && rows <= 256 * 256)
      return launch_cfg<T, DQK, DV, CAUSAL, WIN, 1, 4, 2, 64, false, 2, F8, ROTQ>(a, fastc, st);
    if constexpr (CAUSAL && !WIN) {
      if (!a.varlen && !a.kvcache)
        return launch_cfg<T, DQK, DV, CAUSAL, WIN, 1, 4, 1, 64, true, 2, F8, ROTQ>(a, fastc, st);
    }
    return launch_cfg<T, DQK, DV, CAUSAL, WIN, 1, 4, 1, 64, false, 2, F8, ROTQ>(a, fastc, st);
  }
}

template <class T, int DQK, int DV, bool F8 = false, bool ROTQ = false>
static hipError_t launch_tile_c(const AttnArgs& a, bool causal, bool fastc, hipStream_t st) {
  const bool win = a.wl < kNoWindow || a.wr < kNoWindow;
  if (win)
    return causal ? launch_dims<T, DQK, DV, true, true, F8, ROTQ>(a, fastc, st)
                  : launch_dims<T, DQK, DV, false, true, F8, ROTQ>(a, fastc, st);
  return causal ? launch_dims<T, DQK, DV, true, false, F8, ROTQ>(a, fastc, st)
                : launch_dims<T, DQK, DV, false, false, F8, ROTQ>(a, fastc, st);
}

template <class T, bool ROTQ>
static hipError_t launch_tile_t(const AttnArgs& a, int dqk, int dv, bool causal, bool fastc, hipStream_t st) {
  if (dqk == 16 && dv == 16) return launch_tile_c<T, 16, 16, false, ROTQ>(a, causal, fastc, st);
  if (dqk == 64 && dv == 64) return launch_tile_c<T, 64, 64, false, ROTQ>(a, causal, fastc, st);
  if (dqk == 128 && dv == 128) return launch_tile_c<T, 128, 128, false, ROTQ>(a, causal, fastc, st);
  if (dqk == 192 && dv == 128) return launch_tile_c<T, 192, 128, false, ROTQ>(a, causal, fastc, st);
  return hipErrorInvalidValue;
}

hipError_t run_tile_attn(const AttnArgs& a, int dtype_bf16, int dqk, int dv, bool causal,
                         hipStream_t st) {
  const bool fastc = a.c > 0.f;
  if (a.rotq)
    return dtype_bf16 ? launch_tile_t<BF16, true>(a, dqk, dv, causal, fastc, st)
                      : launch_tile_t<F16, true>(a, dqk, dv, causal, fastc, st);
  return dtype_bf16 ? launch_tile_t<BF16, false>(a, dqk, dv, causal, fastc, st)
                    : launch_tile_t<F16, false>(a, dqk, dv, causal, fastc, st);
}

hipError_t run_tile_attn_fp8(const AttnArgs& a, int d, bool causal, hipStream_t st) {
  const bool fastc = a.c > 0.f;
  if (d == 64) return launch_tile_c<BF16, 64, 64, true>(a, causal, fastc, st);
  if (d == 128) return launch_tile_c<BF16, 128, 128, true>(a, causal, fastc, st);
  return hipErrorInvalidValue;
}

}  // namespace attn
