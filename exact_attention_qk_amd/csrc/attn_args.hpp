// Kernel argument block shared by the attention kernels and the host dispatcher.
#pragma once
#include <stdint.h>

namespace attn {

constexpr int kNoWindow = 1 << 29;   // window side without a limit (positions stay far below)

struct AttnArgs {
  const uint16_t* q;  int64_t q_sb, q_ss, q_sh;
  const uint16_t* k;  int64_t k_sb, k_ss, k_sh;
  const uint16_t* v;  int64_t v_sb, v_ss, v_sh;
  uint16_t* out;      int64_t o_sb, o_ss, o_sh;
  float* lse;                 // [B, Hq, Sq] or null; element (b, h, i) at b*lse_sb + h*lse_sh + i
  int64_t lse_sb, lse_sh;     // (packed sequences: 0 and total_q, i counted over the whole pack)
  int varlen;                 // 1: packed sequences, bounds from cu_q / cu_k (device [B+1])
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* seqlens;     // per-batch cache_seqlens (kvcache mode) or null
  int seqlen_scalar;          // cache_seqlens for every batch when seqlens is null
  int B, Sq, Sk, Hq, Hkv, group, Snew;
  int kvcache;                // 1: key length c_b + Snew, query i at c_b + i
                              // 0: key length Sk, query i at i + Sk - Sq
  int causal;                 // key j allowed for query i iff j <= position(i)
  int wl, wr;                 // local window: key j allowed iff pos - wl <= j <= pos + wr
                              // (kNoWindow when a side is unbounded)
  int num_qtiles;             // tiled kernel: ceil(Sq / rows per workgroup)
  int xcd_remap;              // tiled kernel: 1 when the grid is a multiple of 8
  int lpt;                    // tiled kernel: longest-first unit order from the device-side lengths
  int qmajor;                 // tiled kernel, causal: units ordered by query tile, last (heaviest) first
  float c;                    // softmax_scale * log2(e)
  float oscale;               // FP8 inputs: the descale of v, applied to the output
  // split-KV decode
  int split_len, num_splits;   // split length (the smallest one when split_auto), splits per batch at most
  int split_auto;             // 0, or the number of (kv head, split) waves the kernels size splits for
  int split_slots;            // splits of all batches together that the workspace holds
  float* ws_o;                // [split_slots, Hkv, R, Dv] fp32 partial numerators, a batch's splits adjacent
  float* ws_ml;               // [split_slots, Hkv, R, 2]  running max (log2 units), sum
  // decode with the append and the rotary embedding done in the same kernel
  int fused;                  // 1: keys >= c_b come from kn/vn (rotated) and are written to the cache
  const uint16_t* kn; int64_t kn_sb, kn_ss, kn_sh;
  const uint16_t* vn; int64_t vn_sb, vn_ss, vn_sh;
  const uint16_t* rcos; const uint16_t* rsin;   // [*, rd/2] tables, rows 16-byte aligned
  int rd, rinter;             // rotary width (0: none, else a multiple of 16), interleaved pairs
  int rotq;                   // tiled kernel: rotate q as it is loaded (rd, rcos, rsin, rinter above)
};

// Gradients of attention (dQ, dK, dV) for a given dO.
struct BwdArgs {
  const uint16_t* q;  int64_t q_sb, q_ss, q_sh;
  const uint16_t* k;  int64_t k_sb, k_ss, k_sh;
  const uint16_t* v;  int64_t v_sb, v_ss, v_sh;
  const uint16_t* o;  int64_t o_sb, o_ss, o_sh;
  const uint16_t* dout; int64_t do_sb, do_ss, do_sh;
  uint16_t* dq;       int64_t dq_sb, dq_ss, dq_sh;
  uint16_t* dk;       int64_t dk_sb, dk_ss, dk_sh;
  uint16_t* dv;       int64_t dv_sb, dv_ss, dv_sh;
  const float* lse;   // [B, Hq, Sq] from the forward pass (natural log)
  float* ld;          // workspace [B, Hq, Sq, 2]: lse * log2(e), rowsum(dO * O)
  int B, Sq, Sk, Hq, Hkv, group;
  int causal, wl, wr; // masks as in AttnArgs (wl, wr = kNoWindow when unbounded)
  float c;            // softmax_scale * log2(e)
  float scale;        // softmax_scale
  int num_tiles;      // row tiles (dQ kernel) or key tiles (dK/dV kernel) per (batch, head)
  int xcd_remap;
};

struct RopeArgs {
  const uint16_t* x;  int64_t x_sb, x_ss, x_sh;
  uint16_t* y;        int64_t y_sb, y_ss, y_sh;
  int B, S, H, D;
  const uint16_t* cos; const uint16_t* sin;
  int rd, interleaved, conjugate;
  const int32_t* offsets; int offset_scalar;
  int copy_only;              // 1: plain row copy (v rows of the cache append)
};

struct RowSet {
  RopeArgs t;
  int dst_at_offset;          // 1: destination row index = off_b + s, else s
};

}  // namespace attn
