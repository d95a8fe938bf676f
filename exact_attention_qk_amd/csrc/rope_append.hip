// Rotary embedding and KV-cache append for gfx950.
//
// Rotation (ROCm/flash-attention PR #99 "Added Support for Rotary Positional
// Embeddings (both non-fused and fused kernel)", Motivation and rotary kernel
// argument review; flash-attention issue #1402, second script): a row at
// absolute position p has its first rd dims rotated pairwise by the angle whose
// cos/sin sit in row p of [seqlen_ro, rd/2] tables.  Pairs are (j, j + rd/2),
// or (2j, 2j+1) when interleaved; conjugate flips the sign of sin.  Each output
// is x1*c - x2*s (resp. x1*s + x2*c) evaluated in fp32 -- both products of
// 16-bit inputs are exact in fp32, so the result is the exact value rounded
// once -- and then rounded to the storage type (round to nearest even).
//
// Vector path (rd a multiple of 16, 16-byte aligned tables): a lane owns 8
// consecutive elements (16 bytes) of a row and a wave holds 64 / (D/8) rows.
// Interleaved pairs lie inside a lane's chunk; for the half-split layout a
// lane also reads its partner chunk (rd/2 elements away) before any lane of
// the row stores, so rotating in place is safe.  Other rotary widths use one
// wave per row, a lane owning whole pairs.
// The KV-cache append runs three row sets in one launch (blockIdx.y):
// new keys (rotated, written to cache rows c_b + i), new values (copied to
// cache rows c_b + i) and, with rotary tables, the queries (rotated into a
// workspace copy that the attention kernels read).
#include "device_common.hpp"
#include "attn_args.hpp"
#include "launchers.hpp"

namespace attn {

template <class T>
__device__ __forceinline__ void process_row(const RowSet& rs, int row, int lane) {
  const RopeArgs& a = rs.t;
  const int h = row % a.H;
  const int bs = row / a.H;
  const int s = bs % a.S;
  const int b = bs / a.S;
  const int off = a.offsets ? a.offsets[b] : a.offset_scalar;
  const int ds = rs.dst_at_offset ? off + s : s;
  const uint16_t* x = a.x + (int64_t)b * a.x_sb + (int64_t)s * a.x_ss + (int64_t)h * a.x_sh;
  uint16_t* y = a.y + (int64_t)b * a.y_sb + (int64_t)ds * a.y_ss + (int64_t)h * a.y_sh;
  if (a.copy_only || a.rd == 0) {
    for (int d = lane * 8; d < a.D; d += 512) stg16(y + d, ldg16(x + d));
    return;
  }
  const int half = a.rd >> 1;
  const int64_t pos = off + s;
  const uint16_t* cr = a.cos + pos * half;
  const uint16_t* sr = a.sin + pos * half;
  for (int p = lane; p < half; p += 64) {
    const int i1 = a.interleaved ? 2 * p : p;
    const int i2 = a.interleaved ? 2 * p + 1 : p + half;
    const float x1 = T::to_f32(x[i1]), x2 = T::to_f32(x[i2]);
    const float c = T::to_f32(cr[p]);
    float sn = T::to_f32(sr[p]);
    if (a.conjugate) sn = -sn;
    float y1 = x1 * c - x2 * sn;
    float y2 = x1 * sn + x2 * c;
    // Keep the fp32 rounding: without this barrier the compiler may fuse the
    // fma and the fp16 conversion into v_fma_mixlo_f16, which rounds the exact
    // value once to fp16 instead of first to fp32.
    asm volatile("" : "+v"(y1), "+v"(y2));
    y[i1] = T::from_f32(y1);
    y[i2] = T::from_f32(y2);
  }
  for (int d = a.rd + lane; d < a.D; d += 64) y[d] = x[d];
}

template <class T>
__global__ __launch_bounds__(256) void rope_vec_kernel(RowSet s0, RowSet s1, RowSet s2) {
  const RowSet& rs = blockIdx.y == 0 ? s0 : (blockIdx.y == 1 ? s1 : s2);
  const RopeArgs& a = rs.t;
  const int lpr = a.D >> 3;                 // lanes per row
  const int rpw = 64 / lpr;                 // rows per wave
  const int lane = threadIdx.x & 63;
  const int sub = lane / lpr;
  const int c = lane - sub * lpr;           // 16-byte chunk of the row
  if (sub >= rpw) return;
  const int row = (blockIdx.x * 4 + (threadIdx.x >> 6)) * rpw + sub;
  const int total = a.B * a.S * a.H;
  if (row >= total) return;
  const int h = row % a.H;
  const int bs = row / a.H;
  const int s = bs % a.S;
  const int b = bs / a.S;
  const int off = a.offsets ? a.offsets[b] : a.offset_scalar;
  const int ds = rs.dst_at_offset ? off + s : s;
  const uint16_t* x = a.x + (int64_t)b * a.x_sb + (int64_t)s * a.x_ss + (int64_t)h * a.x_sh;
  uint16_t* y = a.y + (int64_t)b * a.y_sb + (int64_t)ds * a.y_ss + (int64_t)h * a.y_sh;
  const int d0 = c * 8;
  const int rd = a.copy_only ? 0 : a.rd;
  stg16(y + d0, rope_chunk<T>(x, d0, a.cos, a.sin, (int64_t)off + s, rd, a.interleaved, a.conjugate));
}

template <class T>
__global__ __launch_bounds__(256) void rope_rows_kernel(RowSet s0, RowSet s1, RowSet s2) {
  const RowSet& rs = blockIdx.y == 0 ? s0 : (blockIdx.y == 1 ? s1 : s2);
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int total = rs.t.B * rs.t.S * rs.t.H;
  if (row >= total) return;
  process_row<T>(rs, row, threadIdx.x & 63);
}

static bool vec_ok(const RowSet& r) {
  const RopeArgs& a = r.t;
  if (a.D % 8 != 0 || a.D > 512) return false;
  if (a.copy_only || a.rd == 0) return true;
  if (a.rd % 16 != 0) return false;
  return (reinterpret_cast<uintptr_t>(a.cos) % 16 == 0) && (reinterpret_cast<uintptr_t>(a.sin) % 16 == 0);
}

hipError_t run_rope_rows(const RowSet* sets, int nsets, int dtype_bf16, hipStream_t st) {
  if (nsets <= 0) return hipSuccess;
  RowSet s[3] = {sets[0], nsets > 1 ? sets[1] : sets[0], nsets > 2 ? sets[2] : sets[0]};
  int64_t maxrows = 0;
  bool vec = true;
  int64_t vec_blocks = 0;
  for (int i = 0; i < nsets; ++i) {
    const int64_t n = (int64_t)sets[i].t.B * sets[i].t.S * sets[i].t.H;
    if (n > maxrows) maxrows = n;
    vec = vec && vec_ok(sets[i]);
    if (vec) {
      const int rpw = 64 / (sets[i].t.D / 8);
      const int64_t blocks = (n + 4 * rpw - 1) / (4 * rpw);
      if (blocks > vec_blocks) vec_blocks = blocks;
    }
  }
  if (maxrows == 0) return hipSuccess;
  if (vec) {
    const dim3 grid((unsigned)vec_blocks, (unsigned)nsets);
    if (dtype_bf16)
      hipLaunchKernelGGL(rope_vec_kernel<BF16>, grid, dim3(256), 0, st, s[0], s[1], s[2]);
    else
      hipLaunchKernelGGL(rope_vec_kernel<F16>, grid, dim3(256), 0, st, s[0], s[1], s[2]);
    return hipGetLastError();
  }
  dim3 grid((unsigned)((maxrows + 3) / 4), (unsigned)nsets);
  if (dtype_bf16)
    hipLaunchKernelGGL(rope_rows_kernel<BF16>, grid, dim3(256), 0, st, s[0], s[1], s[2]);
  else
    hipLaunchKernelGGL(rope_rows_kernel<F16>, grid, dim3(256), 0, st, s[0], s[1], s[2]);
  return hipGetLastError();
}

}  // namespace attn
