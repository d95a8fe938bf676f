/*
 * attn.h -- C ABI of the MI355X (gfx950) exact-attention library (libattn.so).
 *
 * The operations, named after the functions the pages discuss:
 *
 *   attn_fwd          exact attention softmax(scale * Q K^T + mask) V computed
 *                     tile by tile with an online softmax, so the score matrix
 *                     never reaches HBM.  The plain definition is the "standard
 *                     attention" of the skill page "Flash Attention - Fast
 *                     Memory-Efficient Attention" (Workflow 1, Step 2); the
 *                     flash_attn_func call of that page (Quick start; Workflow 2
 *                     Step 2) fixes the [batch, seqlen, heads, head_dim] layout,
 *                     the causal flag, the automatic scale and (Workflow 2 Step 3)
 *                     fewer K/V heads than q heads.  head_dim of q/k may differ
 *                     from head_dim of v (flash-attention PR #1604 "Support
 *                     hdimQK != hdimV backward", PR body: d=192 with d_v=128).
 *
 *   attn_fwd_kvcache  the decode-time variant flash_attn_with_kvcache
 *                     (flash-attention issue #1402 "is flash_attn_with_kvcache()
 *                     supposed to work for seqlen > 1 ?", both scripts): append
 *                     k_new/v_new into a preallocated cache at per-batch
 *                     cache_seqlens (an int for all batches or an int32 tensor
 *                     with one value per batch: ROCm/flash-attention PR #99
 *                     "Added Support for Rotary Positional Embeddings (both
 *                     non-fused and fused kernel)", rotary kernel argument
 *                     review), optionally rotating q and k_new (RoPE) with
 *                     cos/sin tables offset by the cache position, then attend
 *                     q over the cache prefix.
 *
 *   rope_apply        the same rotation as a standalone (non-fused) operation
 *                     (PR #99 title: fused and non-fused rotary), with the
 *                     conjugate (inverse-angle) flag named in that PR's review.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors are described by attn_tensor4: a device pointer to element
 *   [0,0,0,0] and element strides of the first three dims of a logical
 *   [batch, seqlen, heads, head_dim] tensor; head_dim is contiguous (stride 1).
 *   Strided views (e.g. the .transpose(1, 2) views of issue #1402) are fine.
 *   Every data pointer must be 16-byte aligned and every stride a multiple of
 *   8 elements (16 bytes), so rows can be moved with 16-byte accesses.  The
 *   sequence stride must be below 2^24 elements (tiles of up to 64 rows are
 *   addressed with 32-bit byte offsets); a larger one is ATTN_E_UNSUPPORTED.
 * - Ownership: the caller owns every buffer.  The library allocates no device
 *   or host memory on any call (the ATTN_CHECK=1 debug mode aside, which
 *   copies lengths to host vectors); the KV-cache, backward and FP8 paths use
 *   a caller-provided workspace sized by the matching *_workspace_size().
 * - Read-only inputs (q, k, v, k_new, v_new, cos/sin, cache_seqlens) may alias
 *   one another (issue #1402 passes one tensor as q, k and v).  out, lse, the
 *   caches and the workspace must not alias any other argument.
 * - Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL is the null
 *   stream) and the call returns without waiting.
 * - Errors: a non-zero return means nothing was enqueued (except
 *   ATTN_E_HIP, a failed launch); attn_last_error() returns a thread-local
 *   message describing the last failure of the calling thread.
 * - Supported: dtype fp16 or bf16 (outputs in the input dtype, accumulation
 *   in fp32); (Dqk, Dv) in {(16,16), (64,64), (128,128), (192,128)};
 *   Hq a multiple of Hkv (q head h reads kv head h / (Hq/Hkv)).  attn_fwd_fp8
 *   takes e4m3 inputs instead (its own section below).
 * - softmax_scale: a NaN value selects 1/sqrt(Dqk); any other value,
 *   zero included, is used as given.
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum attn_dtype { ATTN_DTYPE_F16 = 0, ATTN_DTYPE_BF16 = 1 } attn_dtype;

enum {
  ATTN_OK = 0,
  ATTN_E_NULL = -1,        /* a required pointer is NULL                        */
  ATTN_E_SHAPE = -2,       /* inconsistent or non-positive sizes                */
  ATTN_E_UNSUPPORTED = -3, /* valid but not implemented (head dims, dtype)      */
  ATTN_E_ALIGN = -4,       /* pointer not 16-byte aligned / stride not x8       */
  ATTN_E_WORKSPACE = -5,   /* workspace missing or smaller than required        */
  ATTN_E_OVERFLOW = -6,    /* scalar cache_seqlens + Snew exceeds the capacity  */
  ATTN_E_HIP = -7          /* a HIP launch failed                               */
};

typedef struct attn_tensor4 {
  void* data;        /* device pointer to element [0,0,0,0]                 */
  int64_t stride_b;  /* elements between consecutive batch entries          */
  int64_t stride_s;  /* elements between consecutive sequence positions     */
  int64_t stride_h;  /* elements between consecutive heads                  */
} attn_tensor4;

/* ---------------------------------------------------------------- attn_fwd
 * q   [B, Sq, Hq,  Dqk]   read
 * k   [B, Sk, Hkv, Dqk]   read
 * v   [B, Sk, Hkv, Dv ]   read
 * out [B, Sq, Hq,  Dv ]   written
 * lse [B, Hq, Sq] fp32, contiguous, written when non-NULL: natural-log
 *     sum of exp(scale * q.k) over the allowed keys (-inf for a row with none).
 * causal: key j is allowed for query i iff j <= i + Sk - Sq (bottom-right
 *     alignment, i.e. j <= i when Sq == Sk); a row with no allowed key
 *     produces zeros.
 * window_left, window_right: local (sliding-window) attention, the
 *     window_size=(left, right) of the skill page "Flash Attention - Fast
 *     Memory-Efficient Attention" (Workflow 2, Step 3).  With query i at
 *     position p = i + Sk - Sq, key j is allowed only if p - window_left <=
 *     j <= p + window_right; -1 leaves that side unbounded (-1, -1 = no
 *     window).  Combined with causal by intersection.  Values < -1 are
 *     rejected (ATTN_E_SHAPE).
 */
typedef struct attn_fwd_params {
  attn_dtype dtype;
  int B, Sq, Sk, Hq, Hkv, Dqk, Dv;
  attn_tensor4 q, k, v, out;
  float* lse;
  int causal;
  float softmax_scale;
  int window_left, window_right;
} attn_fwd_params;

int attn_fwd(const attn_fwd_params* p, void* stream);

/* --------------------------------------------------------- attn_fwd_varlen
 * Packed variable-length sequences (the variable-length mode that
 * ROCm/flash-attention PR #99 "Added Support for Rotary Positional Embeddings
 * (both non-fused and fused kernel)" names for its rotary kernel, review
 * thread on IS_VARLEN; decode keeps the batched layout).  Sequence b owns
 * query rows [cu_seqlens_q[b], cu_seqlens_q[b+1]) of q and key rows
 * [cu_seqlens_k[b], cu_seqlens_k[b+1]) of k and v, and is attended exactly
 * like one batch element of attn_fwd (same causal alignment, window and
 * empty-row rules, positions counted inside the sequence).
 * q   [total_q, Hq,  Dqk]   read     (attn_tensor4 with stride_b ignored)
 * k   [total_k, Hkv, Dqk]   read
 * v   [total_k, Hkv, Dv ]   read
 * out [total_q, Hq,  Dv ]   written
 * lse [Hq, total_q] fp32, contiguous, written when non-NULL.
 * cu_seqlens_q, cu_seqlens_k: device int32 [B + 1], non-decreasing, starting
 * at 0 and ending at total_q / total_k.  max_seqlen_q >= every query length
 * (it sizes the grid).  These device-side preconditions are not checked
 * unless ATTN_CHECK=1 is set (the call then copies both arrays to the host).
 */
typedef struct attn_varlen_params {
  attn_dtype dtype;
  int B, total_q, total_k, max_seqlen_q, Hq, Hkv, Dqk, Dv;
  attn_tensor4 q, k, v, out;
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
  float* lse;
  int causal;
  float softmax_scale;
  int window_left, window_right;
} attn_varlen_params;

int attn_fwd_varlen(const attn_varlen_params* p, void* stream);

/* -------------------------------------------------------- attn_fwd_kvcache
 * q       [B, Sq, Hq, Dqk]            read
 * k_cache [B, capacity, Hkv, Dqk]     read; rows [c_b, c_b + Snew) written
 * v_cache [B, capacity, Hkv, Dv]      read; rows [c_b, c_b + Snew) written
 * k_new   [B, Snew, Hkv, Dqk]         read (data NULL iff Snew == 0)
 * v_new   [B, Snew, Hkv, Dv]          read (data NULL iff Snew == 0)
 * out     [B, Sq, Hq, Dv]             written
 * lse     [B, Hq, Sq] fp32 contiguous written when non-NULL
 *
 * c_b = cache_seqlens[b] (device int32 [B]) when cache_seqlens is non-NULL,
 * else cache_seqlens_scalar for every batch.  Snew is 0 or Sq.  Query token i
 * of batch b sits at absolute position c_b + i; with causal set it attends
 * keys j <= c_b + i, otherwise all keys j < c_b + Snew.  Cache rows at or
 * past c_b + Snew are never read, so their content (NaN included) does not
 * matter, and rows outside [c_b, c_b + Snew) are never written.
 *
 * Rotary embedding (when rotary_cos and rotary_sin are non-NULL): tables
 * [seqlen_ro, rotary_dim/2] in the working dtype, contiguous.  q and k_new
 * (never v, never the existing cache) are rotated at their absolute
 * positions; dims >= rotary_dim pass through.  Pairs are (j, j + rd/2), or
 * (2j, 2j+1) when rotary_interleaved.  Each rotated value is
 * x1*cos - x2*sin (resp. x1*sin + x2*cos) rounded once to fp32 and then to
 * the dtype (round-to-nearest-even); the cache receives exactly that value.
 *
 * Device-side preconditions (not checked unless the environment variable
 * ATTN_CHECK=1 is set, which makes the call copy cache_seqlens to the host
 * and validate them synchronously): 0 <= c_b <= capacity - Snew and, with
 * rotary tables, c_b + max(Sq, Snew) <= seqlen_ro.
 *
 * workspace: device memory of at least attn_fwd_kvcache_workspace_size(p)
 * bytes, 256-byte aligned (NULL allowed when that size is 0); its content on
 * entry is irrelevant.  Calls that may overlap in time must not share a
 * workspace.  num_splits: 0 lets the single-token decode path size its splits
 * from the device-side cache lengths (at least 32 keys each, about 1408
 * (kv head, split) pairs in all, so its workspace does not grow with the
 * capacity); a positive value forces the count per batch.
 *
 * On the single-token decode path (at most 16 query rows per kv head) the
 * rotary embedding (when rotary_dim is a multiple of 16 and the tables are
 * 16-byte aligned) and the append run inside the attention kernel; otherwise
 * a separate append/rotation pass runs first.
 */
typedef struct attn_kvcache_params {
  attn_dtype dtype;
  int B, Sq, Hq, Hkv, Dqk, Dv, capacity, Snew;
  attn_tensor4 q, k_cache, v_cache, k_new, v_new, out;
  int cache_seqlens_scalar;
  const int32_t* cache_seqlens;
  const void* rotary_cos;
  const void* rotary_sin;
  int rotary_dim, seqlen_ro, rotary_interleaved;
  int causal;
  float softmax_scale;
  float* lse;
  void* workspace;
  size_t workspace_bytes;
  int num_splits;
  int window_left, window_right;   /* as in attn_fwd_params, on absolute positions */
} attn_kvcache_params;

size_t attn_fwd_kvcache_workspace_size(const attn_kvcache_params* p);
int attn_fwd_kvcache(const attn_kvcache_params* p, void* stream);

/* ------------------------------------------------ attn_fwd_kvcache_noalloc
 * For callers that cannot allocate device memory at call time (work under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * attn_fwd_kvcache with the same arguments, results and errors, except that
 * p->workspace and p->workspace_bytes are ignored.  The workspace comes from
 * a device array inside the library instead, 16 MiB per GPU, which each GPU
 * the library runs on holds from its first use until the process ends; its
 * address is looked up once per device on the first call there.  A call
 * whose attn_fwd_kvcache_workspace_size() exceeds 16 MiB returns
 * ATTN_E_WORKSPACE before anything is enqueued (the single-token decode of
 * B=8, Hq=32, Hkv=8, D=128 with automatic splits needs 2.9 MiB whatever the
 * capacity).  The call allocates
 * nothing: no hipMalloc/hipFree, no host allocation.  Nothing in the array has
 * to start at zero: every byte a call reads was written earlier in that call.
 * Every call on one GPU shares its array, so calls that may overlap on one
 * GPU (different streams, or host threads without ordering between them)
 * race: order them on one stream.
 */
int attn_fwd_kvcache_noalloc(const attn_kvcache_params* p, void* stream);

/* ------------------------------------------------------------- attn_fwd_fp8
 * attn_fwd on FP8 inputs: the skill page "Flash Attention - Fast
 * Memory-Efficient Attention", Workflow 3 (H100 FP8 optimization with
 * FlashAttention-3) converts q, k and v to FP8 and runs attention on them.
 * q, k, v hold e4m3 codes in the "fn" form (1 sign, 4 exponent bits with bias
 * 7, 3 mantissa bits, no infinities, S.1111.111 = NaN); element x stands for
 * decode(x) * descale_q (resp. descale_k, descale_v).  The result is attn_fwd
 * of those values: out = softmax(scale * Q K^T + mask) V.
 * q   [B, Sq, Hq,  D]  1-byte elements, read
 * k   [B, Sk, Hkv, D]  1-byte elements, read
 * v   [B, Sk, Hkv, D]  1-byte elements, read
 *     (strides in elements = bytes, multiples of 16; pointers 16-byte aligned)
 * out [B, Sq, Hq,  D]  bf16, written (strides multiples of 8 elements)
 * lse [B, Hq, Sq] fp32 or NULL: as attn_fwd, of the descaled scores.
 * D in {64, 128}.  causal, softmax_scale (NaN = 1/sqrt(D)) and the window
 * as in attn_fwd.  descale_*: finite (ATTN_E_SHAPE otherwise).
 * Arithmetic: Q K^T on the fp8 matrix cores with fp32 accumulation (exact
 * products); each v tile is converted to bf16 (exactly) as the kernel stages
 * it in LDS; the weights P are rounded to bf16 for the P V product, whose
 * sums are fp32.
 * workspace: attn_fwd_fp8_workspace_size(p) bytes (0: the call needs none;
 *     workspace may be NULL).  Kept so callers that size one keep working.
 */
typedef struct attn_fp8_params {
  int B, Sq, Sk, Hq, Hkv, D;
  attn_tensor4 q, k, v, out;
  float* lse;
  int causal;
  float softmax_scale;
  float descale_q, descale_k, descale_v;
  int window_left, window_right;
  void* workspace;
  size_t workspace_bytes;
} attn_fp8_params;

size_t attn_fwd_fp8_workspace_size(const attn_fp8_params* p);
int attn_fwd_fp8(const attn_fp8_params* p, void* stream);

/* ----------------------------------------------------------------- attn_bwd
 * Gradients of attn_fwd (flash-attention PR #1604 "Support hdimQK != hdimV
 * backward": dQ, dK, dV with head_dim_qk != head_dim_v).  For the forward
 * call with the same q, k, v, causal, softmax_scale and window, and an
 * upstream gradient dout of the output:
 *   P = softmax(scale * q k^T + mask), dv = P^T dout, dP = dout v^T,
 *   dS = P * (dP - rowsum(dout * out)), dq = scale * dS k, dk = scale * dS^T q,
 * with dk, dv of a kv head summed over the q heads that read it.
 * q, k, v, out, dout: as in attn_fwd (out is the forward output); read.
 * lse [B, Hq, Sq] fp32 contiguous: the forward's lse; read.
 * dq [B, Sq, Hq, Dqk], dk [B, Sk, Hkv, Dqk], dv [B, Sk, Hkv, Dv]: written
 *     (every element, zeros where no query reaches a key).
 * (Dqk, Dv) in {(64, 64), (128, 128), (192, 128)}; other supported forward
 * sizes return ATTN_E_UNSUPPORTED here.
 * workspace: attn_bwd_workspace_size(p) bytes, 256-byte aligned, scratch.
 */
typedef struct attn_bwd_params {
  attn_dtype dtype;
  int B, Sq, Sk, Hq, Hkv, Dqk, Dv;
  attn_tensor4 q, k, v, out, dout, dq, dk, dv;
  const float* lse;
  int causal;
  float softmax_scale;
  int window_left, window_right;
  void* workspace;
  size_t workspace_bytes;
} attn_bwd_params;

size_t attn_bwd_workspace_size(const attn_bwd_params* p);
int attn_bwd(const attn_bwd_params* p, void* stream);

/* -------------------------------------------------------------- rope_apply
 * x   [B, S, H, D]  read
 * out [B, S, H, D]  written; may be the same memory as x (in place)
 * Token s of batch b is at position off_b + s with off_b = offsets[b]
 * (device int32 [B]) when offsets is non-NULL, else offset_scalar.
 * Same pairing and rounding as the kvcache rotation; conjugate rotates by
 * the opposite angle (sin -> -sin).  Precondition: off_b + S <= seqlen_ro.
 */
typedef struct attn_rope_params {
  attn_dtype dtype;
  int B, S, H, D;
  attn_tensor4 x, out;
  const void* cos;
  const void* sin;
  int rotary_dim, seqlen_ro, interleaved, conjugate;
  int offset_scalar;
  const int32_t* offsets;
} attn_rope_params;

int rope_apply(const attn_rope_params* p, void* stream);

/* ------------------------------------------------------------ host helpers
 * The attn_validate_* functions run the argument checks of the matching
 * entry point on the host only (no HIP call, nothing enqueued) and return
 * the status that entry point would return.
 */
int attn_validate_fwd(const attn_fwd_params* p);
int attn_validate_kvcache(const attn_kvcache_params* p);
int attn_validate_varlen(const attn_varlen_params* p);
int attn_validate_bwd(const attn_bwd_params* p);
int attn_validate_fp8(const attn_fp8_params* p);
int attn_validate_rope(const attn_rope_params* p);
const char* attn_last_error(void);
int attn_abi_version(void);  /* 3 */

#ifdef __cplusplus
}
#endif
#endif /* ATTN_H_ */
