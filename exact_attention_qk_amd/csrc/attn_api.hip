// C ABI of libattn: argument validation, workspace planning and kernel
// dispatch.  Everything here is host code; it never allocates device memory
// and never reads device memory unless ATTN_CHECK=1 asks it to validate the
// device-side cache lengths.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "attn.h"
#include "launchers.hpp"

namespace {

// The last failure's message, per thread, in a fixed buffer (no allocation).
thread_local char g_err[512];

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return ATTN_OK;
}

bool dims_supported(int dqk, int dv) {
  return (dqk == 16 && dv == 16) || (dqk == 64 && dv == 64) || (dqk == 128 && dv == 128) ||
         (dqk == 192 && dv == 128);
}

int check_dtype(attn_dtype d) {
  if (d != ATTN_DTYPE_F16 && d != ATTN_DTYPE_BF16)
    return fail(ATTN_E_UNSUPPORTED, "dtype %d is not fp16 (0) or bf16 (1)", (int)d);
  return ATTN_OK;
}

// Key/value tiles of up to 64 rows are addressed with 32-bit byte offsets
// (buffer resources and LDS-DMA offsets): 64 rows * 2 bytes * stride < 2^31.
constexpr int64_t kMaxRowStride = (int64_t)1 << 24;

// rows: the tensor's sequence length.  A zero sequence stride over more than
// one row (an expanded view) is refused: key tiles are read through buffer
// resources sized rows * stride, which would be empty.
int check_tensor(const attn_tensor4& t, const char* name, int64_t rows) {
  if (!t.data) return fail(ATTN_E_NULL, "%s: data pointer is NULL", name);
  if (rows > 1 && t.stride_s == 0)
    return fail(ATTN_E_UNSUPPORTED, "%s: sequence stride 0 over %lld rows (expanded view) is not supported", name,
                (long long)rows);
  if (reinterpret_cast<uintptr_t>(t.data) % 16)
    return fail(ATTN_E_ALIGN, "%s: data pointer is not 16-byte aligned", name);
  if (t.stride_b % 8 || t.stride_s % 8 || t.stride_h % 8)
    return fail(ATTN_E_ALIGN, "%s: strides (%lld, %lld, %lld) must be multiples of 8 elements", name,
                (long long)t.stride_b, (long long)t.stride_s, (long long)t.stride_h);
  if (t.stride_b < 0 || t.stride_s < 0 || t.stride_h < 0)
    return fail(ATTN_E_SHAPE, "%s: negative stride", name);
  if (t.stride_s >= kMaxRowStride)
    return fail(ATTN_E_UNSUPPORTED, "%s: sequence stride %lld is not below 2^24 elements", name,
                (long long)t.stride_s);
  return ATTN_OK;
}

float resolve_c(float scale, int dqk) {
  const float s = std::isnan(scale) ? 1.0f / std::sqrt((float)dqk) : scale;
  return s * 1.4426950408889634f;
}

attn::AttnArgs base_args() {
  attn::AttnArgs a;
  std::memset(&a, 0, sizeof(a));
  return a;
}

void set_q(attn::AttnArgs& a, const attn_tensor4& t) {
  a.q = static_cast<const uint16_t*>(t.data); a.q_sb = t.stride_b; a.q_ss = t.stride_s; a.q_sh = t.stride_h;
}
void set_k(attn::AttnArgs& a, const attn_tensor4& t) {
  a.k = static_cast<const uint16_t*>(t.data); a.k_sb = t.stride_b; a.k_ss = t.stride_s; a.k_sh = t.stride_h;
}
void set_v(attn::AttnArgs& a, const attn_tensor4& t) {
  a.v = static_cast<const uint16_t*>(t.data); a.v_sb = t.stride_b; a.v_ss = t.stride_s; a.v_sh = t.stride_h;
}
// -1 (unbounded) becomes a distance no position can exceed
void set_window(attn::AttnArgs& a, int left, int right) {
  a.wl = (left < 0 || left > attn::kNoWindow) ? attn::kNoWindow : left;
  a.wr = (right < 0 || right > attn::kNoWindow) ? attn::kNoWindow : right;
}

void set_o(attn::AttnArgs& a, const attn_tensor4& t) {
  a.out = static_cast<uint16_t*>(t.data); a.o_sb = t.stride_b; a.o_ss = t.stride_s; a.o_sh = t.stride_h;
}

// ---------------------------------------------------------------- kvcache plan
constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct KVPlan {
  bool rotary = false;
  bool decode = false;      // split-KV path (few query rows per kv head)
  bool fused = false;       // decode kernel also appends the new rows and applies the rotary embedding
  bool rotq = false;        // tiled kernel rotates q as it loads it (the append pass then skips q)
  int split_len = 0, num_splits = 0;
  int split_auto = 0;       // > 0: the kernels size the splits from the device-side lengths
  int split_slots = 0;      // splits of all batches together that the workspace holds
  size_t off_qrot = 0, off_o = 0, off_ml = 0, total = 0;
};

// (kv head, split) waves the single-token decode aims for when it sizes its
// splits from the cache lengths
constexpr int kSplitWaves = 1408;

bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

KVPlan plan_kvcache(const attn_kvcache_params* p) {
  KVPlan k;
  k.rotary = p->rotary_cos != nullptr;
  const int group = p->Hq / p->Hkv;
  const int R = group * p->Sq;
  k.decode = R <= 16;
  k.fused = k.decode && (!k.rotary || (p->rotary_dim % 16 == 0 && aligned16(p->rotary_cos) &&
                                       aligned16(p->rotary_sin)));
  k.rotq = !k.decode && k.rotary && p->rotary_dim % 16 == 0 && aligned16(p->rotary_cos) &&
           aligned16(p->rotary_sin);
  size_t off = 0;
  if (k.rotary && !k.fused && !k.rotq) {
    k.off_qrot = off;
    off = align_up(off + (size_t)p->B * p->Sq * p->Hq * p->Dqk * 2);
  }
  if (k.decode) {
    const int cap = p->capacity;
    int len;
    if (p->num_splits > 0) {
      len = (cap + p->num_splits - 1) / p->num_splits;
    } else {
      // The kernels pick the split length from the actual key counts, for
      // about kSplitWaves (kv head, split) waves in all (a workgroup holds the
      // waves of up to 8 kv heads of one split, so about 176 workgroups on the
      // 256-CU MI355X; measured on random cache fills, more splits cost more
      // in the merge than they gain), and never below one 32-key step.
      k.split_auto = kSplitWaves;
      len = 32;
    }
    len = (len + 31) / 32 * 32;
    if (len < 32) len = 32;
    k.split_len = len;
    k.num_splits = (cap + len - 1) / len;
    // Splits are numbered across batches (a batch without keys counts one).
    // Sized from the key counts, batch b has ceil(n_b / len) < n_b / len + 1
    // splits with len >= total * Hkv / kSplitWaves, so all batches together
    // have fewer than kSplitWaves / Hkv + B; whatever the lengths, the cache
    // capacity bounds each batch to num_splits.
    int64_t slots_all = (int64_t)p->B * k.num_splits;
    if (k.split_auto) slots_all = std::min<int64_t>(slots_all, kSplitWaves / p->Hkv + p->B + 1);
    k.split_slots = (int)slots_all;
    const size_t slots = (size_t)k.split_slots * p->Hkv * R;
    k.off_o = off;
    off = align_up(off + slots * p->Dv * sizeof(float));
    k.off_ml = off;
    off = align_up(off + slots * 2 * sizeof(float));
  }
  k.total = off;
  return k;
}

int validate_fwd(const attn_fwd_params* p) {
  if (!p) return fail(ATTN_E_NULL, "params pointer is NULL");
  int e;
  if ((e = check_dtype(p->dtype))) return e;
  if (p->B < 0 || p->Sq < 0 || p->Sk < 0 || p->Hq < 1 || p->Hkv < 1)
    return fail(ATTN_E_SHAPE, "sizes must satisfy B, Sq, Sk >= 0 and Hq, Hkv >= 1");
  if (p->Sq >= attn::kNoWindow || p->Sk >= attn::kNoWindow)
    return fail(ATTN_E_SHAPE, "sequence lengths must be below 2^29");
  if (p->Hq % p->Hkv)
    return fail(ATTN_E_SHAPE, "Hq (%d) must be a multiple of Hkv (%d)", p->Hq, p->Hkv);
  if (!dims_supported(p->Dqk, p->Dv))
    return fail(ATTN_E_UNSUPPORTED, "(Dqk, Dv) = (%d, %d) is not one of (16,16), (64,64), (128,128), (192,128)",
                p->Dqk, p->Dv);
  if (p->window_left < -1 || p->window_right < -1)
    return fail(ATTN_E_SHAPE, "window (%d, %d): each side must be >= -1", p->window_left, p->window_right);
  if (p->B == 0 || p->Sq == 0) return ok();
  if ((e = check_tensor(p->q, "q", p->Sq))) return e;
  if (p->Sk > 0) {
    if ((e = check_tensor(p->k, "k", p->Sk))) return e;
    if ((e = check_tensor(p->v, "v", p->Sk))) return e;
  }
  if ((e = check_tensor(p->out, "out", p->Sq))) return e;
  return ok();
}

// check_ws: whether the caller's workspace is checked (the no-allocation entry
// point brings its own scratch instead)
int validate_kvcache(const attn_kvcache_params* p, bool check_ws = true) {
  if (!p) return fail(ATTN_E_NULL, "params pointer is NULL");
  int e;
  if ((e = check_dtype(p->dtype))) return e;
  if (p->B < 0 || p->Sq < 0 || p->Hq < 1 || p->Hkv < 1 || p->capacity < 1 || p->Snew < 0)
    return fail(ATTN_E_SHAPE, "sizes must satisfy B, Sq, Snew >= 0 and Hq, Hkv, capacity >= 1");
  if (p->Sq >= attn::kNoWindow || p->capacity >= attn::kNoWindow)
    return fail(ATTN_E_SHAPE, "sequence lengths must be below 2^29");
  if (p->Hq % p->Hkv)
    return fail(ATTN_E_SHAPE, "Hq (%d) must be a multiple of Hkv (%d)", p->Hq, p->Hkv);
  if (!dims_supported(p->Dqk, p->Dv))
    return fail(ATTN_E_UNSUPPORTED, "(Dqk, Dv) = (%d, %d) is not one of (16,16), (64,64), (128,128), (192,128)",
                p->Dqk, p->Dv);
  if (p->Snew != 0 && p->Snew != p->Sq)
    return fail(ATTN_E_SHAPE, "Snew (%d) must be 0 or equal to Sq (%d)", p->Snew, p->Sq);
  if (p->window_left < -1 || p->window_right < -1)
    return fail(ATTN_E_SHAPE, "window (%d, %d): each side must be >= -1", p->window_left, p->window_right);
  if (p->Snew > p->capacity)
    return fail(ATTN_E_OVERFLOW, "Snew (%d) exceeds the cache capacity (%d)", p->Snew, p->capacity);
  if (!p->cache_seqlens) {
    if (p->cache_seqlens_scalar < 0)
      return fail(ATTN_E_SHAPE, "cache_seqlens (%d) is negative", p->cache_seqlens_scalar);
    if ((int64_t)p->cache_seqlens_scalar + p->Snew > p->capacity)
      return fail(ATTN_E_OVERFLOW, "cache_seqlens (%d) + Snew (%d) exceeds the capacity (%d)",
                  p->cache_seqlens_scalar, p->Snew, p->capacity);
  }
  const bool rot = p->rotary_cos || p->rotary_sin;
  if (rot) {
    if (!p->rotary_cos || !p->rotary_sin)
      return fail(ATTN_E_NULL, "rotary_cos and rotary_sin must both be given or both be NULL");
    if (p->rotary_dim < 2 || p->rotary_dim % 2 || p->rotary_dim > p->Dqk)
      return fail(ATTN_E_SHAPE, "rotary_dim (%d) must be even and in [2, Dqk=%d]", p->rotary_dim, p->Dqk);
    if (p->seqlen_ro < 1) return fail(ATTN_E_SHAPE, "seqlen_ro must be >= 1");
    if (!p->cache_seqlens &&
        (int64_t)p->cache_seqlens_scalar + (p->Sq > p->Snew ? p->Sq : p->Snew) > p->seqlen_ro)
      return fail(ATTN_E_SHAPE, "positions up to %d exceed the rotary tables (%d rows)",
                  p->cache_seqlens_scalar + (p->Sq > p->Snew ? p->Sq : p->Snew) - 1, p->seqlen_ro);
  }
  if (p->num_splits < 0) return fail(ATTN_E_SHAPE, "num_splits must be >= 0");
  if (p->B == 0 || p->Sq == 0) return ok();
  if ((e = check_tensor(p->q, "q", p->Sq))) return e;
  if ((e = check_tensor(p->k_cache, "k_cache", p->capacity))) return e;
  if ((e = check_tensor(p->v_cache, "v_cache", p->capacity))) return e;
  if ((e = check_tensor(p->out, "out", p->Sq))) return e;
  if (p->Snew > 0) {
    if ((e = check_tensor(p->k_new, "k_new", p->Snew))) return e;
    if ((e = check_tensor(p->v_new, "v_new", p->Snew))) return e;
  }
  const KVPlan plan = plan_kvcache(p);
  if (check_ws && plan.total > 0) {
    if (!p->workspace)
      return fail(ATTN_E_WORKSPACE, "workspace of %zu bytes required, got NULL", plan.total);
    if (p->workspace_bytes < plan.total)
      return fail(ATTN_E_WORKSPACE, "workspace of %zu bytes required, got %zu", plan.total,
                  p->workspace_bytes);
    if (reinterpret_cast<uintptr_t>(p->workspace) % kAlign)
      return fail(ATTN_E_ALIGN, "workspace must be 256-byte aligned");
  }
  return ok();
}

int validate_rope(const attn_rope_params* p) {
  if (!p) return fail(ATTN_E_NULL, "params pointer is NULL");
  int e;
  if ((e = check_dtype(p->dtype))) return e;
  if (p->B < 0 || p->S < 0 || p->H < 0 || p->D < 8 || p->D % 8)
    return fail(ATTN_E_SHAPE, "sizes must satisfy B, S, H >= 0 and D a positive multiple of 8");
  if (p->rotary_dim < 0 || p->rotary_dim % 2 || p->rotary_dim > p->D)
    return fail(ATTN_E_SHAPE, "rotary_dim (%d) must be even and in [0, D=%d]", p->rotary_dim, p->D);
  if (p->seqlen_ro < 1) return fail(ATTN_E_SHAPE, "seqlen_ro must be >= 1");
  if (!p->offsets) {
    if (p->offset_scalar < 0) return fail(ATTN_E_SHAPE, "offset (%d) is negative", p->offset_scalar);
    if ((int64_t)p->offset_scalar + p->S > p->seqlen_ro)
      return fail(ATTN_E_SHAPE, "positions up to %d exceed the rotary tables (%d rows)",
                  p->offset_scalar + p->S - 1, p->seqlen_ro);
  }
  if ((int64_t)p->B * p->S * p->H == 0) return ok();
  if (p->rotary_dim > 0 && (!p->cos || !p->sin)) return fail(ATTN_E_NULL, "cos/sin table is NULL");
  if ((e = check_tensor(p->x, "x", p->S))) return e;
  if ((e = check_tensor(p->out, "out", p->S))) return e;
  return ok();
}

bool env_check() {
  const char* s = std::getenv("ATTN_CHECK");
  return s && s[0] == '1';
}

int hip_fail(hipError_t e, const char* what) {
  return fail(ATTN_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

int validate_varlen(const attn_varlen_params* p) {
  if (!p) return fail(ATTN_E_NULL, "params pointer is NULL");
  int e;
  if ((e = check_dtype(p->dtype))) return e;
  if (p->B < 0 || p->total_q < 0 || p->total_k < 0 || p->max_seqlen_q < 0 || p->Hq < 1 || p->Hkv < 1)
    return fail(ATTN_E_SHAPE, "sizes must satisfy B, total_q, total_k, max_seqlen_q >= 0 and Hq, Hkv >= 1");
  if (p->total_q >= attn::kNoWindow || p->total_k >= attn::kNoWindow)
    return fail(ATTN_E_SHAPE, "sequence lengths must be below 2^29");
  if (p->Hq % p->Hkv)
    return fail(ATTN_E_SHAPE, "Hq (%d) must be a multiple of Hkv (%d)", p->Hq, p->Hkv);
  if (!dims_supported(p->Dqk, p->Dv))
    return fail(ATTN_E_UNSUPPORTED, "(Dqk, Dv) = (%d, %d) is not one of (16,16), (64,64), (128,128), (192,128)",
                p->Dqk, p->Dv);
  if (p->window_left < -1 || p->window_right < -1)
    return fail(ATTN_E_SHAPE, "window (%d, %d): each side must be >= -1", p->window_left, p->window_right);
  if (p->B == 0 || p->total_q == 0) return ok();
  if (!p->cu_seqlens_q || !p->cu_seqlens_k) return fail(ATTN_E_NULL, "cu_seqlens_q / cu_seqlens_k is NULL");
  if ((e = check_tensor(p->q, "q", p->total_q))) return e;
  if (p->total_k > 0) {
    if ((e = check_tensor(p->k, "k", p->total_k))) return e;
    if ((e = check_tensor(p->v, "v", p->total_k))) return e;
  }
  if ((e = check_tensor(p->out, "out", p->total_q))) return e;
  return ok();
}

int validate_bwd(const attn_bwd_params* p) {
  if (!p) return fail(ATTN_E_NULL, "params pointer is NULL");
  int e;
  if ((e = check_dtype(p->dtype))) return e;
  if (p->B < 0 || p->Sq < 0 || p->Sk < 0 || p->Hq < 1 || p->Hkv < 1)
    return fail(ATTN_E_SHAPE, "sizes must satisfy B, Sq, Sk >= 0 and Hq, Hkv >= 1");
  if (p->Sq >= attn::kNoWindow || p->Sk >= attn::kNoWindow)
    return fail(ATTN_E_SHAPE, "sequence lengths must be below 2^29");
  if (p->Hq % p->Hkv)
    return fail(ATTN_E_SHAPE, "Hq (%d) must be a multiple of Hkv (%d)", p->Hq, p->Hkv);
  const bool dims = (p->Dqk == 64 && p->Dv == 64) || (p->Dqk == 128 && p->Dv == 128) ||
                    (p->Dqk == 192 && p->Dv == 128);
  if (!dims)
    return fail(ATTN_E_UNSUPPORTED, "backward (Dqk, Dv) = (%d, %d) is not one of (64,64), (128,128), (192,128)",
                p->Dqk, p->Dv);
  if (p->window_left < -1 || p->window_right < -1)
    return fail(ATTN_E_SHAPE, "window (%d, %d): each side must be >= -1", p->window_left, p->window_right);
  if (p->B == 0 || (p->Sq == 0 && p->Sk == 0)) return ok();
  if (p->Sq > 0) {
    if ((e = check_tensor(p->q, "q", p->Sq))) return e;
    if ((e = check_tensor(p->out, "out", p->Sq))) return e;
    if ((e = check_tensor(p->dout, "dout", p->Sq))) return e;
    if ((e = check_tensor(p->dq, "dq", p->Sq))) return e;
    if (!p->lse) return fail(ATTN_E_NULL, "lse is NULL");
  }
  if (p->Sk > 0) {
    if ((e = check_tensor(p->k, "k", p->Sk))) return e;
    if ((e = check_tensor(p->v, "v", p->Sk))) return e;
    if ((e = check_tensor(p->dk, "dk", p->Sk))) return e;
    if ((e = check_tensor(p->dv, "dv", p->Sk))) return e;
  }
  const size_t need = align_up((size_t)p->B * p->Hq * p->Sq * 2 * sizeof(float));
  if (p->Sq > 0 && p->Sk > 0) {
    if (!p->workspace) return fail(ATTN_E_WORKSPACE, "workspace of %zu bytes required, got NULL", need);
    if (p->workspace_bytes < need)
      return fail(ATTN_E_WORKSPACE, "workspace of %zu bytes required, got %zu", need, p->workspace_bytes);
    if (reinterpret_cast<uintptr_t>(p->workspace) % kAlign)
      return fail(ATTN_E_ALIGN, "workspace must be 256-byte aligned");
  }
  return ok();
}

void set_t(const uint16_t*& ptr, int64_t& sb, int64_t& ss, int64_t& sh, const attn_tensor4& t) {
  ptr = static_cast<const uint16_t*>(t.data); sb = t.stride_b; ss = t.stride_s; sh = t.stride_h;
}
void set_t(uint16_t*& ptr, int64_t& sb, int64_t& ss, int64_t& sh, const attn_tensor4& t) {
  ptr = static_cast<uint16_t*>(t.data); sb = t.stride_b; ss = t.stride_s; sh = t.stride_h;
}

int check_fp8_tensor(const attn_tensor4& t, const char* name, int64_t rows) {
  if (!t.data) return fail(ATTN_E_NULL, "%s: data pointer is NULL", name);
  if (rows > 1 && t.stride_s == 0)
    return fail(ATTN_E_UNSUPPORTED, "%s: sequence stride 0 over %lld rows (expanded view) is not supported", name,
                (long long)rows);
  if (reinterpret_cast<uintptr_t>(t.data) % 16)
    return fail(ATTN_E_ALIGN, "%s: data pointer is not 16-byte aligned", name);
  if (t.stride_b % 16 || t.stride_s % 16 || t.stride_h % 16)
    return fail(ATTN_E_ALIGN, "%s: strides (%lld, %lld, %lld) of a 1-byte tensor must be multiples of 16", name,
                (long long)t.stride_b, (long long)t.stride_s, (long long)t.stride_h);
  if (t.stride_b < 0 || t.stride_s < 0 || t.stride_h < 0)
    return fail(ATTN_E_SHAPE, "%s: negative stride", name);
  if (t.stride_s >= kMaxRowStride)
    return fail(ATTN_E_UNSUPPORTED, "%s: sequence stride %lld is not below 2^24 elements", name,
                (long long)t.stride_s);
  return ATTN_OK;
}

// The FP8 path converts v inside the attention kernel: no workspace.
size_t fp8_workspace(const attn_fp8_params*) { return 0; }

int validate_fp8(const attn_fp8_params* p) {
  if (!p) return fail(ATTN_E_NULL, "params pointer is NULL");
  int e;
  if (p->B < 0 || p->Sq < 0 || p->Sk < 0 || p->Hq < 1 || p->Hkv < 1)
    return fail(ATTN_E_SHAPE, "sizes must satisfy B, Sq, Sk >= 0 and Hq, Hkv >= 1");
  if (p->Sq >= attn::kNoWindow || p->Sk >= attn::kNoWindow)
    return fail(ATTN_E_SHAPE, "sequence lengths must be below 2^29");
  if (p->Hq % p->Hkv)
    return fail(ATTN_E_SHAPE, "Hq (%d) must be a multiple of Hkv (%d)", p->Hq, p->Hkv);
  if (p->D != 64 && p->D != 128)
    return fail(ATTN_E_UNSUPPORTED, "fp8 head size %d is not 64 or 128", p->D);
  if (p->window_left < -1 || p->window_right < -1)
    return fail(ATTN_E_SHAPE, "window (%d, %d): each side must be >= -1", p->window_left, p->window_right);
  if (!std::isfinite(p->descale_q) || !std::isfinite(p->descale_k) || !std::isfinite(p->descale_v))
    return fail(ATTN_E_SHAPE, "descale factors must be finite");
  if (p->B == 0 || p->Sq == 0) return ok();
  if ((e = check_fp8_tensor(p->q, "q", p->Sq))) return e;
  if (p->Sk > 0) {
    if ((e = check_fp8_tensor(p->k, "k", p->Sk))) return e;
    if ((e = check_fp8_tensor(p->v, "v", p->Sk))) return e;
  }
  if ((e = check_tensor(p->out, "out", p->Sq))) return e;
  return ok();
}

extern "C" {

int attn_abi_version(void) { return 3; }

const char* attn_last_error(void) { return g_err; }

int attn_validate_fwd(const attn_fwd_params* p) { return validate_fwd(p); }
int attn_validate_kvcache(const attn_kvcache_params* p) { return validate_kvcache(p); }
int attn_validate_varlen(const attn_varlen_params* p) { return validate_varlen(p); }
int attn_validate_bwd(const attn_bwd_params* p) { return validate_bwd(p); }
int attn_validate_fp8(const attn_fp8_params* p) { return validate_fp8(p); }
int attn_validate_rope(const attn_rope_params* p) { return validate_rope(p); }

int attn_fwd(const attn_fwd_params* p, void* stream) {
  int e = validate_fwd(p);
  if (e) return e;
  if (p->B == 0 || p->Sq == 0) return ok();
  attn::AttnArgs a = base_args();
  set_q(a, p->q); set_k(a, p->k); set_v(a, p->v); set_o(a, p->out);
  a.lse = p->lse;
  a.lse_sb = (int64_t)p->Hq * p->Sq; a.lse_sh = p->Sq;
  a.B = p->B; a.Sq = p->Sq; a.Sk = p->Sk; a.Hq = p->Hq; a.Hkv = p->Hkv; a.group = p->Hq / p->Hkv;
  a.kvcache = 0;
  a.causal = p->causal ? 1 : 0;
  set_window(a, p->window_left, p->window_right);
  a.c = resolve_c(p->softmax_scale, p->Dqk);
  hipError_t he = attn::run_tile_attn(a, p->dtype == ATTN_DTYPE_BF16, p->Dqk, p->Dv, p->causal != 0,
                                      static_cast<hipStream_t>(stream));
  if (he != hipSuccess) return hip_fail(he, "attn_fwd launch");
  return ok();
}

int attn_fwd_varlen(const attn_varlen_params* p, void* stream) {
  int e = validate_varlen(p);
  if (e) return e;
  if (p->B == 0 || p->total_q == 0) return ok();
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (env_check()) {
    std::vector<int32_t> cq(p->B + 1), ck(p->B + 1);
    hipError_t he = hipMemcpyAsync(cq.data(), p->cu_seqlens_q, sizeof(int32_t) * cq.size(),
                                   hipMemcpyDeviceToHost, st);
    if (he == hipSuccess)
      he = hipMemcpyAsync(ck.data(), p->cu_seqlens_k, sizeof(int32_t) * ck.size(), hipMemcpyDeviceToHost, st);
    if (he == hipSuccess) he = hipStreamSynchronize(st);
    if (he != hipSuccess) return hip_fail(he, "ATTN_CHECK copy of cu_seqlens");
    if (cq[0] != 0 || ck[0] != 0 || cq[p->B] != p->total_q || ck[p->B] != p->total_k)
      return fail(ATTN_E_SHAPE, "cu_seqlens must start at 0 and end at total_q / total_k");
    for (int b = 0; b < p->B; ++b) {
      if (cq[b + 1] < cq[b] || ck[b + 1] < ck[b])
        return fail(ATTN_E_SHAPE, "cu_seqlens must be non-decreasing (sequence %d)", b);
      if (cq[b + 1] - cq[b] > p->max_seqlen_q)
        return fail(ATTN_E_SHAPE, "sequence %d has %d query rows > max_seqlen_q %d", b, cq[b + 1] - cq[b],
                    p->max_seqlen_q);
    }
  }
  attn::AttnArgs a = base_args();
  set_q(a, p->q); set_k(a, p->k); set_v(a, p->v); set_o(a, p->out);
  a.q_sb = a.k_sb = a.v_sb = a.o_sb = 0;
  a.lse = p->lse;
  a.lse_sb = 0; a.lse_sh = p->total_q;
  a.varlen = 1;
  a.cu_q = p->cu_seqlens_q;
  a.cu_k = p->cu_seqlens_k;
  a.B = p->B; a.Sq = p->max_seqlen_q; a.Sk = 0; a.Hq = p->Hq; a.Hkv = p->Hkv; a.group = p->Hq / p->Hkv;
  a.kvcache = 0;
  a.causal = p->causal ? 1 : 0;
  set_window(a, p->window_left, p->window_right);
  a.c = resolve_c(p->softmax_scale, p->Dqk);
  if (p->max_seqlen_q == 0) return ok();
  hipError_t he = attn::run_tile_attn(a, p->dtype == ATTN_DTYPE_BF16, p->Dqk, p->Dv, p->causal != 0, st);
  if (he != hipSuccess) return hip_fail(he, "attn_fwd_varlen launch");
  return ok();
}

size_t attn_fwd_fp8_workspace_size(const attn_fp8_params* p) { return fp8_workspace(p); }

int attn_fwd_fp8(const attn_fp8_params* p, void* stream) {
  int e = validate_fp8(p);
  if (e) return e;
  if (p->B == 0 || p->Sq == 0) return ok();
  hipStream_t st = static_cast<hipStream_t>(stream);
  attn::AttnArgs a = base_args();
  set_q(a, p->q); set_k(a, p->k); set_v(a, p->v); set_o(a, p->out);   // e4m3 q, k, v: byte strides
  a.lse = p->lse;
  a.lse_sb = (int64_t)p->Hq * p->Sq; a.lse_sh = p->Sq;
  a.B = p->B; a.Sq = p->Sq; a.Sk = p->Sk; a.Hq = p->Hq; a.Hkv = p->Hkv; a.group = p->Hq / p->Hkv;
  a.causal = p->causal ? 1 : 0;
  set_window(a, p->window_left, p->window_right);
  a.c = resolve_c(p->softmax_scale, p->D) * p->descale_q * p->descale_k;
  a.oscale = p->descale_v;
  hipError_t he = attn::run_tile_attn_fp8(a, p->D, p->causal != 0, st);
  if (he != hipSuccess) return hip_fail(he, "attn_fwd_fp8 launch");
  return ok();
}

size_t attn_bwd_workspace_size(const attn_bwd_params* p) {
  if (!p || p->B < 0 || p->Hq < 1 || p->Sq < 0) return 0;
  return align_up((size_t)p->B * p->Hq * p->Sq * 2 * sizeof(float));
}

int attn_bwd(const attn_bwd_params* p, void* stream) {
  int e = validate_bwd(p);
  if (e) return e;
  if (p->B == 0 || (p->Sq == 0 && p->Sk == 0)) return ok();
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool bf16 = p->dtype == ATTN_DTYPE_BF16;
  if (p->Sq == 0 || p->Sk == 0) {
    // no (query, key) pair: every gradient is zero
    hipError_t he = hipSuccess;
    if (p->Sq) he = attn::run_zero_rows(p->dq.data, p->dq.stride_b, p->dq.stride_s, p->dq.stride_h, p->B, p->Sq,
                                        p->Hq, p->Dqk, st);
    if (he == hipSuccess && p->Sk)
      he = attn::run_zero_rows(p->dk.data, p->dk.stride_b, p->dk.stride_s, p->dk.stride_h, p->B, p->Sk, p->Hkv,
                               p->Dqk, st);
    if (he == hipSuccess && p->Sk)
      he = attn::run_zero_rows(p->dv.data, p->dv.stride_b, p->dv.stride_s, p->dv.stride_h, p->B, p->Sk, p->Hkv,
                               p->Dv, st);
    if (he != hipSuccess) return hip_fail(he, "attn_bwd zero fill");
    return ok();
  }
  attn::BwdArgs a;
  std::memset(&a, 0, sizeof(a));
  set_t(a.q, a.q_sb, a.q_ss, a.q_sh, p->q);
  set_t(a.k, a.k_sb, a.k_ss, a.k_sh, p->k);
  set_t(a.v, a.v_sb, a.v_ss, a.v_sh, p->v);
  set_t(a.o, a.o_sb, a.o_ss, a.o_sh, p->out);
  set_t(a.dout, a.do_sb, a.do_ss, a.do_sh, p->dout);
  set_t(a.dq, a.dq_sb, a.dq_ss, a.dq_sh, p->dq);
  set_t(a.dk, a.dk_sb, a.dk_ss, a.dk_sh, p->dk);
  set_t(a.dv, a.dv_sb, a.dv_ss, a.dv_sh, p->dv);
  a.lse = p->lse;
  a.ld = static_cast<float*>(p->workspace);
  a.B = p->B; a.Sq = p->Sq; a.Sk = p->Sk; a.Hq = p->Hq; a.Hkv = p->Hkv; a.group = p->Hq / p->Hkv;
  a.causal = p->causal ? 1 : 0;
  a.wl = (p->window_left < 0 || p->window_left > attn::kNoWindow) ? attn::kNoWindow : p->window_left;
  a.wr = (p->window_right < 0 || p->window_right > attn::kNoWindow) ? attn::kNoWindow : p->window_right;
  a.c = resolve_c(p->softmax_scale, p->Dqk);
  a.scale = std::isnan(p->softmax_scale) ? 1.0f / std::sqrt((float)p->Dqk) : p->softmax_scale;
  hipError_t he = attn::run_attn_bwd(a, bf16, p->Dqk, p->Dv, st);
  if (he != hipSuccess) return hip_fail(he, "attn_bwd launch");
  return ok();
}

size_t attn_fwd_kvcache_workspace_size(const attn_kvcache_params* p) {
  if (!p || p->Hkv < 1 || p->Hq < 1 || p->capacity < 1 || p->Hq % p->Hkv) return 0;
  return plan_kvcache(p).total;
}

}  // extern "C"

namespace {

// The kvcache call after validation: ws is the workspace the plan's offsets
// point into (the caller's, or the no-allocation entry point's scratch).
int run_kvcache(const attn_kvcache_params* p, hipStream_t st, char* ws) {
  const KVPlan plan = plan_kvcache(p);
  const bool bf16 = p->dtype == ATTN_DTYPE_BF16;
  const int maxrows = p->Sq > p->Snew ? p->Sq : p->Snew;

  if (p->cache_seqlens && env_check()) {
    // debug mode: copy the device lengths to the host in fixed-size chunks
    // (no allocation) and validate them before anything is launched
    int32_t h[256];
    for (int b0 = 0; b0 < p->B; b0 += 256) {
      const int n = p->B - b0 < 256 ? p->B - b0 : 256;
      hipError_t he = hipMemcpyAsync(h, p->cache_seqlens + b0, sizeof(int32_t) * n, hipMemcpyDeviceToHost, st);
      if (he == hipSuccess) he = hipStreamSynchronize(st);
      if (he != hipSuccess) return hip_fail(he, "ATTN_CHECK copy of cache_seqlens");
      for (int i = 0; i < n; ++i) {
        const int b = b0 + i;
        if (h[i] < 0 || (int64_t)h[i] + p->Snew > p->capacity)
          return fail(ATTN_E_OVERFLOW, "cache_seqlens[%d] = %d with Snew %d does not fit capacity %d", b,
                      h[i], p->Snew, p->capacity);
        if (plan.rotary && (int64_t)h[i] + maxrows > p->seqlen_ro)
          return fail(ATTN_E_SHAPE, "cache_seqlens[%d] = %d: positions exceed the rotary tables (%d rows)",
                      b, h[i], p->seqlen_ro);
      }
    }
  }

  uint16_t* qrot = (plan.rotary && !plan.fused && !plan.rotq) ? reinterpret_cast<uint16_t*>(ws + plan.off_qrot)
                                                               : nullptr;
  const int64_t qr_sh = p->Dqk, qr_ss = (int64_t)p->Hq * p->Dqk, qr_sb = (int64_t)p->Sq * qr_ss;

  // 1. append new rows (rotating keys) and rotate the queries, unless the
  //    decode kernel does both itself
  attn::RowSet sets[3];
  int ns = 0;
  auto rowset = [&](const attn_tensor4& x, const uint16_t* ydata, int64_t ysb, int64_t yss,
                    int64_t ysh, int S, int H, int D, bool rotate, bool at_offset) {
    attn::RowSet r;
    std::memset(&r, 0, sizeof(r));
    r.t.x = static_cast<const uint16_t*>(x.data);
    r.t.x_sb = x.stride_b; r.t.x_ss = x.stride_s; r.t.x_sh = x.stride_h;
    r.t.y = const_cast<uint16_t*>(ydata);
    r.t.y_sb = ysb; r.t.y_ss = yss; r.t.y_sh = ysh;
    r.t.B = p->B; r.t.S = S; r.t.H = H; r.t.D = D;
    r.t.cos = static_cast<const uint16_t*>(p->rotary_cos);
    r.t.sin = static_cast<const uint16_t*>(p->rotary_sin);
    r.t.rd = rotate ? p->rotary_dim : 0;
    r.t.interleaved = p->rotary_interleaved ? 1 : 0;
    r.t.conjugate = 0;
    r.t.offsets = p->cache_seqlens;
    r.t.offset_scalar = p->cache_seqlens_scalar;
    r.t.copy_only = rotate ? 0 : 1;
    r.dst_at_offset = at_offset ? 1 : 0;
    sets[ns++] = r;
  };
  if (!plan.fused) {
    if (p->Snew > 0) {
      rowset(p->k_new, static_cast<uint16_t*>(p->k_cache.data), p->k_cache.stride_b, p->k_cache.stride_s,
             p->k_cache.stride_h, p->Snew, p->Hkv, p->Dqk, plan.rotary, true);
      rowset(p->v_new, static_cast<uint16_t*>(p->v_cache.data), p->v_cache.stride_b, p->v_cache.stride_s,
             p->v_cache.stride_h, p->Snew, p->Hkv, p->Dv, false, true);
    }
    if (plan.rotary && !plan.rotq) rowset(p->q, qrot, qr_sb, qr_ss, qr_sh, p->Sq, p->Hq, p->Dqk, true, false);
  }
  if (ns > 0) {
    hipError_t he = attn::run_rope_rows(sets, ns, bf16, st);
    if (he != hipSuccess) return hip_fail(he, "kvcache append launch");
  }

  // 2. attention over the cache prefix
  attn::AttnArgs a = base_args();
  if (qrot) {
    a.q = qrot; a.q_sb = qr_sb; a.q_ss = qr_ss; a.q_sh = qr_sh;
  } else {
    set_q(a, p->q);
  }
  set_k(a, p->k_cache); set_v(a, p->v_cache); set_o(a, p->out);
  a.lse = p->lse;
  a.lse_sb = (int64_t)p->Hq * p->Sq; a.lse_sh = p->Sq;
  a.seqlens = p->cache_seqlens;
  a.seqlen_scalar = p->cache_seqlens_scalar;
  a.B = p->B; a.Sq = p->Sq; a.Sk = p->capacity; a.Hq = p->Hq; a.Hkv = p->Hkv; a.group = p->Hq / p->Hkv;
  a.Snew = p->Snew;
  a.kvcache = 1;
  a.causal = p->causal ? 1 : 0;
  set_window(a, p->window_left, p->window_right);
  a.c = resolve_c(p->softmax_scale, p->Dqk);
  hipError_t he;
  if (plan.decode) {
    a.split_len = plan.split_len;
    a.num_splits = plan.num_splits;
    a.ws_o = reinterpret_cast<float*>(ws + plan.off_o);
    a.ws_ml = reinterpret_cast<float*>(ws + plan.off_ml);
    a.split_auto = plan.split_auto;
    a.split_slots = plan.split_slots;
    if (plan.fused) {
      a.fused = 1;
      if (p->Snew > 0) {
        a.kn = static_cast<const uint16_t*>(p->k_new.data);
        a.kn_sb = p->k_new.stride_b; a.kn_ss = p->k_new.stride_s; a.kn_sh = p->k_new.stride_h;
        a.vn = static_cast<const uint16_t*>(p->v_new.data);
        a.vn_sb = p->v_new.stride_b; a.vn_ss = p->v_new.stride_s; a.vn_sh = p->v_new.stride_h;
      }
      if (plan.rotary) {
        a.rcos = static_cast<const uint16_t*>(p->rotary_cos);
        a.rsin = static_cast<const uint16_t*>(p->rotary_sin);
        a.rd = p->rotary_dim;
        a.rinter = p->rotary_interleaved ? 1 : 0;
      }
    }
    he = attn::run_decode_attn(a, bf16, p->Dqk, p->Dv, p->causal != 0, st);
  } else {
    if (plan.rotq) {
      a.rotq = 1;
      a.rcos = static_cast<const uint16_t*>(p->rotary_cos);
      a.rsin = static_cast<const uint16_t*>(p->rotary_sin);
      a.rd = p->rotary_dim;
      a.rinter = p->rotary_interleaved ? 1 : 0;
    }
    he = attn::run_tile_attn(a, bf16, p->Dqk, p->Dv, p->causal != 0, st);
  }
  if (he != hipSuccess) return hip_fail(he, "kvcache attention launch");
  return ok();
}

// ---------------------------------------------------------------- no-allocation scratch
// Device memory for the workspace of attn_fwd_kvcache_noalloc: one array per
// GPU the library runs on, held until the process ends.  Its device address
// is looked up once per device (with that device current) and kept; host code
// never hands the array's own name to a kernel.
constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The scratch address on the device that runs `st` (ATTN_OK), or an error code.
int scratch_for(hipStream_t st, char** out) {
  int cur = 0;
  hipError_t he = hipGetDevice(&cur);
  if (he != hipSuccess) return hip_fail(he, "hipGetDevice");
  int dev = cur;
  if (st && (he = hipStreamGetDevice(st, &dev)) != hipSuccess) return hip_fail(he, "hipStreamGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(ATTN_E_UNSUPPORTED, "device %d is beyond the %d devices the scratch table holds", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && (he = hipSetDevice(dev)) != hipSuccess) return hip_fail(he, "hipSetDevice");
    void* ptr = nullptr;
    he = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (he != hipSuccess) return hip_fail(he, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(ATTN_E_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = ptr;
  }
  *out = static_cast<char*>(g_scratch_ptr[dev]);
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_fwd_kvcache(const attn_kvcache_params* p, void* stream) {
  int e = validate_kvcache(p);
  if (e) return e;
  if (p->B == 0 || p->Sq == 0) return ok();
  return run_kvcache(p, static_cast<hipStream_t>(stream), static_cast<char*>(p->workspace));
}

int attn_fwd_kvcache_noalloc(const attn_kvcache_params* p, void* stream) {
  int e = validate_kvcache(p, false);
  if (e) return e;
  if (p->B == 0 || p->Sq == 0) return ok();
  const KVPlan plan = plan_kvcache(p);
  if (plan.total > kScratchBytes)
    return fail(ATTN_E_WORKSPACE,
                "attn_fwd_kvcache_noalloc: this call needs %zu bytes of workspace, above the %zu-byte device "
                "scratch; use attn_fwd_kvcache with a caller workspace", plan.total, kScratchBytes);
  char* ws = nullptr;
  if (plan.total > 0 && (e = scratch_for(static_cast<hipStream_t>(stream), &ws))) return e;
  return run_kvcache(p, static_cast<hipStream_t>(stream), ws);
}

int rope_apply(const attn_rope_params* p, void* stream) {
  int e = validate_rope(p);
  if (e) return e;
  if ((int64_t)p->B * p->S * p->H == 0) return ok();
  attn::RowSet r;
  std::memset(&r, 0, sizeof(r));
  r.t.x = static_cast<const uint16_t*>(p->x.data);
  r.t.x_sb = p->x.stride_b; r.t.x_ss = p->x.stride_s; r.t.x_sh = p->x.stride_h;
  r.t.y = static_cast<uint16_t*>(p->out.data);
  r.t.y_sb = p->out.stride_b; r.t.y_ss = p->out.stride_s; r.t.y_sh = p->out.stride_h;
  r.t.B = p->B; r.t.S = p->S; r.t.H = p->H; r.t.D = p->D;
  r.t.cos = static_cast<const uint16_t*>(p->cos);
  r.t.sin = static_cast<const uint16_t*>(p->sin);
  r.t.rd = p->rotary_dim;
  r.t.interleaved = p->interleaved ? 1 : 0;
  r.t.conjugate = p->conjugate ? 1 : 0;
  r.t.offsets = p->offsets;
  r.t.offset_scalar = p->offset_scalar;
  r.t.copy_only = p->rotary_dim == 0 ? 1 : 0;
  r.dst_at_offset = 0;
  hipError_t he = attn::run_rope_rows(&r, 1, p->dtype == ATTN_DTYPE_BF16, static_cast<hipStream_t>(stream));
  if (he != hipSuccess) return hip_fail(he, "rope_apply launch");
  return ok();
}

}  // extern "C"
