// Device-side building blocks shared by the gfx950 attention kernels.
//
// Layout facts used throughout (checked on gfx950 with a one-wave probe):
//  * v_mfma_f32_32x32x16_{f16,bf16}: lane l holds A[l%32][8*(l/32)+j] and
//    B[8*(l/32)+j][l%32] (j = 0..7); result element r of lane l is
//    C[(r/4)*8 + 4*(l/32) + r%4][l%32].
//  * v_mfma_f32_16x16x32_{f16,bf16}: lane l holds A[l%16][8*(l/16)+j] and
//    B[8*(l/16)+j][l%16]; result element r of lane l is C[4*(l/16)+r][l%16].
//  * ds_read_b64_tr_b16: inside each group of 16 lanes, output lane i gets
//    element t (t = 0..3) from element i%4 of the 8 bytes read by input lane
//    4t + i/4.  So if input lane 4t+q reads row t, columns c0+4q..c0+4q+3 of a
//    row-major tile, output lane i holds column c0+i of rows 0..3: a transposed
//    read that turns a row-major V tile into the MFMA operand that contracts
//    over V's rows.
//  * v_permlane32_swap(x, x) returns {x[l or l-32], x[l+32 or l]}; the max
//    (or sum) of the two results combines lane l with lane l^32.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_AS __attribute__((address_space(3)))

// Element type traits: storage is always 16-bit; T selects MFMA flavour and conversions.
struct F16 {
  typedef _Float16 scalar;
  typedef f16x8 vec8;
  static __device__ __forceinline__ float to_f32(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
  }
  static __device__ __forceinline__ uint16_t from_f32(float x) {  // round to nearest even
    return __builtin_bit_cast(uint16_t, (_Float16)x);
  }
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    f16x2 v = __builtin_convertvector((f32x2){a, b}, f16x2);
    return __builtin_bit_cast(uint32_t, v);
  }
  static __device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};

struct BF16 {
  typedef __bf16 scalar;
  typedef bf16x8 vec8;
  static __device__ __forceinline__ float to_f32(uint16_t b) {
    return __builtin_bit_cast(float, (uint32_t)b << 16);
  }
  static __device__ __forceinline__ uint16_t from_f32(float x) {  // round to nearest even
    return __builtin_bit_cast(uint16_t, (__bf16)x);
  }
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    bf16x2 v = __builtin_convertvector((f32x2){a, b}, bf16x2);
    return __builtin_bit_cast(uint32_t, v);
  }
  static __device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

__device__ __forceinline__ u32x4 ldg16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void stg16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// 8-byte transposed LDS read (see header comment).
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* lds_ptr) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(lds_ptr));
  return __builtin_bit_cast(u32x2, v);
}

// max / sum of a value held by lane l and lane l^32.
__device__ __forceinline__ float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, x), false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// max / sum of a value held by lane l and lane l^16: v_permlane16_swap(x, x)
// swaps the odd 16-lane rows of its first operand with the even rows of its
// second, so its two results are {x[l], x[l+16]} in rows 0 and 2 and
// {x[l-16], x[l]} in rows 1 and 3 (a VALU exchange, no LDS round trip).
__device__ __forceinline__ float x16_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x), false,
                                            false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float x16_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x), false,
                                            false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// One rotated 16-bit element: the first member of a pair gives x1*c - x2*s,
// the second x1*s + x2*c.  Both products of 16-bit inputs are exact in fp32,
// so the fp32 result is the exact value rounded once; it is then rounded to
// the storage type.  The empty asm keeps the compiler from fusing the fp32
// operation and the 16-bit conversion into one mixed-precision instruction
// (which would round the exact value straight to 16 bits).
template <class T>
__device__ __forceinline__ uint16_t rot_one(uint16_t x1b, uint16_t x2b, uint16_t cb, uint16_t sb, bool second,
                                            bool conj) {
  const float x1 = T::to_f32(x1b), x2 = T::to_f32(x2b), c = T::to_f32(cb);
  float sn = T::to_f32(sb);
  if (conj) sn = -sn;
  float y = second ? x1 * sn + x2 * c : x1 * c - x2 * sn;
  asm volatile("" : "+v"(y));
  return T::from_f32(y);
}

// Elements [d0, d0 + 8) of row x after rotary embedding at table row `pos`:
// the first rd dims are rotated in pairs (2j, 2j+1) when interleaved, else
// (j, j + rd/2); the rest are copied.  Needs d0 % 8 == 0, rd % 16 == 0 and
// 16-byte aligned rows of the [*, rd/2] cos/sin tables.  Every load of the
// row happens before the result exists, so callers may store it in place.
template <class T>
__device__ __forceinline__ u32x4 rope_chunk(const uint16_t* x, int d0, const uint16_t* cos_t,
                                            const uint16_t* sin_t, int64_t pos, int rd, bool interleaved,
                                            bool conj) {
  const u32x4 xv = ldg16(x + d0);
  if (d0 >= rd) return xv;
  const int half = rd >> 1;
  u32x4 out;
  if (interleaved) {
    const u32x2 cc = *reinterpret_cast<const u32x2*>(cos_t + pos * half + (d0 >> 1));
    const u32x2 sv = *reinterpret_cast<const u32x2*>(sin_t + pos * half + (d0 >> 1));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint16_t x1 = (uint16_t)(xv[e] & 0xFFFFu), x2 = (uint16_t)(xv[e] >> 16);
      const uint16_t cb = (uint16_t)(cc[e >> 1] >> (16 * (e & 1)));
      const uint16_t sb = (uint16_t)(sv[e >> 1] >> (16 * (e & 1)));
      out[e] = (uint32_t)rot_one<T>(x1, x2, cb, sb, false, conj) |
               ((uint32_t)rot_one<T>(x1, x2, cb, sb, true, conj) << 16);
    }
  } else {
    const bool second = d0 >= half;
    const int j0 = second ? d0 - half : d0;
    const u32x4 pv = ldg16(x + (second ? d0 - half : d0 + half));
    const u32x4 cc = ldg16(cos_t + pos * half + j0);
    const u32x4 sv = ldg16(sin_t + pos * half + j0);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint16_t own = (uint16_t)(xv[e >> 1] >> (16 * (e & 1)));
      const uint16_t oth = (uint16_t)(pv[e >> 1] >> (16 * (e & 1)));
      const uint16_t cb = (uint16_t)(cc[e >> 1] >> (16 * (e & 1)));
      const uint16_t sb = (uint16_t)(sv[e >> 1] >> (16 * (e & 1)));
      const uint16_t r = second ? rot_one<T>(oth, own, cb, sb, true, conj) : rot_one<T>(own, oth, cb, sb, false, conj);
      if (e & 1)
        out[e >> 1] |= (uint32_t)r << 16;
      else
        out[e >> 1] = r;
    }
  }
  return out;
}

// Buffer resource over [base, base + bytes) for raw (unswizzled, stride 0)
// loads: offsets at or past `bytes` read as zero, per dword.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, int bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  return (i32x4){(int)(uint32_t)p, (int)((uint32_t)(p >> 32) & 0xFFFFu), bytes, 0x00020000};
}

// 16 bytes per lane from a buffer resource (byte offset voff) into LDS at
// lds_addr + 16 * lane.  The instruction has no destination register; the
// caller waits for completion with vmcnt before the LDS data is read.
__device__ __forceinline__ void dma_b128(i32x4 rsrc, uint32_t lds_addr, int voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

// 16-byte chunk swizzles of row-major LDS tiles.  A tile row of D 16-bit
// elements holds C = D/8 chunks; chunk c of row r is stored at position
// c ^ swz(r) of that row.
//  * K tiles are read 16 B per lane from 16 different rows at one chunk
//    column; the swizzle spreads those 16 reads over all 64 banks.
//  * V tiles are read by ds_read_b64_tr_b16: 4 consecutive rows x 2 adjacent
//    chunks per 16-lane group; the swizzle puts the 4 row pairs on 4 disjoint
//    bank ranges.
template <int C>
__device__ __forceinline__ int swz_k(int r) {
  if constexpr (C % 16 == 0) return r & 15;
  else if constexpr (C % 8 == 0) return (r >> 1) & 7;
  else if constexpr (C == 4) return (r >> 2) & 3;
  else if constexpr (C == 2) return (r >> 3) & 1;
  else return 0;
}
template <int C>
__device__ __forceinline__ int swz_v(int r) {
  if constexpr (C % 16 == 0) return (r & 7) << 1;
  else if constexpr (C % 8 == 0) return ((r >> 1) & 3) << 1;
  else return 0;
}
// V tiles of the tiled kernel: each 32-lane half of a ds_read_b64_tr_b16
// reads 4 consecutive rows x 4 adjacent chunks (64 bytes of each row), and
// the LDS serves 32 lanes (256 bytes, all 64 banks) per cycle for this read.
// The swizzle moves the 4 rows' chunk quads onto 4 disjoint quarters of the
// banks: rows of 256 bytes (C = 16) XOR the chunk with 4 * (r % 4); rows of
// 128 bytes (C = 8, two rows per bank line) with 4 * ((r / 2) % 2).
template <int C>
__device__ __forceinline__ int swz_vt(int r) {
  if constexpr (C % 16 == 0) return (r & 3) << 2;
  else if constexpr (C % 8 == 0) return ((r >> 1) & 1) << 2;
  else return 0;
}

}  // namespace attn
