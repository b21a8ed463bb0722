// Matrix-core helpers shared by the gfx950 attention kernels: the 16-bit
// MFMA shapes used, packing of fp32 pairs to 16-bit operands, and element
// access within 16-byte chunks.
//
// Operand layouts (wave64), as the kernels use them:
//   v_mfma_f32_16x16x32_{bf16,f16}: lane l holds A[row l%16][8*(l/16) .. +7]
//     and B[8*(l/16) .. +7][col l%16]; the result D[4*(l/16) + i][col l%16]
//     sits in element i of the lane's f32x4.
//   v_mfma_f32_16x16x16{bf16_1k,f16}: the same with 4 elements per lane:
//     A[row l%16][4*(l/16) .. +3], B[4*(l/16) .. +3][col l%16].
#pragma once

#include "device_common.h"

namespace pkv {

template <typename T> struct Mx;
template <> struct Mx<BF16> {
  __device__ __forceinline__ static f32x4 k32(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  __device__ __forceinline__ static f32x4 k16(const u32x2& a, const u32x2& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
  }
  // Two floats -> packed pair (round to nearest even).
  __device__ __forceinline__ static uint32_t pack(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v;
    v.x = static_cast<__bf16>(lo);
    v.y = static_cast<__bf16>(hi);
    return __builtin_bit_cast(uint32_t, v);
  }
  __device__ __forceinline__ static float lo(uint32_t w) { return bf16_lo(w); }
  __device__ __forceinline__ static float hi(uint32_t w) { return bf16_hi(w); }
  // Exact 16-bit image of an integer in [-128, 127] held as float.
  __device__ __forceinline__ static uint32_t int_bits(float x) { return __float_as_uint(x) >> 16; }
  // Two such integers as one operand dword (lo, hi): their high halves.
  __device__ __forceinline__ static uint32_t int_pair(float lo, float hi) {
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
  }
  // 4-bit codes c as operands without a convert (see nib_split): the low
  // half of an operand pair is u = c + 8 under the high byte 0x43, the bf16
  // value 136 + c; the high half is 7 - c under 0xC3, the value c - 135.
  // Both exact; the offsets stay in the products and are taken out
  // afterwards (kOffsetLo4, kOffsetHi4; kOffsetPair4 is the pair
  // (136, -135)).  Opposite signs keep a common component of the other
  // operand from building up in the accumulators.
  static constexpr uint32_t kMagic4 = 0xC3C34343u;
  static constexpr bool kOffset4 = true;
  static constexpr float kOffsetLo4 = 136.f, kOffsetHi4 = -135.f;
  static constexpr uint32_t kOffsetPair4 = 0xC3074308u;
  __device__ __forceinline__ static uint32_t fix4(uint32_t x) { return x; }
};
template <> struct Mx<F16> {
  __device__ __forceinline__ static f32x4 k32(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ __forceinline__ static f32x4 k16(const u32x2& a, const u32x2& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
  }
  __device__ __forceinline__ static uint32_t pack(float lo, float hi) {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    f16x2 v;
    v.x = static_cast<_Float16>(lo);
    v.y = static_cast<_Float16>(hi);
    return __builtin_bit_cast(uint32_t, v);
  }
  __device__ __forceinline__ static float lo(uint32_t w) { return f16_lo(w); }
  __device__ __forceinline__ static float hi(uint32_t w) { return f16_hi(w); }
  __device__ __forceinline__ static uint32_t int_bits(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
  }
  __device__ __forceinline__ static uint32_t int_pair(float lo, float hi) {
    return pack(lo, hi);   // exact: |x| <= 128 is an f16 value
  }
  // 4-bit codes: c + 8 under the high byte 0x64 is the f16 value 1032 + c
  // (low half), 7 - c under 0xE4 is c - 1031 (high half); one packed f16 add
  // of (-1032, 1031) leaves c exactly, so no offset remains.
  static constexpr uint32_t kMagic4 = 0xE4E46464u;
  static constexpr bool kOffset4 = false;
  static constexpr float kOffsetLo4 = 0.f, kOffsetHi4 = 0.f;
  static constexpr uint32_t kOffsetPair4 = 0u;
  __device__ __forceinline__ static uint32_t fix4(uint32_t x) {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    const f16x2 v = __builtin_bit_cast(f16x2, x) + f16x2{-1032.f16, 1031.f16};
    return __builtin_bit_cast(uint32_t, v);
  }
};

// Loads of 2, 4, 8 or 16 bytes into the low dwords of a u32x4.
template <int B>
__device__ __forceinline__ u32x4 load_bytes(const uint8_t* p) {
  u32x4 r = {0u, 0u, 0u, 0u};
  if constexpr (B == 16) {
    r = *reinterpret_cast<const u32x4*>(p);
  } else if constexpr (B == 8) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(p);
    r.x = v.x;
    r.y = v.y;
  } else if constexpr (B == 4) {
    r.x = *reinterpret_cast<const uint32_t*>(p);
  } else {
    static_assert(B == 2, "load width");
    r.x = *reinterpret_cast<const uint16_t*>(p);
  }
  return r;
}

// load_bytes for K/V tiles in global memory (see load_kv).
template <int B, bool NT>
__device__ __forceinline__ u32x4 load_kv_bytes(const uint8_t* p) {
  u32x4 r = {0u, 0u, 0u, 0u};
  if constexpr (B == 16) {
    r = load_kv<u32x4, NT>(p);
  } else if constexpr (B == 8) {
    const u32x2 v = load_kv<u32x2, NT>(p);
    r.x = v.x;
    r.y = v.y;
  } else if constexpr (B == 4) {
    r.x = load_kv<uint32_t, NT>(p);
  } else {
    static_assert(B == 2, "load width");
    r.x = load_kv<uint16_t, NT>(p);
  }
  return r;
}

// Stores of the low 2, 4, 8 or 16 bytes of a u32x4 (vector stores).
template <int B>
__device__ __forceinline__ void store_bytes(uint8_t* p, const u32x4& v) {
  if constexpr (B == 16) {
    *reinterpret_cast<u32x4*>(p) = v;
  } else if constexpr (B == 8) {
    *reinterpret_cast<u32x2*>(p) = u32x2{v.x, v.y};
  } else if constexpr (B == 4) {
    *reinterpret_cast<uint32_t*>(p) = v.x;
  } else {
    static_assert(B == 2, "store width");
    *reinterpret_cast<uint16_t*>(p) = static_cast<uint16_t>(v.x);
  }
}

// gfx950 LDS transpose read of 16-bit elements (8 bytes per lane).  Within
// each group of 16 lanes, lane j receives element j % 4 of the 4-element
// runs that lanes j / 4, 4 + j / 4, 8 + j / 4 and 12 + j / 4 of the group
// point at (in that order).  So when lane 4k + q points at row k of a
// row-major tile, columns c + 4q .. c + 4q + 3, lane j receives column c + j
// of rows 0 .. 3: a 4 x 16 block transposed.  `p` is an 8-byte aligned
// address in LDS.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint8_t* p) {
  typedef short s16x4_t __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
  const s16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)((__attribute__((address_space(3))) const uint8_t*)p));
  return __builtin_bit_cast(u32x2, r);
}

// gfx950 direct load of 16 bytes per lane from global memory into LDS: lane
// l's bytes land at lds + 16 l (lds: wave-uniform, 16-byte aligned).  The
// load counts in vmcnt like any vector load; its data is in LDS once that
// count has passed it.
__device__ __forceinline__ void load_to_lds16(const void* g, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

__device__ __forceinline__ uint32_t dw(const u32x4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Element j of chunk x in the low half and element j of chunk y in the high
// half of one dword (one v_perm_b32).
__device__ __forceinline__ uint32_t pair_of(const u32x4& x, const u32x4& y, int j) {
  return __builtin_amdgcn_perm(dw(y, j >> 1), dw(x, j >> 1), (j & 1) ? 0x07060302u : 0x05040100u);
}

// byte k of a dword as a float (one byte convert): a sign-flipped int8 code
// read as u = code + 128
__device__ __forceinline__ float u8_value(uint32_t flipped, int k) {
  return static_cast<float>((flipped >> (8 * k)) & 0xffu);
}

// 4-bit codes of one dword (element 2i in the low nibble of byte i), one
// per byte: nib_lo takes elements 0, 2, 4, 6 and nib_hi elements 1, 3, 5, 7.
// A byte bound for the low half of an operand pair is XORed with 8 (c + 8),
// one for the high half with 7 (7 - c): `flip` gives the choice per byte.
constexpr uint32_t kFlipPairs = 0x07080708u;   // bytes 0, 2 low halves; 1, 3 high
constexpr uint32_t kFlipLow = 0x08080808u;
constexpr uint32_t kFlipHigh = 0x07070707u;
__device__ __forceinline__ uint32_t nib_lo(uint32_t w, uint32_t flip) {
  return (w & 0x0F0F0F0Fu) ^ flip;
}
__device__ __forceinline__ uint32_t nib_hi(uint32_t w, uint32_t flip) {
  return ((w >> 4) & 0x0F0F0F0Fu) ^ flip;
}
// Bytes 2p and 2p + 1 of x under the high bytes 0 and 2 of `magic`, as the
// two 16-bit halves of one operand dword.
__device__ __forceinline__ uint32_t magic_pair(uint32_t magic, uint32_t x, int p) {
  return __builtin_amdgcn_perm(magic, x, p ? 0x06030402u : 0x06010400u);
}

// int8 codes as exact f16 operands.  A code k XORed with 0x80 is the byte
// u = k + 128; under the high byte 0x64 a byte u is the f16 value 1024 + u,
// so one byte permute forms a pair (1024 + u0, 1024 + u1) and one packed f16
// add of (-1152, -1152) leaves (k0, k1) exactly (integers below 2048 are f16
// values).  i8_pair takes bytes 2p and 2p + 1 of a dword of flipped codes.
constexpr uint32_t kI8Magic = 0x64646464u;
__device__ __forceinline__ uint32_t i8_pair(uint32_t flipped, int p) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  const uint32_t x = magic_pair(kI8Magic, flipped, p);
  const f16x2 v = __builtin_bit_cast(f16x2, x) + f16x2{-1152.f16, -1152.f16};
  return __builtin_bit_cast(uint32_t, v);
}

// Lazy rescaling of an online softmax: the running reference max moves only
// when a new score exceeds it by more than this (log2 units), so weights
// stay below 2^8 (far from fp32 overflow) and the accumulators are rescaled
// only on the rare blocks that raise the max that much.  The result is the
// same softmax up to rounding: the reference cancels in the final division.
constexpr float kRescaleSlack = 8.f;

// Element j of a chunk of 16-bit values, as the low 16 bits.
__device__ __forceinline__ uint32_t half_of(const u32x4& v, int j) {
  const uint32_t w = dw(v, j >> 1);
  return (j & 1) ? (w >> 16) : (w & 0xffffu);
}

}  // namespace pkv
