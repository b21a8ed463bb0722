// Device helpers shared by the gfx950 kernels of libpkv: storage types,
// exact widening of 16-bit, 8-bit and 4-bit values, round-to-nearest-even
// narrowing, DPP row reductions and the launch checks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "status.h"

namespace pkv {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// Storage tags.  The raw element type is what sits in memory; `bits` is the
// width of one element (I4 packs two codes per byte, element 2i in the low
// nibble), and `bytes` the size of the raw type.
struct F32 { typedef float raw; static constexpr int bytes = 4, bits = 32; };
struct F16 { typedef uint16_t raw; static constexpr int bytes = 2, bits = 16; };
struct BF16 { typedef uint16_t raw; static constexpr int bytes = 2, bits = 16; };
struct I8 { typedef int8_t raw; static constexpr int bytes = 1, bits = 8; };
struct I4 { typedef uint8_t raw; static constexpr int bytes = 1, bits = 4; };

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w & 0xffffu)));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
}
// Signed byte k (0..3) of a dword, widened exactly.
__device__ __forceinline__ float i8_at(uint32_t w, int k) {
  return static_cast<float>(static_cast<int32_t>(w << (24 - 8 * k)) >> 24);
}
// Signed nibble k (0..7) of a dword (two's complement), widened exactly.
__device__ __forceinline__ float i4_at(uint32_t w, int k) {
  return static_cast<float>(static_cast<int32_t>(w << (28 - 4 * k)) >> 28);
}

// fp32 -> bf16 bits, round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (u >> 16) | 0x0040u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));  // RNE conversion
}

// Unpack the elements of one 16-byte chunk to float.
template <typename T> struct Unpack;
template <> struct Unpack<F32> {
  static constexpr int n = 4;
  __device__ __forceinline__ static void run(const u32x4& w, float* x) {
    x[0] = __uint_as_float(w.x); x[1] = __uint_as_float(w.y);
    x[2] = __uint_as_float(w.z); x[3] = __uint_as_float(w.w);
  }
};
template <> struct Unpack<BF16> {
  static constexpr int n = 8;
  __device__ __forceinline__ static void run(const u32x4& w, float* x) {
    const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) { x[2 * i] = bf16_lo(a[i]); x[2 * i + 1] = bf16_hi(a[i]); }
  }
};
template <> struct Unpack<F16> {
  static constexpr int n = 8;
  __device__ __forceinline__ static void run(const u32x4& w, float* x) {
    const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) { x[2 * i] = f16_lo(a[i]); x[2 * i + 1] = f16_hi(a[i]); }
  }
};
// 4-bit storage is read in 8-byte chunks (16 codes): the low two dwords.
template <> struct Unpack<I4> {
  static constexpr int n = 16;
  __device__ __forceinline__ static void run(const u32x4& w, float* x) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      x[k] = i4_at(w.x, k);
      x[8 + k] = i4_at(w.y, k);
    }
  }
};
template <> struct Unpack<I8> {
  static constexpr int n = 16;
  __device__ __forceinline__ static void run(const u32x4& w, float* x) {
    const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int k = 0; k < 4; ++k) x[4 * i + k] = i8_at(a[i], k);
  }
};

// Load `n` consecutive q elements (any float storage) as float.
template <typename T>
__device__ __forceinline__ float load_elem(const typename T::raw* p, int i);
template <> __device__ __forceinline__ float load_elem<F32>(const float* p, int i) { return p[i]; }
template <> __device__ __forceinline__ float load_elem<BF16>(const uint16_t* p, int i) {
  return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}
template <> __device__ __forceinline__ float load_elem<F16>(const uint16_t* p, int i) {
  return static_cast<float>(__builtin_bit_cast(_Float16, p[i]));
}

template <typename T>
__device__ __forceinline__ void store_elem(typename T::raw* p, int i, float v);
template <> __device__ __forceinline__ void store_elem<F32>(float* p, int i, float v) { p[i] = v; }
template <> __device__ __forceinline__ void store_elem<BF16>(uint16_t* p, int i, float v) {
  p[i] = static_cast<uint16_t>(f32_to_bf16_bits(v));
}
template <> __device__ __forceinline__ void store_elem<F16>(uint16_t* p, int i, float v) {
  p[i] = f32_to_f16_bits(v);
}

// ---- cross-lane reductions ------------------------------------------------
// DPP controls (GCN/CDNA encoding).
#define PKV_DPP_QUAD_XOR1 0xB1      // quad_perm [1,0,3,2]
#define PKV_DPP_QUAD_XOR2 0x4E      // quad_perm [2,3,0,1]
#define PKV_DPP_ROW_HALF_MIRROR 0x141
#define PKV_DPP_ROW_MIRROR 0x140

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Combination of lane l with lane l ^ 16 (or l ^ 32), the same in every lane.
// v_permlane16_swap exchanges the odd 16-lane rows of its first operand with
// the even rows of its second (v_permlane32_swap: the upper 32 lanes of the
// first with the lower 32 of the second); with x in both operands, the two
// results hold x's even and odd rows (lower and upper halves), so a
// commutative op of the two results is op(x[l], x[l ^ 16]) in every lane.
// Both run in the VALU; a lane shuffle by 16 or 32 is an LDS permute that
// the wavefront then waits on.
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over aligned groups of N consecutive lanes (N = 8, 16, 32 or 64); every
// lane of a group receives the group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "group size");
  v += dpp<PKV_DPP_QUAD_XOR1>(v);
  v += dpp<PKV_DPP_QUAD_XOR2>(v);
  if (N >= 8) v += dpp<PKV_DPP_ROW_HALF_MIRROR>(v);
  if (N >= 16) v += dpp<PKV_DPP_ROW_MIRROR>(v);
  if (N >= 32) v = sum_xor16(v);
  if (N >= 64) v = sum_xor32(v);
  return v;
}

// Maximum over aligned groups of N consecutive lanes, the same steps as
// group_sum; every lane of a group receives the group's maximum.  All lanes
// of the wavefront must be active.
template <int N>
__device__ __forceinline__ float group_max(float v) {
  static_assert(N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "group size");
  v = fmaxf(v, dpp<PKV_DPP_QUAD_XOR1>(v));
  v = fmaxf(v, dpp<PKV_DPP_QUAD_XOR2>(v));
  if (N >= 8) v = fmaxf(v, dpp<PKV_DPP_ROW_HALF_MIRROR>(v));
  if (N >= 16) v = fmaxf(v, dpp<PKV_DPP_ROW_MIRROR>(v));
  if (N >= 32) v = max_xor16(v);
  if (N >= 64) v = max_xor32(v);
  return v;
}

// Loads of K/V tiles, which a kernel reads once; NT adds the non-temporal
// hint.
template <typename V, bool NT>
__device__ __forceinline__ V load_kv(const void* p) {
  if constexpr (NT) return __builtin_nontemporal_load(static_cast<const V*>(p));
  else return *static_cast<const V*>(p);
}

__device__ __forceinline__ int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace pkv

// Host-side launch check.
#define PKV_LAUNCH_CHECK(what)                                                       \
  do {                                                                               \
    hipError_t e_ = hipGetLastError();                                               \
    if (e_ != hipSuccess)                                                            \
      return pkv::fail(PKV_ERR_DEVICE, "%s launch failed: %s", what, hipGetErrorString(e_)); \
  } while (0)
