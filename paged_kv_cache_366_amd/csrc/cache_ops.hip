// reshape_and_cache and copy_blocks for gfx950.
//
// reshape_and_cache appends the new tokens' K/V rows to the cache: only the
// new token's KV is computed each step and appended (m.nxbn.cn section 一),
// at the slot the page table assigns it (m.nxbn.cn §2.2).  copy_blocks is the
// data copy of copy-on-write (kongchang.com "vLLM架构深度解析…", section
// "KV Cache内存共享").
//
// Both are pure byte movement, bound by HBM: every thread moves 16-byte
// chunks so each wavefront access is a fully used 1 KiB span, and neither
// kernel touches a slot or block outside the pool whatever the index arrays
// hold.
#include <atomic>
#include <type_traits>
#include <unordered_set>
#include <vector>

#include "device_common.h"
#include "host_checks.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;

// One workgroup per new token.  A token's K row is num_kv_heads runs of
// head_bytes bytes, each landing at (block, head, row) of the pool.
__global__ __launch_bounds__(kThreads) void reshape_and_cache_kernel(
    const uint8_t* __restrict__ key, const uint8_t* __restrict__ value, uint8_t* __restrict__ kc,
    uint8_t* __restrict__ vc, const int32_t* __restrict__ slots, int64_t key_stride_b,
    int64_t value_stride_b, int hkv, int head_bytes, int block_size, int64_t num_slots) {
  const int t = blockIdx.x;
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot / block_size;
  const int64_t row = slot % block_size;
  const int chunks_per_head = head_bytes / 16;
  const int total = hkv * chunks_per_head;
  const uint8_t* ksrc = key + t * key_stride_b;
  const uint8_t* vsrc = value + t * value_stride_b;
  for (int c = threadIdx.x; c < total; c += kThreads) {
    const int h = c / chunks_per_head;
    const int o = (c % chunks_per_head) * 16;
    const int64_t dst = ((blk * hkv + h) * block_size + row) * head_bytes + o;
    const int64_t src = static_cast<int64_t>(h) * head_bytes + o;
    *reinterpret_cast<u32x4*>(kc + dst) = *reinterpret_cast<const u32x4*>(ksrc + src);
    *reinterpret_cast<u32x4*>(vc + dst) = *reinterpret_cast<const u32x4*>(vsrc + src);
  }
}

constexpr int kCopyUnroll = 4;
constexpr int kCopyChunkBytes = kThreads * 16 * kCopyUnroll;  // 16 KiB per workgroup

// grid (pair, K or V, chunk of the block).
__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(
    uint8_t* __restrict__ kc, uint8_t* __restrict__ vc, float* __restrict__ ks,
    float* __restrict__ vs, const int32_t* __restrict__ pairs, int64_t block_bytes, int hkv,
    int num_blocks) {
  const int p = blockIdx.x;
  const int src = pairs[2 * p];
  const int dst = pairs[2 * p + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  uint8_t* base = blockIdx.y == 0 ? kc : vc;
  const uint8_t* s = base + src * block_bytes;
  uint8_t* d = base + dst * block_bytes;
  const int64_t start = static_cast<int64_t>(blockIdx.z) * kCopyChunkBytes;
  u32x4 buf[kCopyUnroll];
#pragma unroll
  for (int i = 0; i < kCopyUnroll; ++i) {
    const int64_t o = start + (static_cast<int64_t>(i) * kThreads + threadIdx.x) * 16;
    if (o < block_bytes) buf[i] = *reinterpret_cast<const u32x4*>(s + o);
  }
#pragma unroll
  for (int i = 0; i < kCopyUnroll; ++i) {
    const int64_t o = start + (static_cast<int64_t>(i) * kThreads + threadIdx.x) * 16;
    if (o < block_bytes) *reinterpret_cast<u32x4*>(d + o) = buf[i];
  }
  if (blockIdx.z == 0 && threadIdx.x < hkv) {
    float* sc = blockIdx.y == 0 ? ks : vs;
    if (sc) sc[dst * hkv + threadIdx.x] = sc[src * hkv + threadIdx.x];
  }
}

// Int8 and 4-bit storage of whole blocks: one wavefront per (listed block,
// KV head, K or V) tile.  The first pass takes max |x| over the filled rows,
// the second writes the codes (from registers for tiles up to 4 KiB); every
// step is the float32 arithmetic of the encoding: s = a / Q, code =
// rint(x / s) clamped to [-Q, Q] (Q = 127 for int8, 7 for 4-bit), rows past
// the filled count 0, a subnormal scale counting as zero.  4-bit codes are
// stored two per byte, element 2i in the low nibble.
constexpr float kSmallestNormal = 1.17549435e-38f;

__device__ __forceinline__ float wave_absmax(float v) { return group_max<64>(v); }

template <int BITS> constexpr float kCodeMax = BITS == 8 ? 127.f : 7.f;

// The code of x under scale s > 0: rint(x / s) of the float32 quotient
// (ties to even), clamped to [-Q, Q]; r is float32(1 / s).  Every caller has
// |x / s| <= Q (1 + 2^-23) with Q <= 127, so x * r lies within
// 2^-23 |x / s| < 1.6e-5 of x / s and the float32 quotient within half an
// ulp (< 3.9e-6); their rint can differ only if x * r is within 2e-5 of a
// half-integer.  Values within 2^-14 of one (about 1 in 8,000) take the
// division; the others round x * r.
constexpr float kHalfSlack = 6.103515625e-05f;   // 2^-14
template <int BITS>
__device__ __forceinline__ int encode_one(float x, float s, float r) {
  const float qf = x * r;
  float q = rintf(qf);
  if (!(fabsf(qf - q) < 0.5f - kHalfSlack)) q = rintf(x / s);
  return static_cast<int>(fminf(fmaxf(q, -kCodeMax<BITS>), kCodeMax<BITS>));
}

// Stores E codes at d: one byte each, or two per byte (4-bit).
template <int BITS, int E>
__device__ __forceinline__ void store_codes(uint8_t* d, const int (&q)[E]) {
  if constexpr (BITS == 8) {
    int8_t b[E];
#pragma unroll
    for (int e = 0; e < E; ++e) b[e] = static_cast<int8_t>(q[e]);
    if constexpr (E == 16) {
      *reinterpret_cast<u32x4*>(d) = __builtin_bit_cast(u32x4, b);
    } else if constexpr (E == 8) {
      *reinterpret_cast<uint64_t*>(d) = __builtin_bit_cast(uint64_t, b);
    } else {
      static_assert(E == 4, "chunk");
      *reinterpret_cast<uint32_t*>(d) = __builtin_bit_cast(uint32_t, b);
    }
  } else {
    static_assert(BITS == 4, "code width");
    uint8_t b[E / 2];
#pragma unroll
    for (int i = 0; i < E / 2; ++i)
      b[i] = static_cast<uint8_t>((q[2 * i] & 15) | ((q[2 * i + 1] & 15) << 4));
    if constexpr (E == 32) {
      *reinterpret_cast<u32x4*>(d) = __builtin_bit_cast(u32x4, b);
    } else if constexpr (E == 8) {
      *reinterpret_cast<uint32_t*>(d) = __builtin_bit_cast(uint32_t, b);
    } else {
      static_assert(E == 4, "chunk");
      *reinterpret_cast<uint16_t*>(d) = __builtin_bit_cast(uint16_t, b);
    }
  }
}

// The 128 / BITS codes of 16 stored bytes, widened exactly.
template <int BITS>
__device__ __forceinline__ void load_codes(const u32x4& w, float (&c)[128 / BITS]) {
  const uint32_t a[4] = {w.x, w.y, w.z, w.w};
  constexpr int P = 32 / BITS;   // codes per dword
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int k = 0; k < P; ++k) c[P * i + k] = BITS == 8 ? i8_at(a[i], k) : i4_at(a[i], k);
}

template <typename T, int BITS>
__global__ __launch_bounds__(kThreads) void quantize_blocks_kernel(
    const uint8_t* __restrict__ src_k, const uint8_t* __restrict__ src_v,
    uint8_t* __restrict__ dst_k, uint8_t* __restrict__ dst_v, float* __restrict__ ks,
    float* __restrict__ vs, const int32_t* __restrict__ blocks,
    const int32_t* __restrict__ filled, int n, int hkv, int head_dim, int block_size,
    int num_blocks) {
  constexpr int E = 16 / T::bytes;                 // elements per 16-byte chunk
  const int tile = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (tile >= n * hkv * 2) return;
  const int which = tile & 1;
  const int h = (tile >> 1) % hkv;
  const int i = (tile >> 1) / hkv;
  const int b = blocks[i];
  const int f = min(filled[i], block_size);
  if (b < 0 || b >= num_blocks || f <= 0) return;
  const int64_t elems = static_cast<int64_t>(block_size) * head_dim;
  const int64_t tix = static_cast<int64_t>(b) * hkv + h;
  const uint8_t* src = (which ? src_v : src_k) + tix * elems * T::bytes;
  uint8_t* dst = (which ? dst_v : dst_k) + tix * elems * BITS / 8;
  const int filled_chunks = f * head_dim / E;
  const int all_chunks = block_size * head_dim / E;

  // Tiles of up to 256 chunks (16 rows of 128 bf16 or 64 fp32 values) stay
  // in registers between the two passes; larger ones are read again.
  constexpr int kKeep = 4;
  const bool keep = all_chunks <= 64 * kKeep;
  u32x4 held[kKeep];
  float amax = 0.f;
  if (keep) {
#pragma unroll
    for (int k = 0; k < kKeep; ++k) {
      const int c = lane + 64 * k;
      held[k] = u32x4{0u, 0u, 0u, 0u};
      if (c < filled_chunks) held[k] = *reinterpret_cast<const u32x4*>(src + c * 16);
    }
#pragma unroll
    for (int k = 0; k < kKeep; ++k) {
      float x[E];
      Unpack<T>::run(held[k], x);
#pragma unroll
      for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(x[e]));
    }
  } else {
    for (int c = lane; c < filled_chunks; c += 64) {
      float x[E];
      Unpack<T>::run(*reinterpret_cast<const u32x4*>(src + c * 16), x);
#pragma unroll
      for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(x[e]));
    }
  }
  amax = wave_absmax(amax);
  float sc = amax / kCodeMax<BITS>;
  if (!(sc >= kSmallestNormal)) sc = 0.f;
  const float rsc = sc > 0.f ? 1.f / sc : 0.f;

  auto encode = [&](int c, const u32x4& w) {
    int q[E];
    if (c < filled_chunks && sc > 0.f) {
      float x[E];
      Unpack<T>::run(w, x);
#pragma unroll
      for (int e = 0; e < E; ++e) q[e] = encode_one<BITS>(x[e], sc, rsc);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) q[e] = 0;
    }
    store_codes<BITS, E>(dst + static_cast<int64_t>(c) * E * BITS / 8, q);
  };
  if (keep) {
#pragma unroll
    for (int k = 0; k < kKeep; ++k) {
      const int c = lane + 64 * k;
      if (c < all_chunks) encode(c, held[k]);
    }
  } else {
    for (int c = lane; c < all_chunks; c += 64) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (c < filled_chunks) w = *reinterpret_cast<const u32x4*>(src + c * 16);
      encode(c, w);
    }
  }
  if (lane == 0) (which ? vs : ks)[tix] = sc;
}

// Block copies between two pools (or a pool and a packed staging area):
// block k of the list goes from src block src_ids[k] (or k) to dst block
// dst_ids[k] (or k).  grid (block of the list, K or V, 16 KiB chunk).
__global__ __launch_bounds__(kThreads) void copy_list_kernel(
    uint8_t* __restrict__ dst_k, uint8_t* __restrict__ dst_v, const uint8_t* __restrict__ src_k,
    const uint8_t* __restrict__ src_v, const int32_t* __restrict__ dst_ids,
    const int32_t* __restrict__ src_ids, int64_t block_bytes) {
  const int k = blockIdx.x;
  const int64_t d = dst_ids ? dst_ids[k] : k;
  const int64_t s = src_ids ? src_ids[k] : k;
  const uint8_t* src = (blockIdx.y == 0 ? src_k : src_v) + s * block_bytes;
  uint8_t* dst = (blockIdx.y == 0 ? dst_k : dst_v) + d * block_bytes;
  const int64_t start = static_cast<int64_t>(blockIdx.z) * kCopyChunkBytes;
  u32x4 buf[kCopyUnroll];
#pragma unroll
  for (int i = 0; i < kCopyUnroll; ++i) {
    const int64_t o = start + (static_cast<int64_t>(i) * kThreads + threadIdx.x) * 16;
    if (o < block_bytes) buf[i] = *reinterpret_cast<const u32x4*>(src + o);
  }
#pragma unroll
  for (int i = 0; i < kCopyUnroll; ++i) {
    const int64_t o = start + (static_cast<int64_t>(i) * kThreads + threadIdx.x) * 16;
    if (o < block_bytes) *reinterpret_cast<u32x4*>(dst + o) = buf[i];
  }
}

// Quantise-on-write: new tokens' K/V rows go into int8 or 4-bit pools with
// one scale per (block, KV head).  The slot mapping splits into runs
// (consecutive tokens whose slots are consecutive rows of one block); the
// first token of a run leads it, and one wavefront per (run, head, K or V)
// takes the run's block as written below the run's first row.  The scale
// only grows: to max(old scale, max|new rows| / Q); when it grows, each
// existing code is re-encoded from its value (code x old scale / new scale,
// rounded to nearest even), and the new rows are encoded with the new
// scale.  Writing a whole block in one run is the whole-block encoder
// exactly.
template <typename T, int BITS>
__global__ __launch_bounds__(kThreads) void reshape_and_cache_quant_kernel(
    const uint8_t* __restrict__ key, const uint8_t* __restrict__ value,
    uint8_t* __restrict__ kc, uint8_t* __restrict__ vc, float* __restrict__ ks,
    float* __restrict__ vs, const int32_t* __restrict__ slots, int n, int64_t key_stride_b,
    int64_t value_stride_b, int hkv, int head_dim, int block_size, int64_t num_slots) {
  constexpr int E = 16 / T::bytes;                 // elements per 16-byte chunk
  const int64_t w = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (w >= static_cast<int64_t>(n) * hkv * 2) return;
  const int which = static_cast<int>(w & 1);
  const int h = static_cast<int>((w >> 1) % hkv);
  const int t = static_cast<int>((w >> 1) / hkv);
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t b = slot / block_size;
  const int r0 = static_cast<int>(slot % block_size);
  if (t > 0 && r0 > 0 && slots[t - 1] == slot - 1) return;   // inside a run led earlier
  int k = 1;                                                  // the run's rows
  while (t + k < n && k < block_size - r0 && slots[t + k] == slot + k) ++k;

  const int64_t tix = b * hkv + h;
  const int row_b = head_dim * BITS / 8;           // bytes of one stored row
  uint8_t* dst = (which ? vc : kc) + tix * block_size * row_b;
  float* scale = which ? vs : ks;
  const uint8_t* src = (which ? value : key) + static_cast<int64_t>(h) * head_dim * T::bytes;
  const int64_t stride = which ? value_stride_b : key_stride_b;
  const int ch = head_dim / E;                     // 16-byte chunks per source row

  float amax = 0.f;
  for (int c = lane; c < k * ch; c += 64) {
    float x[E];
    Unpack<T>::run(*reinterpret_cast<const u32x4*>(src + (t + c / ch) * stride + (c % ch) * 16),
                   x);
#pragma unroll
    for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(x[e]));
  }
  amax = wave_absmax(amax);
  const float s_old = r0 > 0 ? scale[tix] : 0.f;
  float s_new = fmaxf(s_old, amax / kCodeMax<BITS>);
  if (!(s_new >= kSmallestNormal)) s_new = 0.f;
  const float r_new = s_new > 0.f ? 1.f / s_new : 0.f;

  if (s_new > s_old && r0 > 0) {
    // existing rows: 16 bytes (128 / BITS codes) per lane step
    constexpr int N = 128 / BITS;
    for (int o = lane * 16; o < r0 * row_b; o += 64 * 16) {
      float old[N];
      load_codes<BITS>(*reinterpret_cast<const u32x4*>(dst + o), old);
      int q[N];
#pragma unroll
      for (int e = 0; e < N; ++e) q[e] = encode_one<BITS>(old[e] * s_old, s_new, r_new);
      store_codes<BITS, N>(dst + o, q);
    }
  }
  for (int c = lane; c < k * ch; c += 64) {
    const int i = c / ch;
    int q[E];
    if (s_new > 0.f) {
      float x[E];
      Unpack<T>::run(*reinterpret_cast<const u32x4*>(src + (t + i) * stride + (c % ch) * 16), x);
#pragma unroll
      for (int e = 0; e < E; ++e) q[e] = encode_one<BITS>(x[e], s_new, r_new);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) q[e] = 0;
    }
    store_codes<BITS, E>(dst + static_cast<int64_t>(r0 + i) * row_b + (c % ch) * E * BITS / 8, q);
  }
  if (lane == 0) scale[tix] = s_new;
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" pkv_status pkv_reshape_and_cache(const void* key, const void* value, void* k_cache,
                                            void* v_cache, const int32_t* slot_mapping,
                                            int32_t num_tokens, int64_t key_stride,
                                            int64_t value_stride, int32_t num_kv_heads,
                                            int32_t head_dim, int32_t block_size,
                                            int32_t num_blocks, pkv_dtype dtype, void* stream) {
  PKV_GUARD({
    const int eb = dtype_bytes(dtype);
    if (dtype != PKV_F32 && dtype != PKV_F16 && dtype != PKV_BF16)
      return fail(PKV_ERR_UNSUPPORTED, "reshape_and_cache: dtype %s not supported",
                  dtype_name(dtype));
    if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        num_blocks <= 0)
      return fail(PKV_ERR_INVALID, "reshape_and_cache: bad sizes");
    if (num_tokens == 0) return PKV_OK;
    if (!key || !value || !k_cache || !v_cache || !slot_mapping)
      return fail(PKV_ERR_INVALID, "reshape_and_cache: NULL pointer");
    const int head_bytes = head_dim * eb;
    if (head_bytes % 16 != 0)
      return fail(PKV_ERR_UNSUPPORTED, "reshape_and_cache: head_dim * element size must be a "
                                       "multiple of 16 bytes");
    if (key_stride == 0) key_stride = static_cast<int64_t>(num_kv_heads) * head_dim;
    if (value_stride == 0) value_stride = static_cast<int64_t>(num_kv_heads) * head_dim;
    if (key_stride < static_cast<int64_t>(num_kv_heads) * head_dim ||
        value_stride < static_cast<int64_t>(num_kv_heads) * head_dim)
      return fail(PKV_ERR_INVALID, "reshape_and_cache: row stride shorter than a row");
    if ((key_stride * eb) % 16 || (value_stride * eb) % 16 || !aligned(key, 16) ||
        !aligned(value, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
      return fail(PKV_ERR_INVALID, "reshape_and_cache: pointers and strides must be 16-byte "
                                   "aligned");
    const int64_t num_slots = static_cast<int64_t>(num_blocks) * block_size;
    if (deep_validation()) {
      std::vector<int32_t> s;
      pkv_status st = fetch_i32(slot_mapping, num_tokens, stream, s);
      if (st) return st;
      std::unordered_set<int32_t> seen;
      for (int32_t i = 0; i < num_tokens; ++i) {
        if (s[i] < 0) continue;
        if (s[i] >= num_slots)
          return fail(PKV_ERR_INVALID, "slot_mapping[%d] = %d outside the pool (%lld slots)", i,
                      s[i], (long long)num_slots);
        if (!seen.insert(s[i]).second)
          return fail(PKV_ERR_INVALID, "slot %d appears twice in slot_mapping", s[i]);
      }
    }
    hipLaunchKernelGGL(reshape_and_cache_kernel, dim3(num_tokens), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(key),
                       static_cast<const uint8_t*>(value), static_cast<uint8_t*>(k_cache),
                       static_cast<uint8_t*>(v_cache), slot_mapping, key_stride * eb,
                       value_stride * eb, num_kv_heads, head_bytes, block_size, num_slots);
    PKV_LAUNCH_CHECK("reshape_and_cache");
    return PKV_OK;
  })
}

namespace {

// Quantise-on-write into int8 (BITS 8) or 4-bit (BITS 4) pools.
pkv_status reshape_and_cache_quant(const char* who, int bits, const void* key, const void* value,
                                   pkv_dtype src_dtype, uint8_t* k_codes, uint8_t* v_codes,
                                   float* k_scale, float* v_scale, const int32_t* slot_mapping,
                                   int32_t num_tokens, int64_t key_stride, int64_t value_stride,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                   int32_t num_blocks, void* stream) {
  if (src_dtype != PKV_F32 && src_dtype != PKV_F16 && src_dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "%s: source dtype %s (f32, f16 or bf16)", who,
                dtype_name(src_dtype));
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      num_blocks <= 0)
    return fail(PKV_ERR_INVALID, "%s: bad sizes", who);
  // a stored row is whole 16-byte chunks
  const int dim_step = bits == 8 ? 16 : 32;
  if (head_dim % dim_step != 0)
    return fail(PKV_ERR_UNSUPPORTED, "%s: head_dim must be a multiple of %d", who, dim_step);
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !k_codes || !v_codes || !k_scale || !v_scale || !slot_mapping)
    return fail(PKV_ERR_INVALID, "%s: NULL pointer", who);
  const int eb = dtype_bytes(src_dtype);
  if (key_stride == 0) key_stride = static_cast<int64_t>(num_kv_heads) * head_dim;
  if (value_stride == 0) value_stride = static_cast<int64_t>(num_kv_heads) * head_dim;
  if (key_stride < static_cast<int64_t>(num_kv_heads) * head_dim ||
      value_stride < static_cast<int64_t>(num_kv_heads) * head_dim)
    return fail(PKV_ERR_INVALID, "%s: row stride shorter than a row", who);
  if ((key_stride * eb) % 16 || (value_stride * eb) % 16 || !aligned(key, 16) ||
      !aligned(value, 16) || !aligned(k_codes, 16) || !aligned(v_codes, 16))
    return fail(PKV_ERR_INVALID, "%s: pointers and strides must be 16-byte aligned", who);
  const int64_t num_slots = static_cast<int64_t>(num_blocks) * block_size;
  if (deep_validation()) {
    std::vector<int32_t> s;
    pkv_status st = fetch_i32(slot_mapping, num_tokens, stream, s);
    if (st) return st;
    std::unordered_set<int32_t> seen, run_blocks;
    for (int32_t i = 0; i < num_tokens; ++i) {
      if (s[i] < 0) continue;
      if (s[i] >= num_slots)
        return fail(PKV_ERR_INVALID, "slot_mapping[%d] = %d outside the pool (%lld slots)", i,
                    s[i], (long long)num_slots);
      if (!seen.insert(s[i]).second)
        return fail(PKV_ERR_INVALID, "slot %d appears twice in slot_mapping", s[i]);
      const bool leads = !(i > 0 && s[i] % block_size > 0 && s[i - 1] == s[i] - 1);
      if (leads && !run_blocks.insert(s[i] / block_size).second)
        return fail(PKV_ERR_INVALID, "%s: block %d gets two runs of rows in one call", who,
                    s[i] / block_size);
    }
  }
  const int64_t waves = static_cast<int64_t>(num_tokens) * num_kv_heads * 2;
  const int64_t wgs = (waves + kThreads / 64 - 1) / (kThreads / 64);
  if (wgs > 0x7fffffff) return fail(PKV_ERR_UNSUPPORTED, "%s: too many tokens", who);
  auto launch = [&](auto tag, auto width) {
    using T = decltype(tag);
    hipLaunchKernelGGL((reshape_and_cache_quant_kernel<T, decltype(width)::value>),
                       dim3(static_cast<unsigned>(wgs)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(key),
                       static_cast<const uint8_t*>(value), k_codes, v_codes, k_scale, v_scale,
                       slot_mapping, num_tokens, key_stride * eb, value_stride * eb,
                       num_kv_heads, head_dim, block_size, num_slots);
  };
  auto by_source = [&](auto width) {
    if (src_dtype == PKV_BF16)
      launch(BF16{}, width);
    else if (src_dtype == PKV_F16)
      launch(F16{}, width);
    else
      launch(F32{}, width);
  };
  if (bits == 8)
    by_source(std::integral_constant<int, 8>{});
  else
    by_source(std::integral_constant<int, 4>{});
  PKV_LAUNCH_CHECK(who);
  return PKV_OK;
}

// Whole-block encoding into int8 (BITS 8) or 4-bit (BITS 4) pools.
pkv_status quantize_blocks_impl(const char* who, int bits, const void* src_k, const void* src_v,
                                pkv_dtype src_dtype, uint8_t* dst_k, uint8_t* dst_v,
                                float* k_scale, float* v_scale, const int32_t* blocks,
                                const int32_t* filled, int32_t num_listed, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                void* stream) {
  if (src_dtype != PKV_F32 && src_dtype != PKV_F16 && src_dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "%s: source dtype %s (f32, f16 or bf16)", who,
                dtype_name(src_dtype));
  if (num_listed < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      num_blocks <= 0)
    return fail(PKV_ERR_INVALID, "%s: bad sizes", who);
  if (num_listed == 0) return PKV_OK;
  if (!src_k || !src_v || !dst_k || !dst_v || !k_scale || !v_scale || !blocks || !filled)
    return fail(PKV_ERR_INVALID, "%s: NULL pointer", who);
  const int eb = dtype_bytes(src_dtype);
  if ((head_dim * eb) % 16 != 0)
    return fail(PKV_ERR_UNSUPPORTED, "%s: head_dim * element size must be a multiple of 16",
                who);
  // a 16-byte source chunk becomes 8 (16-bit source) or 4 (fp32) int8
  // codes, or half as many bytes of 4-bit codes
  const size_t dst_align = static_cast<size_t>(16 / eb) * bits / 8;
  if (!aligned(src_k, 16) || !aligned(src_v, 16) || !aligned(dst_k, dst_align) ||
      !aligned(dst_v, dst_align))
    return fail(PKV_ERR_INVALID, "%s: pools must be 16-byte (source) / %zu-byte (codes) aligned",
                who, dst_align);
  if (static_cast<int64_t>(num_listed) * num_kv_heads * 2 > 0x7fffffffLL)
    return fail(PKV_ERR_UNSUPPORTED, "%s: too many tiles", who);
  if (deep_validation()) {
    std::vector<int32_t> bl, fl;
    pkv_status st = fetch_i32(blocks, num_listed, stream, bl);
    if (st) return st;
    st = fetch_i32(filled, num_listed, stream, fl);
    if (st) return st;
    std::unordered_set<int32_t> seen;
    for (int32_t i = 0; i < num_listed; ++i) {
      if (bl[i] < 0 || bl[i] >= num_blocks)
        return fail(PKV_ERR_INVALID, "%s: blocks[%d] = %d outside the pool", who, i, bl[i]);
      if (fl[i] < 0 || fl[i] > block_size)
        return fail(PKV_ERR_INVALID, "%s: filled[%d] = %d outside [0, %d]", who, i, fl[i],
                    block_size);
      if (!seen.insert(bl[i]).second)
        return fail(PKV_ERR_INVALID, "%s: block %d listed twice", who, bl[i]);
    }
  }
  const int64_t tiles = static_cast<int64_t>(num_listed) * num_kv_heads * 2;
  const dim3 grid(static_cast<unsigned>((tiles + 3) / 4));
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint8_t* sk = static_cast<const uint8_t*>(src_k);
  const uint8_t* sv = static_cast<const uint8_t*>(src_v);
  auto launch = [&](auto tag, auto width) {
    hipLaunchKernelGGL((quantize_blocks_kernel<decltype(tag), decltype(width)::value>), grid,
                       dim3(kThreads), 0, st, sk, sv, dst_k, dst_v, k_scale, v_scale, blocks,
                       filled, num_listed, num_kv_heads, head_dim, block_size, num_blocks);
  };
  auto by_source = [&](auto width) {
    if (src_dtype == PKV_BF16)
      launch(BF16{}, width);
    else if (src_dtype == PKV_F16)
      launch(F16{}, width);
    else
      launch(F32{}, width);
  };
  if (bits == 8)
    by_source(std::integral_constant<int, 8>{});
  else
    by_source(std::integral_constant<int, 4>{});
  PKV_LAUNCH_CHECK(who);
  return PKV_OK;
}

}  // namespace

extern "C" pkv_status pkv_reshape_and_cache_int8(
    const void* key, const void* value, pkv_dtype src_dtype, int8_t* k_codes, int8_t* v_codes,
    float* k_scale, float* v_scale, const int32_t* slot_mapping, int32_t num_tokens,
    int64_t key_stride, int64_t value_stride, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t num_blocks, void* stream) {
  PKV_GUARD({
    return reshape_and_cache_quant("reshape_and_cache_int8", 8, key, value, src_dtype,
                                   reinterpret_cast<uint8_t*>(k_codes),
                                   reinterpret_cast<uint8_t*>(v_codes), k_scale, v_scale,
                                   slot_mapping, num_tokens, key_stride, value_stride,
                                   num_kv_heads, head_dim, block_size, num_blocks, stream);
  })
}

extern "C" pkv_status pkv_reshape_and_cache_int4(
    const void* key, const void* value, pkv_dtype src_dtype, uint8_t* k_codes, uint8_t* v_codes,
    float* k_scale, float* v_scale, const int32_t* slot_mapping, int32_t num_tokens,
    int64_t key_stride, int64_t value_stride, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t num_blocks, void* stream) {
  PKV_GUARD({
    return reshape_and_cache_quant("reshape_and_cache_int4", 4, key, value, src_dtype, k_codes,
                                   v_codes, k_scale, v_scale, slot_mapping, num_tokens,
                                   key_stride, value_stride, num_kv_heads, head_dim, block_size,
                                   num_blocks, stream);
  })
}

extern "C" pkv_status pkv_copy_blocks(void* k_cache, void* v_cache, float* k_scale,
                                      float* v_scale, const int32_t* pairs, int32_t num_pairs,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                      int32_t num_blocks, pkv_dtype dtype, void* stream) {
  PKV_GUARD({
    const int eb = dtype_bytes(dtype);
    if (eb == 0) return fail(PKV_ERR_INVALID, "copy_blocks: unknown dtype");
    if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        num_blocks <= 0)
      return fail(PKV_ERR_INVALID, "copy_blocks: bad sizes");
    if (num_pairs == 0) return PKV_OK;
    if (!k_cache || !v_cache || !pairs) return fail(PKV_ERR_INVALID, "copy_blocks: NULL pointer");
    if (has_scales(dtype) && (!k_scale || !v_scale))
      return fail(PKV_ERR_INVALID, "copy_blocks: %s storage needs k_scale and v_scale",
                  dtype_name(dtype));
    if (dtype == PKV_I4 && head_dim % 2)
      return fail(PKV_ERR_INVALID, "copy_blocks: 4-bit rows need an even head_dim");
    if (num_kv_heads > 256) return fail(PKV_ERR_UNSUPPORTED, "copy_blocks: > 256 kv heads");
    const int64_t block_bytes =
        static_cast<int64_t>(num_kv_heads) * block_size * row_bytes(dtype, head_dim);
    if (block_bytes % 16 || !aligned(k_cache, 16) || !aligned(v_cache, 16))
      return fail(PKV_ERR_INVALID, "copy_blocks: blocks must be 16-byte multiples and aligned");
    if (deep_validation()) {
      std::vector<int32_t> p;
      pkv_status st = fetch_i32(pairs, static_cast<size_t>(num_pairs) * 2, stream, p);
      if (st) return st;
      std::unordered_set<int32_t> srcs, dsts;
      for (int32_t i = 0; i < num_pairs; ++i) {
        if (p[2 * i] < 0 || p[2 * i] >= num_blocks || p[2 * i + 1] < 0 ||
            p[2 * i + 1] >= num_blocks)
          return fail(PKV_ERR_INVALID, "copy pair %d (%d -> %d) outside the pool", i, p[2 * i],
                      p[2 * i + 1]);
        srcs.insert(p[2 * i]);
        if (!dsts.insert(p[2 * i + 1]).second)
          return fail(PKV_ERR_INVALID, "block %d is the destination of two pairs", p[2 * i + 1]);
      }
      for (int32_t d : dsts)
        if (srcs.count(d))
          return fail(PKV_ERR_INVALID, "block %d is both a source and a destination", d);
    }
    const int64_t chunks = (block_bytes + kCopyChunkBytes - 1) / kCopyChunkBytes;
    if (chunks > 65535) return fail(PKV_ERR_UNSUPPORTED, "copy_blocks: blocks too large");
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(num_pairs, 2, static_cast<unsigned>(chunks)),
                       dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache),
                       has_scales(dtype) ? k_scale : nullptr, has_scales(dtype) ? v_scale : nullptr,
                       pairs, block_bytes, num_kv_heads, num_blocks);
    PKV_LAUNCH_CHECK("copy_blocks");
    return PKV_OK;
  })
}

extern "C" pkv_status pkv_quantize_blocks(const void* src_k, const void* src_v,
                                          pkv_dtype src_dtype, int8_t* dst_k, int8_t* dst_v,
                                          float* k_scale, float* v_scale, const int32_t* blocks,
                                          const int32_t* filled, int32_t num_listed,
                                          int32_t num_kv_heads, int32_t head_dim,
                                          int32_t block_size, int32_t num_blocks, void* stream) {
  PKV_GUARD({
    return quantize_blocks_impl("quantize_blocks", 8, src_k, src_v, src_dtype,
                                reinterpret_cast<uint8_t*>(dst_k),
                                reinterpret_cast<uint8_t*>(dst_v), k_scale, v_scale, blocks,
                                filled, num_listed, num_kv_heads, head_dim, block_size,
                                num_blocks, stream);
  })
}

extern "C" pkv_status pkv_quantize_blocks_int4(const void* src_k, const void* src_v,
                                               pkv_dtype src_dtype, uint8_t* dst_k,
                                               uint8_t* dst_v, float* k_scale, float* v_scale,
                                               const int32_t* blocks, const int32_t* filled,
                                               int32_t num_listed, int32_t num_kv_heads,
                                               int32_t head_dim, int32_t block_size,
                                               int32_t num_blocks, void* stream) {
  PKV_GUARD({
    return quantize_blocks_impl("quantize_blocks_int4", 4, src_k, src_v, src_dtype, dst_k, dst_v,
                                k_scale, v_scale, blocks, filled, num_listed, num_kv_heads,
                                head_dim, block_size, num_blocks, stream);
  })
}

// swap_blocks.  Device <-> host swaps go through the DMA engines in
// contiguous runs: with a workspace, the scattered device blocks are first
// gathered into it (or scattered from it) by a copy kernel at HBM speed, so
// the PCIe side moves long runs; without one, each run of consecutive pairs
// is one copy.  Device <-> device swaps run the copy kernel directly.
namespace {

// Process-wide swap counters for the swap-rate health metric
// (cnnetsun.cn "别再让GPU内存拖后腿了…" §4.2 lists page swaps per second,
// with frequent swapping a sign that pages are too small).
struct SwapCounters {
  std::atomic<int64_t> calls{0}, to_host{0}, to_device{0}, device_to_device{0}, host_to_host{0},
      bytes{0};
};
SwapCounters& swap_counters() {
  static SwapCounters c;
  return c;
}

bool is_device_memory(const void* p) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();   // pageable host memory is unknown to the runtime
    return false;
  }
  return attr.type == hipMemoryTypeDevice;
}

}  // namespace

extern "C" size_t pkv_swap_workspace_bytes(int32_t max_pairs, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t block_size,
                                           pkv_dtype dtype) {
  const int eb = dtype_bytes(dtype);
  if (max_pairs <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || eb == 0)
    return 0;
  const size_t bb = static_cast<size_t>(num_kv_heads) * block_size * row_bytes(dtype, head_dim);
  const size_t per = 2 * bb + (has_scales(dtype) ? 2 * sizeof(float) * num_kv_heads : 0);
  return 256 + static_cast<size_t>(max_pairs) * (sizeof(int32_t) + per + 64);
}

extern "C" pkv_status pkv_swap_blocks(void* dst_k, void* dst_v, float* dst_k_scale,
                                      float* dst_v_scale, int32_t dst_num_blocks,
                                      const void* src_k, const void* src_v,
                                      const float* src_k_scale, const float* src_v_scale,
                                      int32_t src_num_blocks, const int32_t* pairs,
                                      int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, pkv_dtype dtype, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  PKV_GUARD({
    const char* who = "swap_blocks";
    const int eb = dtype_bytes(dtype);
    if (eb == 0) return fail(PKV_ERR_INVALID, "%s: unknown dtype", who);
    if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        dst_num_blocks <= 0 || src_num_blocks <= 0)
      return fail(PKV_ERR_INVALID, "%s: bad sizes", who);
    if (num_pairs == 0) return PKV_OK;
    if (!dst_k || !dst_v || !src_k || !src_v || !pairs)
      return fail(PKV_ERR_INVALID, "%s: NULL pointer", who);
    const bool scales = has_scales(dtype);
    if (scales && (!dst_k_scale || !dst_v_scale || !src_k_scale || !src_v_scale))
      return fail(PKV_ERR_INVALID, "%s: %s pools need all four scale arrays", who,
                  dtype_name(dtype));
    if (dtype == PKV_I4 && head_dim % 2)
      return fail(PKV_ERR_INVALID, "%s: 4-bit rows need an even head_dim", who);
    std::unordered_set<int32_t> seen_dst;
    for (int32_t i = 0; i < num_pairs; ++i) {
      const int32_t s_ = pairs[2 * i], d_ = pairs[2 * i + 1];
      if (s_ < 0 || s_ >= src_num_blocks || d_ < 0 || d_ >= dst_num_blocks)
        return fail(PKV_ERR_INVALID, "%s: pair %d (%d -> %d) outside the pools", who, i, s_, d_);
      if (!seen_dst.insert(d_).second)
        return fail(PKV_ERR_INVALID, "%s: block %d is the destination of two pairs", who, d_);
    }
    const size_t bb = static_cast<size_t>(num_kv_heads) * block_size * row_bytes(dtype, head_dim);
    const size_t sb = static_cast<size_t>(num_kv_heads) * sizeof(float);
    if (bb % 16 != 0 || !aligned(dst_k, 16) || !aligned(dst_v, 16) || !aligned(src_k, 16) ||
        !aligned(src_v, 16))
      return fail(PKV_ERR_INVALID, "%s: pools must be 16-byte aligned with 16-byte blocks", who);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool src_dev = is_device_memory(src_k) && is_device_memory(src_v);
    const bool dst_dev = is_device_memory(dst_k) && is_device_memory(dst_v);
    const int64_t chunks = (static_cast<int64_t>(bb) + kCopyChunkBytes - 1) / kCopyChunkBytes;
    if (chunks > 65535) return fail(PKV_ERR_UNSUPPORTED, "%s: blocks too large", who);

    auto memcpy_runs = [&](void* d_base, const void* s_base, size_t unit, const int32_t* dl,
                           const int32_t* sl, int32_t n, int32_t d_stride, int32_t s_stride) {
      // copies list entries k (dst id dl[k*d_stride] or k, src id sl[k*s_stride] or k),
      // merged into runs where both sides continue
      for (int32_t i = 0; i < n;) {
        const int32_t d0 = dl ? dl[i * d_stride] : i, s0 = sl ? sl[i * s_stride] : i;
        int32_t len = 1;
        while (i + len < n && (dl ? dl[(i + len) * d_stride] : i + len) == d0 + len &&
               (sl ? sl[(i + len) * s_stride] : i + len) == s0 + len)
          ++len;
        const hipError_t e = hipMemcpyAsync(static_cast<char*>(d_base) + unit * d0,
                                            static_cast<const char*>(s_base) + unit * s0,
                                            unit * len, hipMemcpyDefault, st);
        if (e != hipSuccess) return e;
        i += len;
      }
      return hipSuccess;
    };

    hipError_t e = hipSuccess;
    if (src_dev && dst_dev) {
      // both pools on the device: the copy kernel, ids through the workspace
      // when there is one, else one copy per run
      if (workspace && workspace_bytes >= 256 + static_cast<size_t>(num_pairs) * 8 &&
          aligned(workspace, 256)) {
        int32_t* ids = static_cast<int32_t*>(workspace);
        {
          // source ids, then destination ids
          std::vector<int32_t> sd(2 * static_cast<size_t>(num_pairs));
          for (int32_t i = 0; i < num_pairs; ++i) {
            sd[i] = pairs[2 * i];
            sd[num_pairs + i] = pairs[2 * i + 1];
          }
          e = hipMemcpyAsync(ids, sd.data(), sd.size() * sizeof(int32_t), hipMemcpyHostToDevice, st);
          if (e == hipSuccess) {
            hipLaunchKernelGGL(copy_list_kernel, dim3(num_pairs, 2, static_cast<unsigned>(chunks)),
                               dim3(kThreads), 0, st, static_cast<uint8_t*>(dst_k),
                               static_cast<uint8_t*>(dst_v), static_cast<const uint8_t*>(src_k),
                               static_cast<const uint8_t*>(src_v), ids + num_pairs, ids,
                               static_cast<int64_t>(bb));
            e = hipGetLastError();
          }
        }
        if (e == hipSuccess && scales) {
          e = memcpy_runs(dst_k_scale, src_k_scale, sb, pairs + 1, pairs, num_pairs, 2, 2);
          if (e == hipSuccess)
            e = memcpy_runs(dst_v_scale, src_v_scale, sb, pairs + 1, pairs, num_pairs, 2, 2);
        }
      } else {
        e = memcpy_runs(dst_k, src_k, bb, pairs + 1, pairs, num_pairs, 2, 2);
        if (e == hipSuccess) e = memcpy_runs(dst_v, src_v, bb, pairs + 1, pairs, num_pairs, 2, 2);
        if (e == hipSuccess && scales) {
          e = memcpy_runs(dst_k_scale, src_k_scale, sb, pairs + 1, pairs, num_pairs, 2, 2);
          if (e == hipSuccess)
            e = memcpy_runs(dst_v_scale, src_v_scale, sb, pairs + 1, pairs, num_pairs, 2, 2);
        }
      }
    } else if (src_dev != dst_dev && workspace && aligned(workspace, 256)) {
      // device <-> host through staging: per chunk of C pairs, the ids, then
      // C packed K blocks, C packed V blocks (and their scales)
      const size_t per = 2 * bb + (scales ? 2 * sb : 0);
      const size_t avail = workspace_bytes > 256 ? workspace_bytes - 256 : 0;
      int64_t cap = static_cast<int64_t>(avail / (sizeof(int32_t) + per + 64));
      if (cap < 1) return fail(PKV_ERR_INVALID, "%s: workspace smaller than one block", who);
      cap = std::min<int64_t>(cap, num_pairs);
      uint8_t* ws = static_cast<uint8_t*>(workspace);
      int32_t* ids = reinterpret_cast<int32_t*>(ws);
      const size_t ids_bytes = (static_cast<size_t>(cap) * sizeof(int32_t) + 255) / 256 * 256;
      uint8_t* stage_k = ws + ids_bytes;
      uint8_t* stage_v = stage_k + cap * bb;
      float* stage_ks = reinterpret_cast<float*>(stage_v + cap * bb);
      float* stage_vs = stage_ks + cap * num_kv_heads;
      std::vector<int32_t> dev_ids(static_cast<size_t>(cap)), host_ids(static_cast<size_t>(cap));
      for (int32_t start = 0; start < num_pairs && e == hipSuccess; start += cap) {
        const int32_t cnt = static_cast<int32_t>(std::min<int64_t>(cap, num_pairs - start));
        for (int32_t k = 0; k < cnt; ++k) {
          const int32_t s_ = pairs[2 * (start + k)], d_ = pairs[2 * (start + k) + 1];
          dev_ids[k] = src_dev ? s_ : d_;
          host_ids[k] = src_dev ? d_ : s_;
        }
        e = hipMemcpyAsync(ids, dev_ids.data(), cnt * sizeof(int32_t), hipMemcpyHostToDevice, st);
        if (e != hipSuccess) break;
        const dim3 grid(cnt, 2, static_cast<unsigned>(chunks));
        if (src_dev) {
          // gather on the device, then long runs over PCIe
          hipLaunchKernelGGL(copy_list_kernel, grid, dim3(kThreads), 0, st, stage_k, stage_v,
                             static_cast<const uint8_t*>(src_k), static_cast<const uint8_t*>(src_v),
                             nullptr, ids, static_cast<int64_t>(bb));
          e = hipGetLastError();
          if (e == hipSuccess && scales) {
            e = memcpy_runs(stage_ks, src_k_scale, sb, nullptr, dev_ids.data(), cnt, 1, 1);
            if (e == hipSuccess)
              e = memcpy_runs(stage_vs, src_v_scale, sb, nullptr, dev_ids.data(), cnt, 1, 1);
          }
          if (e == hipSuccess)
            e = memcpy_runs(dst_k, stage_k, bb, host_ids.data(), nullptr, cnt, 1, 1);
          if (e == hipSuccess)
            e = memcpy_runs(dst_v, stage_v, bb, host_ids.data(), nullptr, cnt, 1, 1);
          if (e == hipSuccess && scales) {
            e = memcpy_runs(dst_k_scale, stage_ks, sb, host_ids.data(), nullptr, cnt, 1, 1);
            if (e == hipSuccess)
              e = memcpy_runs(dst_v_scale, stage_vs, sb, host_ids.data(), nullptr, cnt, 1, 1);
          }
        } else {
          // long runs over PCIe into staging, then scatter on the device
          e = memcpy_runs(stage_k, src_k, bb, nullptr, host_ids.data(), cnt, 1, 1);
          if (e == hipSuccess) e = memcpy_runs(stage_v, src_v, bb, nullptr, host_ids.data(), cnt, 1, 1);
          if (e == hipSuccess && scales) {
            e = memcpy_runs(stage_ks, src_k_scale, sb, nullptr, host_ids.data(), cnt, 1, 1);
            if (e == hipSuccess)
              e = memcpy_runs(stage_vs, src_v_scale, sb, nullptr, host_ids.data(), cnt, 1, 1);
          }
          if (e == hipSuccess) {
            hipLaunchKernelGGL(copy_list_kernel, grid, dim3(kThreads), 0, st,
                               static_cast<uint8_t*>(dst_k), static_cast<uint8_t*>(dst_v),
                               stage_k, stage_v, ids, nullptr, static_cast<int64_t>(bb));
            e = hipGetLastError();
          }
          if (e == hipSuccess && scales) {
            e = memcpy_runs(dst_k_scale, stage_ks, sb, dev_ids.data(), nullptr, cnt, 1, 1);
            if (e == hipSuccess)
              e = memcpy_runs(dst_v_scale, stage_vs, sb, dev_ids.data(), nullptr, cnt, 1, 1);
          }
        }
        // the host-side id vectors are reused by the next chunk: the copies
        // above read them at call time (pageable sources are staged by the
        // runtime before hipMemcpyAsync returns)
      }
    } else {
      e = memcpy_runs(dst_k, src_k, bb, pairs + 1, pairs, num_pairs, 2, 2);
      if (e == hipSuccess) e = memcpy_runs(dst_v, src_v, bb, pairs + 1, pairs, num_pairs, 2, 2);
      if (e == hipSuccess && scales) {
        e = memcpy_runs(dst_k_scale, src_k_scale, sb, pairs + 1, pairs, num_pairs, 2, 2);
        if (e == hipSuccess)
          e = memcpy_runs(dst_v_scale, src_v_scale, sb, pairs + 1, pairs, num_pairs, 2, 2);
      }
    }
    if (e != hipSuccess)
      return fail(PKV_ERR_DEVICE, "%s: copy failed: %s", who, hipGetErrorString(e));
    SwapCounters& sc = swap_counters();
    sc.calls.fetch_add(1);
    (src_dev && !dst_dev   ? sc.to_host
     : !src_dev && dst_dev ? sc.to_device
     : src_dev             ? sc.device_to_device
                           : sc.host_to_host).fetch_add(num_pairs);
    sc.bytes.fetch_add(static_cast<int64_t>(num_pairs) * 2 * (bb + (scales ? sb : 0)));
    return PKV_OK;
  })
}

extern "C" pkv_status pkv_swap_stats_get(pkv_swap_stats* out, int32_t reset) {
  if (!out) return fail(PKV_ERR_INVALID, "swap_stats: out is NULL");
  SwapCounters& sc = swap_counters();
  auto take = [&](std::atomic<int64_t>& c) { return reset ? c.exchange(0) : c.load(); };
  out->calls = take(sc.calls);
  out->blocks_to_host = take(sc.to_host);
  out->blocks_to_device = take(sc.to_device);
  out->blocks_device_to_device = take(sc.device_to_device);
  out->blocks_host_to_host = take(sc.host_to_host);
  out->bytes = take(sc.bytes);
  return PKV_OK;
}

