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
#include <unordered_set>

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

// Int8 storage of whole blocks: one wavefront per (listed block, KV head,
// K or V) tile.  The first pass takes max |x| over the filled rows, the
// second writes the codes (from registers for tiles up to 4 KiB); every
// step is the float32 arithmetic of the encoding: s = a / 127, code =
// rint(x / s) clamped to [-127, 127], rows past the filled count 0, a
// subnormal scale counting as zero.
constexpr float kSmallestNormal = 1.17549435e-38f;

__device__ __forceinline__ float wave_absmax(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void quantize_blocks_kernel(
    const uint8_t* __restrict__ src_k, const uint8_t* __restrict__ src_v,
    int8_t* __restrict__ dst_k, int8_t* __restrict__ dst_v, float* __restrict__ ks,
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
  int8_t* dst = (which ? dst_v : dst_k) + tix * elems;
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
  float sc = amax / 127.f;
  if (!(sc >= kSmallestNormal)) sc = 0.f;

  auto encode = [&](int c, const u32x4& w) {
    int8_t q[E];
    if (c < filled_chunks && sc > 0.f) {
      float x[E];
      Unpack<T>::run(w, x);
#pragma unroll
      for (int e = 0; e < E; ++e)
        q[e] = static_cast<int8_t>(fminf(fmaxf(rintf(x[e] / sc), -127.f), 127.f));
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) q[e] = 0;
    }
    int8_t* d = dst + static_cast<int64_t>(c) * E;
    if constexpr (E == 8) {
      *reinterpret_cast<uint64_t*>(d) = __builtin_bit_cast(uint64_t, q);
    } else {
      *reinterpret_cast<uint32_t*>(d) = __builtin_bit_cast(uint32_t, q);
    }
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
    if (dtype == PKV_I8 && (!k_scale || !v_scale))
      return fail(PKV_ERR_INVALID, "copy_blocks: int8 storage needs k_scale and v_scale");
    if (num_kv_heads > 256) return fail(PKV_ERR_UNSUPPORTED, "copy_blocks: > 256 kv heads");
    const int64_t block_bytes = static_cast<int64_t>(num_kv_heads) * block_size * head_dim * eb;
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
                       dtype == PKV_I8 ? k_scale : nullptr, dtype == PKV_I8 ? v_scale : nullptr,
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
    const char* who = "quantize_blocks";
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
    if (!aligned(src_k, 16) || !aligned(src_v, 16) || !aligned(dst_k, 8) || !aligned(dst_v, 8))
      return fail(PKV_ERR_INVALID, "%s: pools must be 16-byte (source) / 8-byte (int8) aligned",
                  who);
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
    auto launch = [&](auto tag) {
      hipLaunchKernelGGL(quantize_blocks_kernel<decltype(tag)>, grid, dim3(kThreads), 0, st, sk,
                         sv, dst_k, dst_v, k_scale, v_scale, blocks, filled, num_listed,
                         num_kv_heads, head_dim, block_size, num_blocks);
    };
    if (src_dtype == PKV_BF16)
      launch(BF16{});
    else if (src_dtype == PKV_F16)
      launch(F16{});
    else
      launch(F32{});
    PKV_LAUNCH_CHECK("quantize_blocks");
    return PKV_OK;
  })
}
