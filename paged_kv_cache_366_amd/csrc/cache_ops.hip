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
