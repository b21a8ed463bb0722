// C entry points of paged attention: argument checks, workspace layout and
// the choice between the wavefront and matrix-core kernels.
#include <algorithm>
#include <atomic>
#include <climits>
#include <cmath>
#include <vector>

#include "attention_common.h"
#include "host_checks.h"
#include "partition.h"

namespace pkv {
pkv_status launch_decode_wave(const AttnArgs& a, pkv_dtype q_dt, pkv_dtype kv_dt, int D,
                              int group, hipStream_t st);
pkv_status launch_reduce(const AttnArgs& a, int D, hipStream_t st);
pkv_status launch_decode_mfma(const AttnArgs& a, pkv_dtype q_dt, pkv_dtype kv_dt, int D,
                              int group, hipStream_t st);
pkv_status launch_prefill_mfma(const AttnArgs& a, pkv_dtype q_dt, int D, int group,
                               int max_query_len, hipStream_t st);
pkv_status decode_wave_occupancy(pkv_dtype q_dt, pkv_dtype kv_dt, int D, int group,
                                 int part_tokens, bool nt, int* wg_per_cu, int* heads_per_wg,
                                 int* min_part_tokens);
pkv_status decode_mfma_occupancy(pkv_dtype q_dt, pkv_dtype kv_dt, int D, bool nt, int* wg_per_cu);
int prefill_tile_rows();
}  // namespace pkv

using namespace pkv;

namespace {

constexpr size_t kAlign = 256;
// Shortest partition the automatic choice takes: below it each workgroup's
// start (table entries, q) and partial-state write outweigh its keys.
constexpr int32_t kMinAutoPartition = 256;
// Prefill workgroups per compute unit the partition choice fills: a unit
// holds up to four (two LDS stages), but past two the per-step time rises
// more than the added workgroups bring (4 long documents, 16,384 keys
// each: 512 workgroups 197 us, 768 210 us, 1,024 215 us).
constexpr int kPrefillPerCu = 2;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int num_partitions(int32_t max_ctx, int32_t part_tokens) {
  if (part_tokens <= 0) return 1;
  int64_t p = (static_cast<int64_t>(max_ctx) + part_tokens - 1) / part_tokens;
  return static_cast<int>(std::max<int64_t>(p, 1));
}

struct WsLayout {
  size_t o_bytes = 0, ml_bytes = 0, total = 0;
};

WsLayout workspace_layout(int64_t rows, int64_t hq, int64_t D, int parts) {
  WsLayout w;
  if (parts <= 1) return w;
  w.o_bytes = align_up(static_cast<size_t>(rows * hq * parts * D) * sizeof(float));
  w.ml_bytes = align_up(static_cast<size_t>(rows * hq * parts * 2) * sizeof(float));
  w.total = w.o_bytes + w.ml_bytes;
  return w;
}

// Decode-step workspace: the split-K layout above, then one int32 arrival
// counter per (row, query head) for the in-kernel merge.
size_t counter_bytes(int64_t rows, int64_t hq, int parts) {
  return parts > 1 ? align_up(static_cast<size_t>(rows * hq) * sizeof(int32_t)) : 0;
}

int out_kind_of(pkv_dtype out_dt) {
  return out_dt == PKV_F32 ? kOutF32 : out_dt == PKV_BF16 ? kOutBF16 : kOutF16;
}

// Block sizes the kernels walk as 1, 2, 4 or 8 tiles of 16 rows ([cnnetsun]
// §2.1 and §4.3 name page sizes from 16 to 128): log2(block_size / 16), or
// -1 for any other size.
int block_shift(int32_t bs) {
  switch (bs) {
    case 16: return 0;
    case 32: return 1;
    case 64: return 2;
    case 128: return 3;
    default: return -1;
  }
}

// Shared checks of decode and prefill arguments.
pkv_status check_common(const char* who, void* out, pkv_dtype out_dt, const void* q,
                        pkv_dtype q_dt, const void* kc, const void* vc, pkv_dtype kv_dt,
                        const float* ks, const float* vs, const int32_t* tables, int32_t mb,
                        const int32_t* lens, int32_t max_ctx, int32_t S, int32_t rows,
                        int32_t hq, int32_t hkv, int32_t D, int32_t bs, int32_t nb, float scale) {
  if (S < 0 || hq <= 0 || hkv <= 0 || nb <= 0 || mb < 0 || max_ctx < 0)
    return fail(PKV_ERR_INVALID, "%s: bad sizes (S=%d Hq=%d Hkv=%d NB=%d MB=%d max_ctx=%d)", who,
                S, hq, hkv, nb, mb, max_ctx);
  if (hq % hkv != 0)
    return fail(PKV_ERR_INVALID, "%s: num_q_heads %d is not a multiple of num_kv_heads %d", who,
                hq, hkv);
  if (D != 64 && D != 128) return fail(PKV_ERR_UNSUPPORTED, "%s: head_dim %d (64 or 128)", who, D);
  if (block_shift(bs) < 0)
    return fail(PKV_ERR_UNSUPPORTED, "%s: block_size %d (16, 32, 64 or 128)", who, bs);
  if (static_cast<int64_t>(max_ctx) > static_cast<int64_t>(mb) * bs)
    return fail(PKV_ERR_INVALID, "%s: max_context_len %d exceeds max_blocks_per_seq * block_size",
                who, max_ctx);
  if (q_dt != PKV_F32 && q_dt != PKV_F16 && q_dt != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "%s: q dtype %s", who, dtype_name(q_dt));
  if (kv_dt != q_dt && !has_scales(kv_dt))
    return fail(PKV_ERR_UNSUPPORTED, "%s: kv dtype %s with q dtype %s", who, dtype_name(kv_dt),
                dtype_name(q_dt));
  if (out_dt != PKV_F32 && out_dt != q_dt)
    return fail(PKV_ERR_UNSUPPORTED, "%s: out dtype must be f32 or the q dtype", who);
  if (has_scales(kv_dt) && (!ks || !vs))
    return fail(PKV_ERR_INVALID, "%s: %s KV needs k_scale and v_scale", who, dtype_name(kv_dt));
  if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID, "%s: scale is not finite", who);
  // q and out are read only when there are query rows (a prefill batch may
  // hold sequences whose chunks are all empty)
  if ((rows > 0 && (!out || !q)) || (S > 0 && (!kc || !vc || !tables || !lens)))
    return fail(PKV_ERR_INVALID, "%s: NULL pointer", who);
  if (!aligned(kc, 16) || !aligned(vc, 16) || !aligned(q, 16) || !aligned(out, 4))
    return fail(PKV_ERR_INVALID, "%s: q, k_cache and v_cache must be 16-byte aligned", who);
  return PKV_OK;
}

// PKV_VALIDATE=1: lengths within bounds, and every table entry a sequence
// reads names a block of the pool.
pkv_status deep_check_tables(const char* who, const int32_t* tables, int32_t mb,
                             const int32_t* lens, int32_t max_ctx, int32_t S, int32_t nb,
                             int32_t bs, void* stream, std::vector<int32_t>* lens_out = nullptr) {
  std::vector<int32_t> L, T;
  pkv_status st = fetch_i32(lens, S, stream, L);
  if (st) return st;
  st = fetch_i32(tables, static_cast<size_t>(S) * mb, stream, T);
  if (st) return st;
  for (int32_t s = 0; s < S; ++s) {
    if (L[s] < 0 || L[s] > max_ctx)
      return fail(PKV_ERR_INVALID, "%s: context_lens[%d] = %d outside [0, %d]", who, s, L[s],
                  max_ctx);
    for (int32_t j = 0; j < (L[s] + bs - 1) / bs; ++j) {
      int32_t b = T[static_cast<size_t>(s) * mb + j];
      if (b < 0 || b >= nb)
        return fail(PKV_ERR_INVALID, "%s: block_tables[%d][%d] = %d outside the pool", who, s, j,
                    b);
    }
  }
  if (lens_out) *lens_out = std::move(L);
  return PKV_OK;
}

bool use_mfma(int32_t algo, pkv_dtype q_dt, int group) {
  const bool able = (q_dt == PKV_BF16 || q_dt == PKV_F16) && group <= 16;
  if (algo == PKV_ALGO_MFMA) return able;
  if (algo == PKV_ALGO_WAVE) return false;
  return able && group >= 4;
}

// kStep: one launch of the main kernel that also appends the step's new K/V
// rows (when given) and merges split rows itself (counters in the workspace).
enum class DecodePart { kAll, kMain, kReduce, kStep };

pkv_status decode_impl(DecodePart which, void* out, pkv_dtype out_dt, const void* q,
                       pkv_dtype q_dt, const void* kc, const void* vc, pkv_dtype kv_dt,
                       const float* ks, const float* vs, const int32_t* tables, int32_t mb,
                       const int32_t* lens, int32_t max_ctx, int32_t S, int32_t hq, int32_t hkv,
                       int32_t D, int32_t bs, int32_t nb, float scale, int32_t part_tokens,
                       int32_t algo, void* ws, size_t ws_bytes, void* stream,
                       const void* new_k = nullptr, const void* new_v = nullptr) {
  const char* who = "paged_attention_decode";
  pkv_status st = check_common(who, out, out_dt, q, q_dt, kc, vc, kv_dt, ks, vs, tables, mb, lens,
                               max_ctx, S, S, hq, hkv, D, bs, nb, scale);
  if (st) return st;
  if (part_tokens < 0 || part_tokens % 16 != 0)
    return fail(PKV_ERR_INVALID, "%s: partition_tokens %d must be 0 or a multiple of 16", who,
                part_tokens);
  const int32_t policy = algo & (PKV_KV_STREAM | PKV_KV_CACHED);
  const bool merge_in_kernel = (algo & PKV_MERGE_IN_KERNEL) != 0;
  algo &= ~(PKV_KV_STREAM | PKV_KV_CACHED | PKV_MERGE_IN_KERNEL);
  if (algo < PKV_ALGO_AUTO || algo > PKV_ALGO_MFMA || policy == (PKV_KV_STREAM | PKV_KV_CACHED))
    return fail(PKV_ERR_INVALID, "%s: unknown algo %d", who, algo | policy);
  if (merge_in_kernel && which != DecodePart::kStep)
    return fail(PKV_ERR_INVALID, "%s: PKV_MERGE_IN_KERNEL applies to the decode step only", who);
  const int group = hq / hkv;
  if (algo == PKV_ALGO_MFMA && !use_mfma(algo, q_dt, group))
    return fail(PKV_ERR_UNSUPPORTED, "%s: MFMA path needs 16-bit q and a group of at most 16",
                who);
  if (which == DecodePart::kStep && (new_k != nullptr) != (new_v != nullptr))
    return fail(PKV_ERR_INVALID, "%s: new_k and new_v are both given or both NULL", who);
  if (new_k != nullptr && has_scales(kv_dt))
    return fail(PKV_ERR_UNSUPPORTED,
                "%s: appending rows to %s KV takes quantise-on-write (pkv_reshape_and_cache_%s)",
                who, dtype_name(kv_dt), kv_dt == PKV_I8 ? "int8" : "int4");
  if (new_k != nullptr && (!aligned(new_k, 16) || !aligned(new_v, 16)))
    return fail(PKV_ERR_INVALID, "%s: new_k and new_v must be 16-byte aligned", who);
  if (S == 0) return PKV_OK;
  const int parts = num_partitions(max_ctx, part_tokens);
  const WsLayout w = workspace_layout(S, hq, D, parts);
  const size_t need = w.total + (which == DecodePart::kStep ? counter_bytes(S, hq, parts) : 0);
  if (need > 0 && (!ws || ws_bytes < need || !aligned(ws, kAlign)))
    return fail(PKV_ERR_INVALID, "%s: workspace needs %zu bytes, 256-byte aligned (got %zu)", who,
                need, ws_bytes);
  if (deep_validation() && which != DecodePart::kReduce) {
    st = deep_check_tables(who, tables, mb, lens, max_ctx, S, nb, bs, stream);
    if (st) return st;
  }
  AttnArgs a{};
  a.out = out;
  a.part_o = parts > 1 ? static_cast<float*>(ws) : nullptr;
  a.part_ml = parts > 1 ? reinterpret_cast<float*>(static_cast<char*>(ws) + w.o_bytes) : nullptr;
  a.q = q;
  a.kc = kc;
  a.vc = vc;
  a.ks = has_scales(kv_dt) ? ks : nullptr;
  a.vs = has_scales(kv_dt) ? vs : nullptr;
  a.tables = tables;
  a.lens = lens;
  a.qsl = nullptr;
  a.max_blocks = mb;
  a.bs_shift = block_shift(bs);
  a.max_ctx = max_ctx;
  a.num_seqs = S;
  a.num_rows = S;
  a.hq = hq;
  a.hkv = hkv;
  a.num_blocks = nb;
  a.num_parts = parts;
  // Without a split one partition covers the longest context.
  a.part_tokens = parts > 1 ? part_tokens : std::max(16, (max_ctx + 15) / 16 * 16);
  a.out_kind = out_kind_of(out_dt);
  a.scale_log2 = scale * kLog2e;
  // Stream the K/V loads unless the pool fits in the memory-side cache
  // (then blocks shared by several sequences can be served from it).
  const double pool_bytes = 2.0 * nb * hkv * bs * static_cast<double>(row_bytes(kv_dt, D));
  a.stream_kv = policy == PKV_KV_STREAM ||
                (policy == 0 && pool_bytes > static_cast<double>(PKV_KV_CACHE_BYTES));
  if (which == DecodePart::kStep) {
    a.new_k = new_k;
    a.new_v = new_v;
    a.counters = (merge_in_kernel && parts > 1)
                     ? reinterpret_cast<int32_t*>(static_cast<char*>(ws) + w.total)
                     : nullptr;
  }
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (which != DecodePart::kReduce) {
    st = use_mfma(algo, q_dt, group) ? launch_decode_mfma(a, q_dt, kv_dt, D, group, hs)
                                     : launch_decode_wave(a, q_dt, kv_dt, D, group, hs);
    if (st) return st;
  }
  const bool reduce = which == DecodePart::kAll || which == DecodePart::kReduce ||
                      (which == DecodePart::kStep && a.counters == nullptr);
  if (reduce && parts > 1) return launch_reduce(a, D, hs);
  return PKV_OK;
}

// Scratch of the allocation-free decode entry point: split-K partial states
// in a file-scope device array, one instance per GPU the library runs on.
// In host code `scratch` names a host-side stand-in, not device memory, so
// its device address is looked up once per device (hipGetSymbolAddress,
// with that device current) and only that address is handed to kernels.
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];

}  // namespace

static __device__ __align__(256) uint8_t scratch[PKV_NOALLOC_SCRATCH_BYTES];

namespace {

pkv_status scratch_address(const char* who, void** addr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return fail(PKV_ERR_DEVICE, "%s: hipGetDevice failed: %s", who, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PKV_ERR_UNSUPPORTED, "%s: device %d beyond the %d the library tracks", who, dev,
                kMaxDevices);
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(PKV_ERR_DEVICE, "%s: scratch address of device %d: %s", who, dev,
                  hipGetErrorString(e));
    g_scratch_addr[dev].store(p, std::memory_order_release);
  }
  *addr = p;
  return PKV_OK;
}

int device_compute_units(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
  return e == hipSuccess && *cus > 0 ? 0 : -1;
}

}  // namespace

extern "C" {

size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                  int32_t max_context_len, int32_t partition_tokens) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len < 0) return 0;
  return workspace_layout(num_seqs, num_q_heads, head_dim,
                          num_partitions(max_context_len, partition_tokens))
      .total;
}

size_t pkv_decode_step_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                       int32_t max_context_len, int32_t partition_tokens) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len < 0) return 0;
  const int parts = num_partitions(max_context_len, partition_tokens);
  return workspace_layout(num_seqs, num_q_heads, head_dim, parts).total +
         counter_bytes(num_seqs, num_q_heads, parts);
}

size_t pkv_prefill_workspace_bytes(int32_t num_query_tokens, int32_t num_q_heads,
                                   int32_t head_dim, int32_t max_context_len,
                                   int32_t partition_tokens) {
  if (num_query_tokens <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len < 0) return 0;
  return workspace_layout(num_query_tokens, num_q_heads, head_dim,
                          num_partitions(max_context_len, partition_tokens))
      .total;
}

pkv_status pkv_decode_partition_tokens(const int32_t* context_lens, int32_t num_seqs,
                                       pkv_dtype q_dtype, pkv_dtype kv_dtype, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                       int32_t num_blocks, int32_t algo, int32_t* partition_tokens) {
  const char* who = "decode_partition_tokens";
  if (!partition_tokens) return fail(PKV_ERR_INVALID, "%s: NULL pointer", who);
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(PKV_ERR_INVALID, "%s: bad sizes (Hq=%d Hkv=%d NB=%d)", who, num_q_heads,
                num_kv_heads, num_blocks);
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "%s: head_dim %d (64 or 128)", who, head_dim);
  if (block_shift(block_size) < 0)
    return fail(PKV_ERR_UNSUPPORTED, "%s: block_size %d (16, 32, 64 or 128)", who, block_size);
  if (q_dtype != PKV_F32 && q_dtype != PKV_F16 && q_dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "%s: q dtype %s", who, dtype_name(q_dtype));
  if (kv_dtype != q_dtype && !has_scales(kv_dtype))
    return fail(PKV_ERR_UNSUPPORTED, "%s: kv dtype %s with q dtype %s", who,
                dtype_name(kv_dtype), dtype_name(q_dtype));
  const int32_t policy = algo & (PKV_KV_STREAM | PKV_KV_CACHED);
  const int32_t base = algo & ~(PKV_KV_STREAM | PKV_KV_CACHED | PKV_MERGE_IN_KERNEL);
  if (base < PKV_ALGO_AUTO || base > PKV_ALGO_MFMA || policy == (PKV_KV_STREAM | PKV_KV_CACHED))
    return fail(PKV_ERR_INVALID, "%s: unknown algo %d", who, algo);
  const int group = num_q_heads / num_kv_heads;
  if (base == PKV_ALGO_MFMA && !use_mfma(base, q_dtype, group))
    return fail(PKV_ERR_UNSUPPORTED, "%s: MFMA path needs 16-bit q and a group of at most 16",
                who);
  // the launch's choice of load policy and kernel
  const double pool_bytes =
      2.0 * num_blocks * num_kv_heads * block_size * static_cast<double>(row_bytes(kv_dtype, head_dim));
  const bool nt = policy == PKV_KV_STREAM ||
                  (policy == 0 && pool_bytes > static_cast<double>(PKV_KV_CACHE_BYTES));
  int per_cu = 0, per_partition = 0, min_tokens = kMinAutoPartition;
  pkv_status st;
  if (use_mfma(base, q_dtype, group)) {
    st = decode_mfma_occupancy(q_dtype, kv_dtype, head_dim, nt, &per_cu);
    per_partition = num_kv_heads;
  } else {
    // the variant of the largest partitions (the 16-wave kernel where it
    // applies, which runs only from its own minimum partition up)
    int heads = 1, wide_min = 0;
    st = decode_wave_occupancy(q_dtype, kv_dtype, head_dim, group, INT32_MAX, nt, &per_cu, &heads,
                               &wide_min);
    per_partition = num_q_heads / heads;
    min_tokens = std::max(min_tokens, wide_min);
  }
  if (st) return st;
  int cus = 0;
  if (device_compute_units(&cus))
    return fail(PKV_ERR_DEVICE, "%s: no device to size the launch for", who);
  if (per_cu <= 0)
    return fail(PKV_ERR_DEVICE, "%s: the decode kernel does not fit a compute unit", who);
  return pkv_decode_partition_for_capacity(context_lens, num_seqs, per_partition,
                                           static_cast<int64_t>(per_cu) * cus, min_tokens,
                                           partition_tokens);
}

pkv_status pkv_prefill_partition_tokens(const int32_t* query_lens, const int32_t* context_lens,
                                        int32_t num_seqs, int32_t num_q_heads, pkv_dtype q_dtype,
                                        int32_t* partition_tokens) {
  const char* who = "prefill_partition_tokens";
  if (!partition_tokens || (num_seqs > 0 && (!query_lens || !context_lens)))
    return fail(PKV_ERR_INVALID, "%s: NULL pointer", who);
  if (num_seqs < 0 || num_q_heads <= 0)
    return fail(PKV_ERR_INVALID, "%s: bad sizes (S=%d Hq=%d)", who, num_seqs, num_q_heads);
  if (q_dtype != PKV_F32 && q_dtype != PKV_F16 && q_dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "%s: q dtype %s", who, dtype_name(q_dtype));
  for (int32_t s = 0; s < num_seqs; ++s)
    if (query_lens[s] < 0 || context_lens[s] < query_lens[s])
      return fail(PKV_ERR_INVALID, "%s: sequence %d has %d query rows over %d keys", who, s,
                  query_lens[s], context_lens[s]);
  *partition_tokens = 0;
  if (q_dtype == PKV_F32) return PKV_OK;   // the wavefront rows: one workgroup per row already
  int cus = 0;
  if (device_compute_units(&cus))
    return fail(PKV_ERR_DEVICE, "%s: no device to size the launch for", who);
  const int rows = prefill_tile_rows();
  PKV_GUARD({
    std::vector<int64_t> weights(static_cast<size_t>(num_seqs));
    for (int32_t s = 0; s < num_seqs; ++s)
      weights[s] = static_cast<int64_t>((query_lens[s] + rows - 1) / rows) * num_q_heads;
    *partition_tokens = partition_for_rounds(context_lens, weights.data(), 0, num_seqs,
                                             static_cast<int64_t>(kPrefillPerCu) * cus,
                                             kMinAutoPartition);
    return PKV_OK;
  })
}

pkv_status pkv_paged_attention_decode(void* out, pkv_dtype out_dtype, const void* q,
                                      pkv_dtype q_dtype, const void* k_cache, const void* v_cache,
                                      pkv_dtype kv_dtype, const float* k_scale,
                                      const float* v_scale, const int32_t* block_tables,
                                      int32_t max_blocks_per_seq, const int32_t* context_lens,
                                      int32_t max_context_len, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, int32_t num_blocks, float scale,
                                      int32_t partition_tokens, int32_t algo, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  PKV_GUARD({
    return decode_impl(DecodePart::kAll, out, out_dtype, q, q_dtype, k_cache, v_cache, kv_dtype,
                       k_scale, v_scale, block_tables, max_blocks_per_seq, context_lens,
                       max_context_len, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                       num_blocks, scale, partition_tokens, algo, workspace, workspace_bytes,
                       stream);
  })
}

pkv_status pkv_paged_attention_decode_step(
    void* out, pkv_dtype out_dtype, const void* q, pkv_dtype q_dtype, const void* new_k,
    const void* new_v, void* k_cache, void* v_cache, pkv_dtype kv_dtype, const float* k_scale,
    const float* v_scale, const int32_t* block_tables, int32_t max_blocks_per_seq,
    const int32_t* context_lens, int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
    int32_t partition_tokens, int32_t algo, void* workspace, size_t workspace_bytes,
    void* stream) {
  PKV_GUARD({
    return decode_impl(DecodePart::kStep, out, out_dtype, q, q_dtype, k_cache, v_cache, kv_dtype,
                       k_scale, v_scale, block_tables, max_blocks_per_seq, context_lens,
                       max_context_len, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                       num_blocks, scale, partition_tokens, algo, workspace, workspace_bytes,
                       stream, new_k, new_v);
  })
}

pkv_status pkv_paged_attention_decode_partials(
    void* out, pkv_dtype out_dtype, const void* q, pkv_dtype q_dtype, const void* k_cache,
    const void* v_cache, pkv_dtype kv_dtype, const float* k_scale, const float* v_scale,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
    int32_t partition_tokens, int32_t algo, void* workspace, size_t workspace_bytes,
    void* stream) {
  PKV_GUARD({
    return decode_impl(DecodePart::kMain, out, out_dtype, q, q_dtype, k_cache, v_cache, kv_dtype,
                       k_scale, v_scale, block_tables, max_blocks_per_seq, context_lens,
                       max_context_len, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                       num_blocks, scale, partition_tokens, algo, workspace, workspace_bytes,
                       stream);
  })
}

pkv_status pkv_paged_attention_decode_noalloc(
    void* out, pkv_dtype out_dtype, const void* q, pkv_dtype q_dtype, const void* k_cache,
    const void* v_cache, pkv_dtype kv_dtype, const float* k_scale, const float* v_scale,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
    int32_t partition_tokens, int32_t algo, void* stream) {
  PKV_GUARD({
    const char* who = "paged_attention_decode_noalloc";
    if (num_seqs < 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len < 0 ||
        partition_tokens < 0)
      return fail(PKV_ERR_INVALID, "%s: bad sizes", who);
    const size_t need = workspace_layout(num_seqs, num_q_heads, head_dim,
                                         num_partitions(max_context_len, partition_tokens))
                            .total;
    if (need > PKV_NOALLOC_SCRATCH_BYTES)
      return fail(PKV_ERR_INVALID,
                  "%s: split-K partial results need %zu bytes, more than the %llu-byte scratch "
                  "(use larger partitions, or the workspace entry point)",
                  who, need, static_cast<unsigned long long>(PKV_NOALLOC_SCRATCH_BYTES));
    void* ws = nullptr;
    if (need > 0) {
      pkv_status st = scratch_address(who, &ws);
      if (st) return st;
    }
    return decode_impl(DecodePart::kAll, out, out_dtype, q, q_dtype, k_cache, v_cache, kv_dtype,
                       k_scale, v_scale, block_tables, max_blocks_per_seq, context_lens,
                       max_context_len, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                       num_blocks, scale, partition_tokens, algo, ws,
                       need > 0 ? PKV_NOALLOC_SCRATCH_BYTES : 0, stream);
  })
}

pkv_status pkv_paged_attention_reduce(void* out, pkv_dtype out_dtype, const int32_t* context_lens,
                                      int32_t max_context_len, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t head_dim,
                                      int32_t partition_tokens, const void* workspace,
                                      size_t workspace_bytes, void* stream) {
  PKV_GUARD({
    const char* who = "paged_attention_reduce";
    if (num_seqs < 0 || num_q_heads <= 0 || (head_dim != 64 && head_dim != 128) ||
        max_context_len < 0 || partition_tokens < 0 || partition_tokens % 16)
      return fail(PKV_ERR_INVALID, "%s: bad sizes", who);
    if (out_dtype != PKV_F32 && out_dtype != PKV_BF16 && out_dtype != PKV_F16)
      return fail(PKV_ERR_UNSUPPORTED, "%s: out dtype", who);
    const int parts = num_partitions(max_context_len, partition_tokens);
    if (num_seqs == 0 || parts <= 1) return PKV_OK;
    const WsLayout w = workspace_layout(num_seqs, num_q_heads, head_dim, parts);
    if (!out || !context_lens || !workspace || workspace_bytes < w.total ||
        !aligned(workspace, kAlign))
      return fail(PKV_ERR_INVALID, "%s: NULL pointer or workspace smaller than %zu bytes", who,
                  w.total);
    AttnArgs a{};
    a.out = out;
    a.part_o = static_cast<float*>(const_cast<void*>(workspace));
    a.part_ml = reinterpret_cast<float*>(static_cast<char*>(const_cast<void*>(workspace)) +
                                         w.o_bytes);
    a.lens = context_lens;
    a.max_blocks = (max_context_len + 15) / 16 + 1;
    a.max_ctx = max_context_len;
    a.num_seqs = num_seqs;
    a.num_rows = num_seqs;
    a.hq = num_q_heads;
    a.hkv = num_q_heads;
    a.num_parts = parts;
    a.part_tokens = partition_tokens;
    a.out_kind = out_kind_of(out_dtype);
    return launch_reduce(a, head_dim, static_cast<hipStream_t>(stream));
  })
}

pkv_status pkv_paged_attention_prefill(
    void* out, pkv_dtype out_dtype, const void* q, pkv_dtype q_dtype, const void* k_cache,
    const void* v_cache, pkv_dtype kv_dtype, const float* k_scale, const float* v_scale,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* query_start_loc,
    const int32_t* context_lens, int32_t max_query_len, int32_t max_context_len, int32_t num_seqs,
    int32_t num_query_tokens, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t num_blocks, float scale, int32_t partition_tokens,
    void* workspace, size_t workspace_bytes, void* stream) {
  PKV_GUARD({
    const char* who = "paged_attention_prefill";
    pkv_status st = check_common(who, out, out_dtype, q, q_dtype, k_cache, v_cache, kv_dtype,
                                 k_scale, v_scale, block_tables, max_blocks_per_seq, context_lens,
                                 max_context_len, num_seqs, num_query_tokens, num_q_heads,
                                 num_kv_heads, head_dim, block_size, num_blocks, scale);
    if (st) return st;
    if (num_query_tokens < 0 || max_query_len < 0 || max_query_len > max_context_len)
      return fail(PKV_ERR_INVALID, "%s: bad query sizes", who);
    if (num_seqs > 0 && !query_start_loc)
      return fail(PKV_ERR_INVALID, "%s: query_start_loc is NULL", who);
    if (has_scales(kv_dtype))
      return fail(PKV_ERR_UNSUPPORTED, "%s: %s KV is a decode-only storage here", who,
                  dtype_name(kv_dtype));
    if (partition_tokens < 0 || partition_tokens % 16 != 0)
      return fail(PKV_ERR_INVALID, "%s: partition_tokens %d must be 0 or a multiple of 16", who,
                  partition_tokens);
    const int parts = num_partitions(max_context_len, partition_tokens);
    const WsLayout w = workspace_layout(num_query_tokens, num_q_heads, head_dim, parts);
    if (w.total > 0 && (!workspace || workspace_bytes < w.total || !aligned(workspace, kAlign)))
      return fail(PKV_ERR_INVALID, "%s: workspace needs %zu bytes, 256-byte aligned (got %zu)",
                  who, w.total, workspace_bytes);
    if (num_seqs == 0 || num_query_tokens == 0) return PKV_OK;
    if (deep_validation()) {
      std::vector<int32_t> L, Q;
      st = deep_check_tables(who, block_tables, max_blocks_per_seq, context_lens,
                             max_context_len, num_seqs, num_blocks, block_size, stream, &L);
      if (st) return st;
      st = fetch_i32(query_start_loc, num_seqs + 1, stream, Q);
      if (st) return st;
      if (Q[0] != 0 || Q[num_seqs] != num_query_tokens)
        return fail(PKV_ERR_INVALID, "%s: query_start_loc must run from 0 to %d", who,
                    num_query_tokens);
      for (int32_t s = 0; s < num_seqs; ++s) {
        const int32_t ql = Q[s + 1] - Q[s];
        if (ql < 0 || ql > max_query_len || ql > L[s])
          return fail(PKV_ERR_INVALID, "%s: chunk %d has length %d (context %d, max %d)", who,
                      s, ql, L[s], max_query_len);
      }
    }
    AttnArgs a{};
    a.out = out;
    a.q = q;
    a.kc = k_cache;
    a.vc = v_cache;
    a.tables = block_tables;
    a.lens = context_lens;
    a.qsl = query_start_loc;
    a.max_blocks = max_blocks_per_seq;
    a.bs_shift = block_shift(block_size);
    a.max_ctx = max_context_len;
    a.num_seqs = num_seqs;
    a.num_rows = num_query_tokens;
    a.hq = num_q_heads;
    a.hkv = num_kv_heads;
    a.num_blocks = num_blocks;
    a.num_parts = parts;
    a.part_tokens = parts > 1 ? partition_tokens : std::max(16, (max_context_len + 15) / 16 * 16);
    a.part_o = parts > 1 ? static_cast<float*>(workspace) : nullptr;
    a.part_ml =
        parts > 1 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + w.o_bytes) : nullptr;
    a.out_kind = out_kind_of(out_dtype);
    a.scale_log2 = scale * kLog2e;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const int group = num_q_heads / num_kv_heads;
    // The matrix-core prefill streams K/V under the pool-size rule of decode
    // when each tile has a single reader (see launch_prefill_mfma); the fp32
    // wavefront rows of one chunk share their keys and keep cached loads.
    if (q_dtype != PKV_F32) {
      const double pool_bytes =
          2.0 * num_blocks * num_kv_heads * block_size * static_cast<double>(row_bytes(kv_dtype, head_dim));
      a.stream_kv = pool_bytes > static_cast<double>(PKV_KV_CACHE_BYTES);
    }
    pkv_status ls = q_dtype == PKV_F32
                        ? launch_decode_wave(a, q_dtype, kv_dtype, head_dim, group, hs)
                        : launch_prefill_mfma(a, q_dtype, head_dim, group, max_query_len, hs);
    if (ls) return ls;
    // Rows whose keys span several partitions left partial results; the
    // decode reduce merges them (it finds each row's keys through qsl).
    return parts > 1 ? launch_reduce(a, head_dim, hs) : PKV_OK;
  })
}

}  // extern "C"
