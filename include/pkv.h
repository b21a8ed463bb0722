/*
 * pkv.h - C ABI of libpkv: paged KV cache and paged attention on AMD
 * Instinct MI355X (gfx950).
 *
 * The KV cache of every sequence is split into fixed-size blocks of
 * `block_size` tokens that sit anywhere in one global pool; a per-sequence
 * block table maps logical block j to a physical block id.  Pages cited:
 *   [kongchang] kongchang.com, "vLLM架构深度解析：PagedAttention如何实现高吞吐LLM推理"
 *   [cnnetsun]  cnnetsun.cn/a/1845762, "别再让GPU内存拖后腿了：vLLM的PagedAttention如何像操作系统一样管理KV Cache"
 *   [aisoosoo]  aisoosoo.com, "vLLM：大模型推理的加速引擎，PagedAttention 颠覆显存管理"
 *   [nxbn]      m.nxbn.cn/news/200425 (VLLM walkthrough, numbered sections 一..六)
 *
 * Conventions for every call:
 *   - Every call returns a pkv_status; 0 is success.  On failure
 *     pkv_last_error() returns a message for the calling thread.  No C++
 *     exception crosses this boundary and no call aborts the process.
 *   - "host" pointers are CPU memory owned by the caller; "device" pointers
 *     are GPU memory (for example torch tensors) owned by the caller.  The
 *     library keeps no pointer after a call returns and allocates no device
 *     memory: scratch space is a caller-provided workspace.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Device
 *     calls only enqueue work; they return before it finishes.
 *   - Device-side layouts (all contiguous, row-major):
 *       cache   k_cache / v_cache   [num_blocks][num_kv_heads][block_size][head_dim]
 *               (I4: [num_blocks][num_kv_heads][block_size][head_dim / 2] bytes)
 *       scales  k_scale / v_scale   float [num_blocks][num_kv_heads] (I8 and I4 only)
 *       tables  block_tables        int32 [num_seqs][max_blocks_per_seq], -1 padded
 *     Position p of a sequence lives in block table[p / block_size] at row
 *     p % block_size ([cnnetsun] §2.1; [nxbn] §2.2); slot = block *
 *     block_size + row addresses one token row of the pool.
 *   - Arguments are validated on the host before anything is enqueued.  With
 *     the environment variable PKV_VALIDATE=1 the device index arrays
 *     (slots, tables, lengths, copy pairs) are also copied back and checked,
 *     which synchronises the stream; kernels in any case skip table entries
 *     and slots outside the pool instead of reading or writing out of bounds.
 *   - The block manager is not thread-safe; device calls may be made from any
 *     thread.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t pkv_status;
#define PKV_OK 0
#define PKV_ERR_INVALID 1        /* bad argument or state; nothing changed       */
#define PKV_ERR_OUT_OF_BLOCKS 2  /* pool cannot satisfy the request; nothing changed */
#define PKV_ERR_UNSUPPORTED 3    /* valid but not implemented (dtype, head_dim...) */
#define PKV_ERR_DEVICE 4         /* a HIP call failed                              */
#define PKV_ERR_INTERNAL 5

typedef int32_t pkv_dtype;
#define PKV_F32 0
#define PKV_F16 1
#define PKV_BF16 2
#define PKV_I8 3   /* KV storage only: symmetric codes with per-(block, kv head) fp32 scales */
#define PKV_I4 4   /* KV storage only: 4-bit symmetric codes in [-7, 7], two per byte
                      (element 2i in the low nibble of byte i, element 2i + 1 in the
                      high nibble, two's complement), per-(block, kv head) fp32 scales */

/* Decode kernel choice. */
#define PKV_ALGO_AUTO 0
#define PKV_ALGO_WAVE 1   /* wavefront dot products + shuffle reductions (any dtype) */
#define PKV_ALGO_MFMA 2   /* matrix cores over a query-head group (bf16/f16 q)      */
/* K/V load policy, OR-ed into algo.  Streaming loads carry the non-temporal
 * hint: each tile passes through the caches without displacing what is
 * reused, the right choice when a call reads every block once (measured
 * about 10% faster on a 1.4 GB pool).  Cached loads keep the tiles, the
 * right choice when sequences share blocks (beams over a shared prompt,
 * forks, prefix caching: pkv_bm_stats_get reports shared_blocks > 0), which
 * the caller knows and the call does not: such callers pass
 * PKV_KV_CACHED.  Neither flag: stream when the pool's K and V bytes exceed
 * PKV_KV_CACHE_BYTES (the 256 MB memory-side cache of an MI355X), cache
 * otherwise. */
#define PKV_KV_STREAM 0x10
#define PKV_KV_CACHED 0x20
#define PKV_KV_CACHE_BYTES (256ull << 20)
/* pkv_paged_attention_decode_step only, OR-ed into algo: split rows are
 * merged inside the attention launch by the last of their partitions to
 * finish, instead of by the reduce kernel after it (see that call). */
#define PKV_MERGE_IN_KERNEL 0x40

/* Thread-local description of the last failure of this thread. */
const char* pkv_last_error(void);
const char* pkv_version(void);

/* ------------------------------------------------------------------------
 * Block manager (host).  A fixed pool of `num_blocks` blocks with a free list
 * used as a stack and a reference count per block ([cnnetsun] §2.1 and §2.2;
 * [kongchang] section "KV Cache内存共享").  Blocks are taken only when tokens
 * arrive, so a sequence of n tokens holds ceil(n / block_size) blocks
 * ([kongchang] section "PagedAttention带来的性能收益"), and return to the
 * pool when their count reaches zero ([nxbn] §2.3).
 * ---------------------------------------------------------------------- */
typedef struct pkv_bm pkv_bm;

/* init_free_order: host int32[num_blocks], a permutation of 0..num_blocks-1
 * giving the initial free list bottom-to-top (allocation pops from the top,
 * i.e. the end), or NULL for 0..num_blocks-1.  *out receives the handle,
 * which the caller releases with pkv_bm_destroy.  INVALID for a non-positive
 * size or a bad permutation. */
pkv_status pkv_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* init_free_order,
                         pkv_bm** out);
void pkv_bm_destroy(pkv_bm* bm);

/* Pop n blocks (refcount 1 each); ids_out: host int32[n] in pop order.
 * OUT_OF_BLOCKS (state unchanged) when fewer than n are free. */
pkv_status pkv_bm_alloc(pkv_bm* bm, int32_t n, int32_t* ids_out);
/* incref needs an allocated block; decref pushes the block back on the free
 * list when its count reaches 0.  INVALID for an unknown or free block. */
pkv_status pkv_bm_incref(pkv_bm* bm, int32_t block);
pkv_status pkv_bm_decref(pkv_bm* bm, int32_t block);
int32_t pkv_bm_num_free(const pkv_bm* bm);
/* free_list: host int32[num_blocks] (bottom to top, *free_len entries used);
 * refcounts: host int32[num_blocks].  Either may be NULL. */
pkv_status pkv_bm_get_state(const pkv_bm* bm, int32_t* free_list, int32_t* free_len,
                            int32_t* refcounts);

typedef struct pkv_bm_stats {
  int32_t num_blocks;
  int32_t block_size;
  int32_t free_blocks;
  int32_t used_blocks;     /* refcount > 0 */
  int32_t shared_blocks;   /* refcount > 1 */
  int32_t num_seqs;
  int64_t logical_blocks;  /* sum over live sequences of their table lengths */
  int64_t tokens;          /* sum over live sequences of their lengths */
  int64_t waste_slots;     /* logical_blocks * block_size - tokens */
} pkv_bm_stats;
/* Usage figures for monitoring ([cnnetsun] §4.2 lists page utilisation and
 * share ratio; [kongchang] section "显存浪费的三种形式" names the waste). */
pkv_status pkv_bm_stats_get(const pkv_bm* bm, pkv_bm_stats* out);

/* Latency of page allocation, the health bar of [cnnetsun] §4.2 (P99 of
 * page allocation under 1 ms).  Every call that takes blocks from the pool
 * (pkv_bm_alloc, pkv_seq_create, pkv_seq_create_cached, pkv_seq_append,
 * pkv_seq_append_batch), failed ones included, times itself on the host's
 * steady clock; the percentiles cover the latest min(calls, 65536) of them
 * (nearest rank).  reset != 0 starts a new count after reading. */
typedef struct pkv_bm_latency {
  int64_t calls;     /* allocating calls since creation or the last reset */
  int32_t window;    /* calls the percentiles cover */
  double p50_us;
  double p99_us;
  double max_us;
} pkv_bm_latency;
pkv_status pkv_bm_latency_get(pkv_bm* bm, pkv_bm_latency* out, int32_t reset);

/* ------------------------------------------------------------------------
 * Sequences (host).  Sequence ids count up from 0 and are never reused.
 * ---------------------------------------------------------------------- */
/* New sequence holding num_tokens positions (ceil(num_tokens/block_size)
 * blocks, logical order = pop order).  OUT_OF_BLOCKS leaves no trace. */
pkv_status pkv_seq_create(pkv_bm* bm, int32_t num_tokens, int64_t* seq_out);
/* Child sharing every block of the parent (each block's count + 1): parallel
 * sampling and beam search share history until they diverge ([kongchang]
 * section "KV Cache内存共享"). */
pkv_status pkv_seq_fork(pkv_bm* bm, int64_t parent, int64_t* child_out);
/* Append num_tokens positions; slots_out: host int32[num_tokens] receives
 * their slots.  If the partly filled tail block is shared (count > 1) it is
 * first replaced by a new block (copy-on-write): *cow_src / *cow_dst receive
 * (shared block, new block), which the caller must copy with
 * pkv_copy_blocks before writing the new rows; otherwise both are -1.  A full
 * tail never needs a copy.  All-or-nothing: OUT_OF_BLOCKS changes nothing. */
pkv_status pkv_seq_append(pkv_bm* bm, int64_t seq, int32_t num_tokens, int32_t* slots_out,
                          int32_t* cow_src, int32_t* cow_dst);
/* One new position for each of n distinct sequences, handled in the order
 * given (so of k beams sharing a partly filled tail the first k-1 copy and
 * the last writes in place).  slots_out: host int32[n]; cow_pairs_out: host
 * int32[n][2] receives *num_cow_out (src, dst) pairs.  All-or-nothing. */
pkv_status pkv_seq_append_batch(pkv_bm* bm, const int64_t* seqs, int32_t n, int32_t* slots_out,
                                int32_t* cow_pairs_out, int32_t* num_cow_out);
/* Slots of positions [start, start+count) of a sequence (host int32[count]). */
pkv_status pkv_seq_slots(const pkv_bm* bm, int64_t seq, int32_t start, int32_t count,
                         int32_t* slots_out);
pkv_status pkv_seq_len(const pkv_bm* bm, int64_t seq, int32_t* len_out);
/* Drop a sequence: decref its blocks in logical order. */
pkv_status pkv_seq_free(pkv_bm* bm, int64_t seq);
/* Block tables and lengths of n sequences: tables_out host
 * int32[n][max_blocks] (-1 padded), lens_out host int32[n].  INVALID if a
 * table is longer than max_blocks. */
pkv_status pkv_seq_export(const pkv_bm* bm, const int64_t* seqs, int32_t n, int32_t max_blocks,
                          int32_t* tables_out, int32_t* lens_out);

/* Block size for a workload whose sequences average avg_context_len tokens:
 * 16 below 512, 32 below 2048, 64 otherwise (the adaptive_page_size rule of
 * [cnnetsun] §4.3: small pages keep utilisation high for short sequences,
 * larger ones cut table entries for long ones).  NaN or negative: 16. */
int32_t pkv_adaptive_block_size(double avg_context_len);

/* ------------------------------------------------------------------------
 * Prefix caching (host).  Requests that begin with the same tokens (a system
 * prompt) share the KV pages of that prefix instead of storing it again:
 * [cnnetsun] §2.2 (share_prefix: find the prefix by its hash, attach to its
 * pages through reference counts) and [aisoosoo] section "技术亮点" (equal
 * prompt prefixes reuse KV pages without recomputation).  The unit is a full
 * block; block j is indexed under (physical block j-1, or -1 for j = 0; its
 * block_size token ids), compared exactly.  An index entry lives as long as
 * its block is allocated and holds no count of its own.
 * ---------------------------------------------------------------------- */
/* New sequence of num_tokens positions (tokens: host int32[num_tokens], the
 * token ids).  Its leading full blocks found in the index are shared (each
 * count + 1), walking from block 0 and stopping at the first miss; the rest
 * are popped as in pkv_seq_create.  *cached_out (may be NULL) receives the
 * number of leading positions whose K/V already sit in shared blocks
 * (block_size x shared blocks): the caller computes and writes only
 * positions [*cached_out, num_tokens).  All-or-nothing. */
pkv_status pkv_seq_create_cached(pkv_bm* bm, const int32_t* tokens, int32_t num_tokens,
                                 int64_t* seq_out, int32_t* cached_out);
/* Index the full blocks among the first num_tokens positions of a sequence
 * (tokens: host int32[num_tokens], its token ids), to be called once their
 * K/V are written.  A key already indexed keeps its block and a block is
 * indexed at most once.  *added_out (may be NULL) receives the number of new
 * entries.  INVALID if num_tokens exceeds the sequence's length. */
pkv_status pkv_seq_publish(pkv_bm* bm, int64_t seq, const int32_t* tokens, int32_t num_tokens,
                           int32_t* added_out);
/* Lookup figures for the share-ratio health metric of [cnnetsun] §4.2:
 * *lookups = full prompt blocks looked up by pkv_seq_create_cached since
 * creation, *hits = those found, *cached_blocks = entries now indexed.
 * Any output may be NULL. */
pkv_status pkv_bm_prefix_stats(const pkv_bm* bm, int64_t* lookups, int64_t* hits,
                               int32_t* cached_blocks);

/* ------------------------------------------------------------------------
 * reshape_and_cache (device).  Only the new tokens' K/V are computed each
 * step and appended to the cache ([nxbn] section 一); each token's row goes to
 * the slot the block table gives it ([nxbn] §2.2).
 *   key, value    device [num_tokens][num_kv_heads][head_dim] in `dtype`,
 *                 consecutive tokens `key_stride` / `value_stride` elements
 *                 apart (0 = num_kv_heads * head_dim, i.e. contiguous)
 *   slot_mapping  device int32[num_tokens]; a negative slot skips the row.
 *                 Slots must be distinct (validated with PKV_VALIDATE=1).
 *   dtype         F32, F16 or BF16 (cache and inputs share it); the copy is
 *                 bit-exact.
 * ---------------------------------------------------------------------- */
pkv_status pkv_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                                 const int32_t* slot_mapping, int32_t num_tokens,
                                 int64_t key_stride, int64_t value_stride, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                 pkv_dtype dtype, void* stream);

/* reshape_and_cache into int8 storage (quantise on write): the new tokens'
 * K/V rows go into int8 pools with one fp32 scale per (block, KV head), the
 * write side of the int8 decode path ([cnnetsun] §3.2 lists INT8 KV; §4.3
 * turns it on for the historical pages).  The slot mapping splits into runs
 * (consecutive tokens whose slots are consecutive rows of one block, as an
 * append writes them); a run's block is taken as written below the run's
 * first row.  The scale only grows, to max(old, max|new rows| / 127): when
 * it grows, the existing codes are re-encoded from their values
 * (code x old / new, rounded to nearest even, clamped to +-127), and the new
 * rows are encoded with the new scale.  A run starting at row 0 ignores the
 * old scale, so a whole block in one run is pkv_quantize_blocks exactly.
 * Rows past the run are left as they are (decode masks them).
 *   key, value     device [num_tokens][num_kv_heads][head_dim] in src_dtype
 *                  (F32/F16/BF16), strides as for pkv_reshape_and_cache
 *   k_codes, v_codes device int8 [num_blocks][num_kv_heads][block_size][head_dim]
 *   k_scale, v_scale device float [num_blocks][num_kv_heads]
 *   slot_mapping   device int32[num_tokens]; -1 skips a token.  A block may
 *                  receive at most one run per call (PKV_VALIDATE=1 checks
 *                  this and rejects slots outside the pool or repeated;
 *                  otherwise such slots are skipped and two runs into one
 *                  block give unspecified codes).
 * head_dim must be a multiple of 16.  Bit-exact against the float32
 * definition. */
pkv_status pkv_reshape_and_cache_int8(const void* key, const void* value, pkv_dtype src_dtype,
                                      int8_t* k_codes, int8_t* v_codes, float* k_scale,
                                      float* v_scale, const int32_t* slot_mapping,
                                      int32_t num_tokens, int64_t key_stride,
                                      int64_t value_stride, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                      void* stream);

/* reshape_and_cache into 4-bit storage: pkv_reshape_and_cache_int8 with
 * codes in [-7, 7] packed two per byte as PKV_I4 states; the grow-only
 * scale becomes max(old scale, max|new rows| / 7), existing codes are
 * re-encoded to [-7, 7] when it grows ([cnnetsun] §3.2 lists 4-bit KV).
 *   k_codes, v_codes device uint8 [num_blocks][num_kv_heads][block_size]
 *                  [head_dim / 2], 16-byte aligned
 * Other arguments, validation and the one-run-per-block rule as for
 * pkv_reshape_and_cache_int8.  head_dim must be a multiple of 32.
 * Bit-exact against the float32 definition. */
pkv_status pkv_reshape_and_cache_int4(const void* key, const void* value, pkv_dtype src_dtype,
                                      uint8_t* k_codes, uint8_t* v_codes, float* k_scale,
                                      float* v_scale, const int32_t* slot_mapping,
                                      int32_t num_tokens, int64_t key_stride,
                                      int64_t value_stride, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                      void* stream);

/* ------------------------------------------------------------------------
 * copy_blocks (device): the data copy of copy-on-write ([kongchang] section
 * "KV Cache内存共享").  For each pair (src, dst): K[dst] = K[src],
 * V[dst] = V[src], and for I8 and I4 storage k_scale[dst] = k_scale[src],
 * same for v_scale (scales may be NULL otherwise).
 *   pairs   device int32[num_pairs][2].  Destinations must be distinct and
 *           never a source of the same call (validated with PKV_VALIDATE=1).
 * Bit-exact. */
pkv_status pkv_copy_blocks(void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                           const int32_t* pairs, int32_t num_pairs, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, int32_t num_blocks,
                           pkv_dtype dtype, void* stream);

/* ------------------------------------------------------------------------
 * swap_blocks: preemption by swapping moves a preempted request's KV blocks
 * over PCIe from GPU memory to CPU memory and back when it resumes
 * ([kongchang] section "抢占与恢复机制"; cold pages may live in host memory,
 * [cnnetsun] §2.3).  For each pair (s, d): block d of the destination pool
 * receives block s of the source pool (K, V, and for I8 and I4 storage the
 * per-(block, kv head) scales); other destination blocks are unchanged.
 *   dst_*, src_*   pools [num_blocks][num_kv_heads][block_size][head_dim] in
 *                  `dtype`, each in device memory or in pinned host memory
 *                  (hipHostMalloc; pageable host memory works but copies
 *                  synchronously); the two pools never overlap
 *   *_scale        float [num_blocks][num_kv_heads], I8 and I4 only (else NULL)
 *   pairs          HOST int32[num_pairs][2] (source block, destination block);
 *                  always validated: ids inside their pools, destinations
 *                  distinct (INVALID otherwise, nothing copied)
 *   workspace      device scratch, 256-byte aligned, or NULL.  Between device
 *                  and host pools the scattered device blocks are gathered
 *                  into it (or scattered from it) by a copy kernel, so the
 *                  PCIe side moves runs of consecutive host blocks; it holds
 *                  as many blocks per round as fit (at least one block, else
 *                  INVALID), pkv_swap_workspace_bytes(n, ...) covers n pairs
 *                  in one round.  With NULL, each run of consecutive pairs
 *                  is one DMA copy.  Between two device pools the copy is a
 *                  kernel (block ids through the workspace when given).
 * The copies run asynchronously on `stream` (DMA engines for host memory);
 * the caller keeps the host pool and the workspace alive until the stream
 * has passed them.  Bit-exact. */
pkv_status pkv_swap_blocks(void* dst_k, void* dst_v, float* dst_k_scale, float* dst_v_scale,
                           int32_t dst_num_blocks, const void* src_k, const void* src_v,
                           const float* src_k_scale, const float* src_v_scale,
                           int32_t src_num_blocks, const int32_t* pairs, int32_t num_pairs,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           pkv_dtype dtype, void* workspace, size_t workspace_bytes,
                           void* stream);
/* Workspace bytes for swapping up to max_pairs blocks in one round. */
size_t pkv_swap_workspace_bytes(int32_t max_pairs, int32_t num_kv_heads, int32_t head_dim,
                                int32_t block_size, pkv_dtype dtype);

/* Process-wide counters of pkv_swap_blocks, for the swap-rate health metric
 * of [cnnetsun] §4.2 (page swaps per second; frequent swapping calls for
 * larger pages): successful calls, blocks moved by direction, and bytes
 * (K and V, with int8 scales).  The caller divides by its own clock.  A
 * non-zero `reset` zeroes them after reading. */
typedef struct pkv_swap_stats {
  int64_t calls;
  int64_t blocks_to_host;
  int64_t blocks_to_device;
  int64_t blocks_device_to_device;
  int64_t blocks_host_to_host;
  int64_t bytes;
} pkv_swap_stats;
pkv_status pkv_swap_stats_get(pkv_swap_stats* out, int32_t reset);

/* ------------------------------------------------------------------------
 * quantize_blocks (device): int8 storage of whole blocks.  cnnetsun.cn §3.2
 * (内存压缩技术) lists INT8 KV at a quarter of fp32's bytes, and §4.3
 * (典型场景优化策略) keeps the historical pages of long documents in INT8.
 * For each listed block b (dst block b <- src block b) and KV head h, over
 * the first filled[i] rows of the tile:
 *     s = max|x| / 127                      (float32, IEEE division)
 *     code = rint(x / s), clamped to [-127, 127]  (ties to even)
 * rows past filled[i] get code 0; a block whose scale is below the smallest
 * normal float32 (values all below ~1.5e-36) stores s = 0 and all-zero codes;
 * filled[i] == 0 leaves block b untouched.  The result is bit-exact: every
 * step is float32 arithmetic.  The int8 pool then serves decode through
 * pkv_paged_attention_decode with kv_dtype I8.
 *   src_k, src_v   device pools [num_blocks][num_kv_heads][block_size][head_dim]
 *                  in src_dtype (F32, F16 or BF16), finite values
 *   dst_k, dst_v   device int8 pools of the same shape (may be other tensors
 *                  than the sources, never overlapping them)
 *   k_scale, v_scale device float[num_blocks][num_kv_heads], written for the
 *                  listed blocks
 *   blocks, filled device int32[num_listed]: distinct block ids, and filled
 *                  row counts in [0, block_size] (validated with PKV_VALIDATE=1;
 *                  otherwise ids outside the pool are skipped and counts are
 *                  clamped to block_size)
 * Requires head_dim * element size to be a multiple of 16 bytes. */
pkv_status pkv_quantize_blocks(const void* src_k, const void* src_v, pkv_dtype src_dtype,
                               int8_t* dst_k, int8_t* dst_v, float* k_scale, float* v_scale,
                               const int32_t* blocks, const int32_t* filled, int32_t num_listed,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t num_blocks, void* stream);

/* 4-bit storage of whole blocks: pkv_quantize_blocks with codes in [-7, 7]
 * and s = max|x| / 7 (float32), packed two per byte as PKV_I4 states.
 * [cnnetsun] §3.2 lists 4-bit KV at an eighth of fp32's bytes.  Arguments
 * as for pkv_quantize_blocks, except
 *   dst_k, dst_v   device uint8 pools [num_blocks][num_kv_heads][block_size]
 *                  [head_dim / 2], 4-byte aligned
 * head_dim must be even and head_dim * source element size a multiple of 16
 * bytes.  Bit-exact against the float32 definition; the pool serves decode
 * with kv_dtype I4. */
pkv_status pkv_quantize_blocks_int4(const void* src_k, const void* src_v, pkv_dtype src_dtype,
                                    uint8_t* dst_k, uint8_t* dst_v, float* k_scale,
                                    float* v_scale, const int32_t* blocks, const int32_t* filled,
                                    int32_t num_listed, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t block_size, int32_t num_blocks, void* stream);

/* ------------------------------------------------------------------------
 * Paged decode attention (device).  One query token per sequence, at
 * position context_lens[s] - 1, attends keys [0, context_lens[s]) (the
 * current token's K/V is already in the cache).  For each table entry the
 * query is scored against that block, the scores of all blocks take one
 * softmax after scaling, and the blocks' value rows are summed with those
 * weights ([cnnetsun] §3.1).  Query head h reads KV head h / (Hq / Hkv).
 *   out            device [num_seqs][num_q_heads][head_dim] in out_dtype
 *                  (F32, or the q dtype); rows with context 0 are zero.
 *   q              device [num_seqs][num_q_heads][head_dim], q_dtype F32/F16/BF16
 *   k_cache,v_cache device pool in kv_dtype: F32/F16/BF16 (same as q), I8 or
 *                  I4 with k_scale/v_scale device float[num_blocks][num_kv_heads];
 *                  a stored element is code * scale of its (block, kv head)
 *   block_tables   device int32[num_seqs][max_blocks_per_seq]
 *   context_lens   device int32[num_seqs], each <= max_context_len
 *                  <= max_blocks_per_seq * block_size
 *   scale          multiplies q.k before the softmax (1/sqrt(head_dim) in
 *                  the usual case)
 *   partition_tokens  0: one workgroup covers a whole context; otherwise a
 *                  multiple of 16: contexts are split into partitions
 *                  of that many tokens, each producing a partial result
 *                  (max, sum, unnormalised output) that a reduce kernel
 *                  merges.  Results are deterministic for a fixed value.
 *   algo           PKV_ALGO_*, optionally OR-ed with PKV_KV_STREAM or
 *                  PKV_KV_CACHED; AUTO picks MFMA for grouped heads with
 *                  16-bit q, else the wavefront kernel.  The load policy
 *                  changes no result bit.
 *   workspace      device scratch of at least
 *                  pkv_decode_workspace_bytes(...) bytes (may be NULL when
 *                  that is 0), 256-byte aligned.
 * Supported: head_dim 64 or 128; block_size 16, 32, 64 or 128 (the kernels
 * walk a block as 16-row tiles; [cnnetsun] §4.3 gives 16-32 for many short
 * conversations and 64-128 for long documents); num_q_heads a multiple of
 * num_kv_heads with a group of at most 16.  Others: UNSUPPORTED. */
size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                  int32_t max_context_len, int32_t partition_tokens);

/* Partition size for a decode launch (host).  The keys of a context may be
 * split into partitions whose partial results merge into one softmax
 * ([cnnetsun] §3.1: a softmax over the scores of every page); how long the
 * partitions are is a choice of the launch, not of the method, and changes
 * results only by rounding.  A decode launch holds one workgroup per
 * (partition, row, workgroup of heads); when the grid needs one round of the
 * workgroups the GPU keeps resident plus a fraction of another, that
 * fraction runs with the GPU mostly idle.  This picks the shortest
 * partition (a multiple of 16 tokens, at least min_tokens) whose workgroups
 * fit in the whole rounds the launch needs without a split, so each round
 * is as full as it can be; 0 (no split) when no split fits in them.
 *   context_lens   host int32[num_seqs], each >= 0 (the lengths the decode
 *                  call will see on the device)
 *   workgroups_per_partition  workgroups a (partition, row) takes
 *   resident_workgroups       workgroups of the launch the GPU holds at once
 *   min_tokens     shortest partition allowed
 *   partition_tokens  out: the partition, or 0
 * Reads only host memory; INVALID for NULL pointers, negative lengths or
 * sizes, or non-positive workgroup counts. */
pkv_status pkv_decode_partition_for_capacity(const int32_t* context_lens, int32_t num_seqs,
                                             int32_t workgroups_per_partition,
                                             int64_t resident_workgroups, int32_t min_tokens,
                                             int32_t* partition_tokens);

/* pkv_decode_partition_for_capacity for the kernel a decode call with these
 * arguments launches on the current device: its resident workgroups come
 * from the runtime's occupancy query times the device's compute units, its
 * workgroups per (partition, row) from its heads per workgroup, and the
 * shortest partition is 256 tokens (1,024 for the 16-wave kernel of one head
 * of streamed 16-bit K/V, which runs only at partitions that long).  Pass
 * the result as partition_tokens to pkv_paged_attention_decode (or _step,
 * _partials), with pkv_decode_workspace_bytes for it.
 *   context_lens   host int32[num_seqs]
 *   q_dtype .. algo  as pkv_paged_attention_decode (num_blocks and
 *                  block_size decide the load policy the launch takes)
 *   partition_tokens  out
 * Errors: INVALID / UNSUPPORTED as the decode call would report them for
 * these types and sizes; DEVICE when the occupancy query fails. */
pkv_status pkv_decode_partition_tokens(const int32_t* context_lens, int32_t num_seqs,
                                       pkv_dtype q_dtype, pkv_dtype kv_dtype, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                       int32_t num_blocks, int32_t algo, int32_t* partition_tokens);

pkv_status pkv_paged_attention_decode(
    void* out, pkv_dtype out_dtype, const void* q, pkv_dtype q_dtype, const void* k_cache,
    const void* v_cache, pkv_dtype kv_dtype, const float* k_scale, const float* v_scale,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
    int32_t partition_tokens, int32_t algo, void* workspace, size_t workspace_bytes, void* stream);

/* One decode step: append the step's new token of every sequence, then
 * attend, in the attention kernel's launch ([nxbn] §1: only the new token's
 * K/V is computed and appended to the cache each step, then the query
 * attends over all of it; [nxbn] §2.2: its address comes from the block
 * table).
 *   new_k, new_v   device [num_seqs][num_kv_heads][head_dim] in kv_dtype
 *                  (F32/F16/BF16), or both NULL (no append).  Row s is the
 *                  K/V of sequence s's position context_lens[s] - 1: the
 *                  kernel writes it to that position's slot
 *                  (block_tables[s][p / block_size], row p % block_size) and
 *                  attends with it; a context of 0 appends nothing.  The
 *                  result is that of pkv_reshape_and_cache with those slots
 *                  followed by pkv_paged_attention_decode.  I8/I4 pools
 *                  append through quantise-on-write instead (UNSUPPORTED
 *                  here); pass NULL rows to decode them in one launch.
 *   Rows whose context spans several partitions are merged by the reduce
 *   kernel in a second launch, or, with PKV_MERGE_IN_KERNEL in algo, inside
 *   the attention launch by the last partition of the row to finish (a
 *   device-scope counter per row and head group; no workgroup waits).  Both
 *   merge in the same order, so the output has the same bits either way and
 *   as pkv_paged_attention_decode's.  On MI355X the separate reduce
 *   measured faster (the in-launch merge puts a row's whole merge, with
 *   reads that bypass the caches, in one workgroup at the launch's tail).
 *   workspace      device memory of pkv_decode_step_workspace_bytes(...)
 *                  bytes, 256-byte aligned: the partial results, then one
 *                  int32 arrival counter per (sequence, query head).  With
 *                  PKV_MERGE_IN_KERNEL the counters must be zero before the
 *                  first call that uses the workspace (allocate it
 *                  zero-filled); every call leaves them zero.  Calls that
 *                  share a workspace must not overlap.
 * Other arguments and rules: as pkv_paged_attention_decode. */
size_t pkv_decode_step_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                       int32_t max_context_len, int32_t partition_tokens);
pkv_status pkv_paged_attention_decode_step(
    void* out, pkv_dtype out_dtype, const void* q, pkv_dtype q_dtype, const void* new_k,
    const void* new_v, void* k_cache, void* v_cache, pkv_dtype kv_dtype, const float* k_scale,
    const float* v_scale, const int32_t* block_tables, int32_t max_blocks_per_seq,
    const int32_t* context_lens, int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
    int32_t partition_tokens, int32_t algo, void* workspace, size_t workspace_bytes, void* stream);

/* The two halves of pkv_paged_attention_decode, for callers that schedule
 * them separately.  _partials runs the main kernel only: sequences that fit
 * in one partition get their final output row, the others leave partial
 * results in the workspace.  _reduce merges those partials (log-sum-exp
 * rescaling of each partition's max and sum) into `out`; it reads
 * context_lens to know each sequence's partition count.  Same arguments and
 * rules as above; with partition_tokens 0 the reduce is a no-op. */
pkv_status pkv_paged_attention_decode_partials(
    void* out, pkv_dtype out_dtype, const void* q, pkv_dtype q_dtype, const void* k_cache,
    const void* v_cache, pkv_dtype kv_dtype, const float* k_scale, const float* v_scale,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
    int32_t partition_tokens, int32_t algo, void* workspace, size_t workspace_bytes, void* stream);

/* pkv_paged_attention_decode without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The split-K partial results go
 * to a scratch array of PKV_NOALLOC_SCRATCH_BYTES that the library holds in
 * device memory, one per GPU, from the first call on that GPU until the
 * process ends.  The call itself allocates nothing.
 *   Same arguments, kernels and results as pkv_paged_attention_decode (bit
 *   for bit, for the same partition_tokens and algo); the thread's current
 *   device must be the one `stream` runs on.
 *   A call whose partial results would need more than the scratch holds
 *   (pkv_decode_workspace_bytes(...) > PKV_NOALLOC_SCRATCH_BYTES) returns
 *   PKV_ERR_INVALID before any launch; larger partitions shrink the need.
 *   Nothing in the scratch must start at zero: every partial state a reduce
 *   reads is written earlier in the same call.
 *   Calls that overlap on one GPU (several streams, several threads) share
 *   its scratch and race: the caller serialises them. */
#define PKV_NOALLOC_SCRATCH_BYTES (64ull << 20)
pkv_status pkv_paged_attention_decode_noalloc(
    void* out, pkv_dtype out_dtype, const void* q, pkv_dtype q_dtype, const void* k_cache,
    const void* v_cache, pkv_dtype kv_dtype, const float* k_scale, const float* v_scale,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
    int32_t partition_tokens, int32_t algo, void* stream);

pkv_status pkv_paged_attention_reduce(void* out, pkv_dtype out_dtype, const int32_t* context_lens,
                                      int32_t max_context_len, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t head_dim,
                                      int32_t partition_tokens, const void* workspace,
                                      size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Chunked prefill attention (device).  Long prompts are processed in chunks
 * that share a batch with decode steps ([nxbn] §3.2; [cnnetsun] §4.1 turns
 * chunking on).  Sequence s owns query rows query_start_loc[s] ..
 * query_start_loc[s+1]-1, its last qlen positions: row i sits at position
 * context_lens[s] - qlen + i and attends keys [0, that position] (causal over
 * absolute positions).  The chunk's own K/V must already be in the cache
 * (pkv_reshape_and_cache first).
 *   out, q         device [num_query_tokens][num_q_heads][head_dim]
 *   query_start_loc device int32[num_seqs + 1], non-decreasing, from 0
 *   context_lens   device int32[num_seqs], each >= its chunk length
 *   max_query_len  the largest chunk (sizes the launch)
 *   partition_tokens  0: one workgroup walks all keys of its rows; otherwise
 *                  a multiple of 16: the keys are split into partitions of
 *                  that many tokens, processed by separate workgroups (so a
 *                  long context no longer serialises on one workgroup), and
 *                  rows whose keys span several partitions are merged by the
 *                  partition reduce (log-sum-exp, as for decode) before the
 *                  call returns.  Results for a fixed value are deterministic.
 *   workspace      device scratch of at least pkv_prefill_workspace_bytes(...)
 *                  bytes (may be NULL when that is 0), 256-byte aligned.
 * q_dtype F16/BF16 with kv_dtype equal to it (MFMA path), or F32 throughout
 * (wavefront path, one query row at a time).  Supported head_dim 64/128,
 * block_size 16/32/64/128, group (num_q_heads / num_kv_heads) of any size.
 * With num_query_tokens = 0 (no sequences, or only empty chunks) the call
 * checks its sizes and returns PKV_OK without launching; out and q may then
 * be NULL. */
size_t pkv_prefill_workspace_bytes(int32_t num_query_tokens, int32_t num_q_heads,
                                   int32_t head_dim, int32_t max_context_len,
                                   int32_t partition_tokens);

/* Key partition size for a chunked-prefill launch (host), the counterpart of
 * pkv_decode_partition_tokens: a matrix-core prefill workgroup owns 64 query
 * rows of one head, so sequence s takes ceil(query_lens[s] / 64) x
 * num_q_heads workgroups per partition of its keys; the result is the
 * shortest partition (a multiple of 16 tokens, at least 256) whose
 * workgroups fit in the whole rounds of two resident workgroups per compute
 * unit that the launch needs without a split, or 0 (no split).  Two, not the
 * three the kernel's LDS allows: with three the per-step time rises more
 * than the third workgroup adds (measured on long documents).  Many row
 * tiles already fill the GPU unsplit (0); a few long chunks get split.
 * fp32 q (the wavefront rows) always gets 0.
 *   query_lens, context_lens  host int32[num_seqs]: each sequence's chunk
 *                  length and its keys (context_lens[s] >= query_lens[s])
 *   partition_tokens  out
 * Errors: INVALID for NULL pointers or inconsistent lengths, UNSUPPORTED
 * for a q dtype prefill does not take, DEVICE without a current device. */
pkv_status pkv_prefill_partition_tokens(const int32_t* query_lens, const int32_t* context_lens,
                                        int32_t num_seqs, int32_t num_q_heads, pkv_dtype q_dtype,
                                        int32_t* partition_tokens);
pkv_status pkv_paged_attention_prefill(
    void* out, pkv_dtype out_dtype, const void* q, pkv_dtype q_dtype, const void* k_cache,
    const void* v_cache, pkv_dtype kv_dtype, const float* k_scale, const float* v_scale,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* query_start_loc,
    const int32_t* context_lens, int32_t max_query_len, int32_t max_context_len, int32_t num_seqs,
    int32_t num_query_tokens, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t num_blocks, float scale, int32_t partition_tokens,
    void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
