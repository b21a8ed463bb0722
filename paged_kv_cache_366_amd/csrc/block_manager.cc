// Host block manager: a fixed pool of KV blocks with a LIFO free list, one
// reference count per block, and sequences that own block tables.
//
// The pool and its stack-like free list follow the allocate() sketch of
// cnnetsun.cn "别再让GPU内存拖后腿了…" §2.1 (ids start in ascending order and
// are taken from the end); sharing through reference counts and
// copy-on-write follow kongchang.com "vLLM架构深度解析…", section
// "KV Cache内存共享", and aisoosoo.com "vLLM：大模型推理的加速引擎…", section
// "技术亮点"; blocks return to the pool when a request ends (m.nxbn.cn §2.3).
//
// Every mutating call is all-or-nothing: it first works out how many blocks
// it needs, fails with PKV_ERR_OUT_OF_BLOCKS before touching anything, and
// only then changes state.
//
// Prefix caching (cnnetsun.cn §2.2, share_prefix looks a prompt prefix up by
// a hash and attaches to its pages; aisoosoo.com section "技术亮点", equal
// prompt prefixes reuse KV pages): each full block that a sequence publishes
// is indexed under (physical block before it, or -1 for the first; its
// block_size token ids).  Chaining through the previous physical block makes
// one entry stand for the whole prefix up to it, so a lookup walks a prompt
// block by block and stops at the first miss.  The index keys on a 64-bit
// hash but every candidate's tokens are compared, so two prefixes never
// share a block by collision.  An entry lives exactly as long as its block
// is allocated: freeing the block (count 0) drops it, and the cache holds no
// reference of its own.
#include <algorithm>
#include <chrono>
#include <cstdlib>
#include <cstring>
#include <new>
#include <stdexcept>
#include <unordered_map>
#include <vector>

#include "status.h"

namespace {

thread_local std::string g_last_error;

struct Sequence {
  std::vector<int32_t> table;  // logical block j -> physical id
  int32_t len = 0;
};

// Index key of one published block.
struct PrefixKey {
  bool indexed = false;
  int32_t parent = -1;
  uint64_t hash = 0;
  std::vector<int32_t> tokens;
};

// splitmix64's finaliser (Steele, Lea and Flood, "Fast splittable
// pseudorandom number generators", OOPSLA 2014) as the mixing step.
uint64_t mix64(uint64_t x) {
  x += 0x9e3779b97f4a7c15ull;
  x = (x ^ (x >> 30)) * 0xbf58476d1ce4e5b9ull;
  x = (x ^ (x >> 27)) * 0x94d049bb133111ebull;
  return x ^ (x >> 31);
}

// Two token ids per mixing step.
uint64_t prefix_hash(int32_t parent, const int32_t* tokens, int32_t n) {
  uint64_t h = mix64(static_cast<uint64_t>(static_cast<int64_t>(parent) + 1));
  int32_t i = 0;
  for (; i + 1 < n; i += 2)
    h = mix64(h ^ (static_cast<uint64_t>(static_cast<uint32_t>(tokens[i + 1])) << 32 |
                   static_cast<uint32_t>(tokens[i])));
  if (i < n) h = mix64(h ^ static_cast<uint32_t>(tokens[i]));
  return h;
}

}  // namespace

namespace pkv {

pkv_status fail(pkv_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

pkv_status ok() { return PKV_OK; }

}  // namespace pkv

struct pkv_bm {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> free_list;  // bottom .. top; pop from the back
  std::vector<int32_t> rc;
  std::unordered_map<int64_t, Sequence> seqs;
  int64_t next_seq = 0;
  // prefix cache: hash -> block, and block -> its key
  std::unordered_multimap<uint64_t, int32_t> prefix_index;
  std::vector<PrefixKey> prefix_keys;  // per block; sized on the first publish
  int32_t prefix_count = 0;
  int64_t prefix_lookups = 0;
  int64_t prefix_hits = 0;
  // Durations of the latest calls that take blocks from the pool (alloc,
  // create, append), in nanoseconds: a ring of the last kLatencyWindow.
  static constexpr int32_t kLatencyWindow = 1 << 16;
  std::vector<uint32_t> latency_ns;
  int64_t latency_calls = 0;
  void record_latency(std::chrono::steady_clock::time_point t0) {
    const auto ns = std::chrono::duration_cast<std::chrono::nanoseconds>(
                        std::chrono::steady_clock::now() - t0)
                        .count();
    if (latency_ns.empty()) latency_ns.resize(kLatencyWindow);
    latency_ns[latency_calls % kLatencyWindow] =
        static_cast<uint32_t>(std::min<int64_t>(ns, UINT32_MAX));
    ++latency_calls;
  }

  int32_t blocks_for(int64_t tokens) const {
    return static_cast<int32_t>((tokens + block_size - 1) / block_size);
  }
  bool allocated(int32_t b) const { return b >= 0 && b < num_blocks && rc[b] > 0; }
  int32_t pop() {
    int32_t b = free_list.back();
    free_list.pop_back();
    rc[b] = 1;
    return b;
  }
  void release(int32_t b) {
    if (--rc[b] == 0) {
      free_list.push_back(b);
      if (prefix_count) unpublish(b);
    }
  }
  bool indexed(int32_t b) const { return prefix_count && prefix_keys[b].indexed; }
  void unpublish(int32_t b) {
    PrefixKey& k = prefix_keys[b];
    if (!k.indexed) return;
    auto range = prefix_index.equal_range(k.hash);
    for (auto it = range.first; it != range.second; ++it) {
      if (it->second == b) {
        prefix_index.erase(it);
        break;
      }
    }
    k.indexed = false;
    --prefix_count;
  }
  // Block indexed under (parent, tokens[0..block_size)), or -1.
  int32_t lookup(int32_t parent, const int32_t* tokens, uint64_t h) const {
    auto range = prefix_index.equal_range(h);
    for (auto it = range.first; it != range.second; ++it) {
      const PrefixKey& k = prefix_keys[it->second];
      if (k.parent == parent &&
          std::equal(k.tokens.begin(), k.tokens.end(), tokens))
        return it->second;
    }
    return -1;
  }
  Sequence* find(int64_t id) {
    auto it = seqs.find(id);
    return it == seqs.end() ? nullptr : &it->second;
  }
  const Sequence* find(int64_t id) const {
    auto it = seqs.find(id);
    return it == seqs.end() ? nullptr : &it->second;
  }
  // Blocks an append of `n` tokens to `s` will take, given the current
  // count of its tail block (`tail_rc`, ignored when the tail is full).
  int64_t append_need(const Sequence& s, int64_t n, int32_t tail_rc) const {
    if (n <= 0) return 0;
    int64_t need = blocks_for(s.len + n) - blocks_for(s.len);
    if (s.len % block_size != 0 && tail_rc > 1) need += 1;  // copy-on-write
    return need;
  }
  // One position; the caller has checked that enough blocks are free.
  int32_t append_one(Sequence& s, int32_t* cow_src, int32_t* cow_dst) {
    if (s.len % block_size == 0) {
      s.table.push_back(pop());
    } else if (rc[s.table.back()] > 1) {
      int32_t src = s.table.back();
      int32_t dst = pop();
      *cow_src = src;
      *cow_dst = dst;
      release(src);  // count > 1, so it stays allocated
      s.table.back() = dst;
    }
    int32_t slot = s.table[s.len / block_size] * block_size + s.len % block_size;
    s.len += 1;
    return slot;
  }
};

namespace {

// Times one allocating call of the block manager, success or failure.
struct AllocTimer {
  pkv_bm* bm;
  std::chrono::steady_clock::time_point t0 = std::chrono::steady_clock::now();
  explicit AllocTimer(pkv_bm* b) : bm(b) {}
  ~AllocTimer() {
    if (bm) bm->record_latency(t0);
  }
};

}  // namespace

extern "C" {

const char* pkv_last_error(void) { return g_last_error.c_str(); }

const char* pkv_version(void) { return "pkv 0.1 (gfx950)"; }

pkv_status pkv_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* init_free_order,
                         pkv_bm** out) {
  PKV_GUARD({
    if (!out) return pkv::fail(PKV_ERR_INVALID, "out is NULL");
    *out = nullptr;
    if (num_blocks <= 0 || block_size <= 0)
      return pkv::fail(PKV_ERR_INVALID, "num_blocks (%d) and block_size (%d) must be positive",
                       num_blocks, block_size);
    auto* bm = new pkv_bm();
    bm->num_blocks = num_blocks;
    bm->block_size = block_size;
    bm->rc.assign(num_blocks, 0);
    bm->free_list.resize(num_blocks);
    if (init_free_order) {
      std::vector<char> seen(num_blocks, 0);
      for (int32_t i = 0; i < num_blocks; ++i) {
        int32_t b = init_free_order[i];
        if (b < 0 || b >= num_blocks || seen[b]) {
          delete bm;
          return pkv::fail(PKV_ERR_INVALID, "init_free_order is not a permutation (entry %d = %d)",
                           i, b);
        }
        seen[b] = 1;
        bm->free_list[i] = b;
      }
    } else {
      for (int32_t i = 0; i < num_blocks; ++i) bm->free_list[i] = i;
    }
    *out = bm;
    return PKV_OK;
  })
}

void pkv_bm_destroy(pkv_bm* bm) { delete bm; }

pkv_status pkv_bm_alloc(pkv_bm* bm, int32_t n, int32_t* ids_out) {
  PKV_GUARD({
    AllocTimer timer(bm);
    if (!bm) return pkv::fail(PKV_ERR_INVALID, "bm is NULL");
    if (n < 0 || (n > 0 && !ids_out)) return pkv::fail(PKV_ERR_INVALID, "bad count or output");
    if (static_cast<size_t>(n) > bm->free_list.size())
      return pkv::fail(PKV_ERR_OUT_OF_BLOCKS, "need %d blocks, %zu free", n, bm->free_list.size());
    for (int32_t i = 0; i < n; ++i) ids_out[i] = bm->pop();
    return PKV_OK;
  })
}

pkv_status pkv_bm_incref(pkv_bm* bm, int32_t block) {
  if (!bm) return pkv::fail(PKV_ERR_INVALID, "bm is NULL");
  if (!bm->allocated(block)) return pkv::fail(PKV_ERR_INVALID, "block %d is not allocated", block);
  bm->rc[block] += 1;
  return PKV_OK;
}

pkv_status pkv_bm_decref(pkv_bm* bm, int32_t block) {
  PKV_GUARD({
    if (!bm) return pkv::fail(PKV_ERR_INVALID, "bm is NULL");
    if (!bm->allocated(block))
      return pkv::fail(PKV_ERR_INVALID, "block %d is not allocated", block);
    bm->release(block);
    return PKV_OK;
  })
}

int32_t pkv_bm_num_free(const pkv_bm* bm) {
  return bm ? static_cast<int32_t>(bm->free_list.size()) : -1;
}

pkv_status pkv_bm_get_state(const pkv_bm* bm, int32_t* free_list, int32_t* free_len,
                            int32_t* refcounts) {
  if (!bm) return pkv::fail(PKV_ERR_INVALID, "bm is NULL");
  if (free_list && !bm->free_list.empty())
    std::memcpy(free_list, bm->free_list.data(), bm->free_list.size() * sizeof(int32_t));
  if (free_len) *free_len = static_cast<int32_t>(bm->free_list.size());
  if (refcounts) std::memcpy(refcounts, bm->rc.data(), bm->rc.size() * sizeof(int32_t));
  return PKV_OK;
}

pkv_status pkv_bm_stats_get(const pkv_bm* bm, pkv_bm_stats* out) {
  if (!bm || !out) return pkv::fail(PKV_ERR_INVALID, "NULL argument");
  pkv_bm_stats s{};
  s.num_blocks = bm->num_blocks;
  s.block_size = bm->block_size;
  s.free_blocks = static_cast<int32_t>(bm->free_list.size());
  for (int32_t r : bm->rc) {
    s.used_blocks += r > 0;
    s.shared_blocks += r > 1;
  }
  s.num_seqs = static_cast<int32_t>(bm->seqs.size());
  for (const auto& kv : bm->seqs) {
    s.logical_blocks += static_cast<int64_t>(kv.second.table.size());
    s.tokens += kv.second.len;
  }
  s.waste_slots = s.logical_blocks * bm->block_size - s.tokens;
  *out = s;
  return PKV_OK;
}

pkv_status pkv_bm_latency_get(pkv_bm* bm, pkv_bm_latency* out, int32_t reset) {
  PKV_GUARD({
    if (!bm || !out) return pkv::fail(PKV_ERR_INVALID, "NULL argument");
    pkv_bm_latency r{};
    r.calls = bm->latency_calls;
    const int64_t w = std::min<int64_t>(bm->latency_calls, pkv_bm::kLatencyWindow);
    r.window = static_cast<int32_t>(w);
    if (w > 0) {
      std::vector<uint32_t> v(bm->latency_ns.begin(), bm->latency_ns.begin() + w);
      // nearest-rank percentiles: the ceil(p * w)-th smallest duration
      auto rank = [&](double p) {
        int64_t k = static_cast<int64_t>(p * static_cast<double>(w) + 0.999999999);
        k = std::max<int64_t>(1, std::min<int64_t>(k, w)) - 1;
        std::nth_element(v.begin(), v.begin() + k, v.end());
        return v[k] * 1e-3;
      };
      r.p50_us = rank(0.50);
      r.p99_us = rank(0.99);
      r.max_us = *std::max_element(v.begin(), v.end()) * 1e-3;
    }
    if (reset) bm->latency_calls = 0;
    *out = r;
    return PKV_OK;
  })
}

pkv_status pkv_seq_create(pkv_bm* bm, int32_t num_tokens, int64_t* seq_out) {
  PKV_GUARD({
    AllocTimer timer(bm);
    if (!bm || !seq_out) return pkv::fail(PKV_ERR_INVALID, "NULL argument");
    if (num_tokens < 0) return pkv::fail(PKV_ERR_INVALID, "negative length %d", num_tokens);
    int32_t nb = bm->blocks_for(num_tokens);
    if (static_cast<size_t>(nb) > bm->free_list.size())
      return pkv::fail(PKV_ERR_OUT_OF_BLOCKS, "need %d blocks, %zu free", nb,
                       bm->free_list.size());
    Sequence s;
    s.table.reserve(nb);
    s.len = num_tokens;
    for (int32_t i = 0; i < nb; ++i) s.table.push_back(bm->pop());
    int64_t id = bm->next_seq++;
    bm->seqs.emplace(id, std::move(s));
    *seq_out = id;
    return PKV_OK;
  })
}

int32_t pkv_adaptive_block_size(double avg_context_len) {
  if (!(avg_context_len >= 512.0)) return 16;  // NaN and negatives too
  return avg_context_len < 2048.0 ? 32 : 64;
}

pkv_status pkv_seq_create_cached(pkv_bm* bm, const int32_t* tokens, int32_t num_tokens,
                                 int64_t* seq_out, int32_t* cached_out) {
  PKV_GUARD({
    AllocTimer timer(bm);
    if (!bm || !seq_out || (num_tokens > 0 && !tokens))
      return pkv::fail(PKV_ERR_INVALID, "NULL argument");
    if (num_tokens < 0) return pkv::fail(PKV_ERR_INVALID, "negative length %d", num_tokens);
    const int32_t bs = bm->block_size;
    const int32_t full = num_tokens / bs;
    std::vector<int32_t> shared;
    int32_t parent = -1;
    for (int32_t j = 0; j < full && !bm->prefix_index.empty(); ++j) {
      const int32_t* t = tokens + static_cast<int64_t>(j) * bs;
      int32_t b = bm->lookup(parent, t, prefix_hash(parent, t, bs));
      if (b < 0) break;
      shared.push_back(b);
      parent = b;
    }
    int32_t need = bm->blocks_for(num_tokens) - static_cast<int32_t>(shared.size());
    if (static_cast<size_t>(need) > bm->free_list.size())
      return pkv::fail(PKV_ERR_OUT_OF_BLOCKS, "need %d blocks, %zu free", need,
                       bm->free_list.size());
    for (int32_t b : shared) bm->rc[b] += 1;
    Sequence s;
    s.table = std::move(shared);
    s.len = num_tokens;
    const int32_t hit = static_cast<int32_t>(s.table.size());
    for (int32_t i = 0; i < need; ++i) s.table.push_back(bm->pop());
    int64_t id = bm->next_seq++;
    bm->seqs.emplace(id, std::move(s));
    bm->prefix_lookups += full;
    bm->prefix_hits += hit;
    *seq_out = id;
    if (cached_out) *cached_out = hit * bs;
    return PKV_OK;
  })
}

pkv_status pkv_seq_publish(pkv_bm* bm, int64_t seq, const int32_t* tokens, int32_t num_tokens,
                           int32_t* added_out) {
  PKV_GUARD({
    if (!bm || (num_tokens > 0 && !tokens)) return pkv::fail(PKV_ERR_INVALID, "NULL argument");
    const Sequence* s = bm->find(seq);
    if (!s) return pkv::fail(PKV_ERR_INVALID, "unknown sequence %lld", (long long)seq);
    if (num_tokens < 0 || num_tokens > s->len)
      return pkv::fail(PKV_ERR_INVALID, "%d tokens for a sequence of %d", num_tokens, s->len);
    const int32_t bs = bm->block_size;
    int32_t added = 0;
    for (int32_t j = 0; j < num_tokens / bs; ++j) {
      const int32_t b = s->table[j];
      const int32_t parent = j ? s->table[j - 1] : -1;
      const int32_t* t = tokens + static_cast<int64_t>(j) * bs;
      if (bm->indexed(b)) continue;
      const uint64_t h = prefix_hash(parent, t, bs);
      if (bm->lookup(parent, t, h) >= 0) continue;
      if (bm->prefix_keys.empty()) bm->prefix_keys.resize(bm->num_blocks);
      PrefixKey& k = bm->prefix_keys[b];
      k.indexed = true;
      k.hash = h;
      k.parent = parent;
      k.tokens.assign(t, t + bs);
      bm->prefix_index.emplace(h, b);
      ++bm->prefix_count;
      ++added;
    }
    if (added_out) *added_out = added;
    return PKV_OK;
  })
}

pkv_status pkv_bm_prefix_stats(const pkv_bm* bm, int64_t* lookups, int64_t* hits,
                               int32_t* cached_blocks) {
  if (!bm) return pkv::fail(PKV_ERR_INVALID, "bm is NULL");
  if (lookups) *lookups = bm->prefix_lookups;
  if (hits) *hits = bm->prefix_hits;
  if (cached_blocks) *cached_blocks = bm->prefix_count;
  return PKV_OK;
}

pkv_status pkv_seq_fork(pkv_bm* bm, int64_t parent, int64_t* child_out) {
  PKV_GUARD({
    if (!bm || !child_out) return pkv::fail(PKV_ERR_INVALID, "NULL argument");
    const Sequence* p = bm->find(parent);
    if (!p) return pkv::fail(PKV_ERR_INVALID, "unknown sequence %lld", (long long)parent);
    Sequence c = *p;
    for (int32_t b : c.table) bm->rc[b] += 1;
    int64_t id = bm->next_seq++;
    bm->seqs.emplace(id, std::move(c));
    *child_out = id;
    return PKV_OK;
  })
}

pkv_status pkv_seq_append(pkv_bm* bm, int64_t seq, int32_t num_tokens, int32_t* slots_out,
                          int32_t* cow_src, int32_t* cow_dst) {
  PKV_GUARD({
    AllocTimer timer(bm);
    if (!bm) return pkv::fail(PKV_ERR_INVALID, "bm is NULL");
    Sequence* s = bm->find(seq);
    if (!s) return pkv::fail(PKV_ERR_INVALID, "unknown sequence %lld", (long long)seq);
    if (num_tokens < 0 || (num_tokens > 0 && !slots_out))
      return pkv::fail(PKV_ERR_INVALID, "bad count or output");
    if (static_cast<int64_t>(s->len) + num_tokens > INT32_MAX / 2)
      return pkv::fail(PKV_ERR_INVALID, "sequence too long");
    int32_t tail_rc = s->table.empty() ? 0 : bm->rc[s->table.back()];
    int64_t need = bm->append_need(*s, num_tokens, tail_rc);
    if (need > static_cast<int64_t>(bm->free_list.size()))
      return pkv::fail(PKV_ERR_OUT_OF_BLOCKS, "need %lld blocks, %zu free", (long long)need,
                       bm->free_list.size());
    int32_t src = -1, dst = -1;
    for (int32_t i = 0; i < num_tokens; ++i) slots_out[i] = bm->append_one(*s, &src, &dst);
    if (cow_src) *cow_src = src;
    if (cow_dst) *cow_dst = dst;
    return PKV_OK;
  })
}

pkv_status pkv_seq_append_batch(pkv_bm* bm, const int64_t* seqs, int32_t n, int32_t* slots_out,
                                int32_t* cow_pairs_out, int32_t* num_cow_out) {
  PKV_GUARD({
    AllocTimer timer(bm);
    if (!bm) return pkv::fail(PKV_ERR_INVALID, "bm is NULL");
    if (n < 0 || (n > 0 && (!seqs || !slots_out || !cow_pairs_out)))
      return pkv::fail(PKV_ERR_INVALID, "bad count or NULL array");
    std::vector<Sequence*> ss(n);
    std::unordered_map<int64_t, int> seen;
    for (int32_t i = 0; i < n; ++i) {
      ss[i] = bm->find(seqs[i]);
      if (!ss[i]) return pkv::fail(PKV_ERR_INVALID, "unknown sequence %lld", (long long)seqs[i]);
      if (seen[seqs[i]]++)
        return pkv::fail(PKV_ERR_INVALID, "sequence %lld appears twice", (long long)seqs[i]);
    }
    // Count the blocks the batch needs, tracking the count drops that earlier
    // copies cause on a tail shared with later members of the batch.
    std::unordered_map<int32_t, int32_t> rc_after;
    int64_t need = 0;
    for (int32_t i = 0; i < n; ++i) {
      const Sequence& s = *ss[i];
      if (s.len % bm->block_size == 0) {
        need += 1;
        continue;
      }
      int32_t tail = s.table.back();
      auto it = rc_after.find(tail);
      int32_t r = it == rc_after.end() ? bm->rc[tail] : it->second;
      if (r > 1) {
        need += 1;
        rc_after[tail] = r - 1;
      }
    }
    if (need > static_cast<int64_t>(bm->free_list.size()))
      return pkv::fail(PKV_ERR_OUT_OF_BLOCKS, "need %lld blocks, %zu free", (long long)need,
                       bm->free_list.size());
    int32_t ncow = 0;
    for (int32_t i = 0; i < n; ++i) {
      int32_t src = -1, dst = -1;
      slots_out[i] = bm->append_one(*ss[i], &src, &dst);
      if (src >= 0) {
        cow_pairs_out[2 * ncow] = src;
        cow_pairs_out[2 * ncow + 1] = dst;
        ++ncow;
      }
    }
    if (num_cow_out) *num_cow_out = ncow;
    return PKV_OK;
  })
}

pkv_status pkv_seq_slots(const pkv_bm* bm, int64_t seq, int32_t start, int32_t count,
                         int32_t* slots_out) {
  if (!bm) return pkv::fail(PKV_ERR_INVALID, "bm is NULL");
  const Sequence* s = bm->find(seq);
  if (!s) return pkv::fail(PKV_ERR_INVALID, "unknown sequence %lld", (long long)seq);
  if (start < 0 || count < 0 || static_cast<int64_t>(start) + count > s->len ||
      (count > 0 && !slots_out))
    return pkv::fail(PKV_ERR_INVALID, "positions [%d, %d) outside [0, %d)", start, start + count,
                     s->len);
  for (int32_t i = 0; i < count; ++i) {
    int32_t p = start + i;
    slots_out[i] = s->table[p / bm->block_size] * bm->block_size + p % bm->block_size;
  }
  return PKV_OK;
}

pkv_status pkv_seq_len(const pkv_bm* bm, int64_t seq, int32_t* len_out) {
  if (!bm || !len_out) return pkv::fail(PKV_ERR_INVALID, "NULL argument");
  const Sequence* s = bm->find(seq);
  if (!s) return pkv::fail(PKV_ERR_INVALID, "unknown sequence %lld", (long long)seq);
  *len_out = s->len;
  return PKV_OK;
}

pkv_status pkv_seq_free(pkv_bm* bm, int64_t seq) {
  PKV_GUARD({
    if (!bm) return pkv::fail(PKV_ERR_INVALID, "bm is NULL");
    auto it = bm->seqs.find(seq);
    if (it == bm->seqs.end())
      return pkv::fail(PKV_ERR_INVALID, "unknown sequence %lld", (long long)seq);
    for (int32_t b : it->second.table) bm->release(b);
    bm->seqs.erase(it);
    return PKV_OK;
  })
}

pkv_status pkv_seq_export(const pkv_bm* bm, const int64_t* seqs, int32_t n, int32_t max_blocks,
                          int32_t* tables_out, int32_t* lens_out) {
  if (!bm) return pkv::fail(PKV_ERR_INVALID, "bm is NULL");
  if (n < 0 || max_blocks < 0 || (n > 0 && (!seqs || (!tables_out && max_blocks > 0))))
    return pkv::fail(PKV_ERR_INVALID, "bad count or NULL array");
  for (int32_t i = 0; i < n; ++i) {
    const Sequence* s = bm->find(seqs[i]);
    if (!s) return pkv::fail(PKV_ERR_INVALID, "unknown sequence %lld", (long long)seqs[i]);
    if (static_cast<int64_t>(s->table.size()) > max_blocks)
      return pkv::fail(PKV_ERR_INVALID, "sequence %lld holds %zu blocks > max_blocks %d",
                       (long long)seqs[i], s->table.size(), max_blocks);
  }
  for (int32_t i = 0; i < n; ++i) {
    const Sequence* s = bm->find(seqs[i]);
    int32_t* row = tables_out ? tables_out + static_cast<int64_t>(i) * max_blocks : nullptr;
    if (row) {
      std::fill(row, row + max_blocks, -1);
      std::copy(s->table.begin(), s->table.end(), row);
    }
    if (lens_out) lens_out[i] = s->len;
  }
  return PKV_OK;
}

}  // extern "C"
