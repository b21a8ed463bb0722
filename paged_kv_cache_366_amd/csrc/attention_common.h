// Arguments and small helpers shared by the paged attention kernels.
#pragma once

#include "device_common.h"

namespace pkv {

// Output element kinds (runtime: the store is once per output element).
enum OutKind : int { kOutF32 = 0, kOutBF16 = 1, kOutF16 = 2 };

struct AttnArgs {
  void* out;                 // [rows][Hq][D] final output
  float* part_o;             // [rows][num_parts][Hq][D] partial outputs (NULL: no split)
  float* part_ml;            // [rows][num_parts][Hq][2] partial (max, sum), log2 domain
  const void* q;             // [rows][Hq][D]
  const void* kc;            // [NB][Hkv][16 << bs_shift][D]
  const void* vc;
  const float* ks;           // [NB][Hkv] int8 scales (NULL otherwise)
  const float* vs;
  const int32_t* tables;     // [S][MB]
  const int32_t* lens;       // [S]
  const int32_t* qsl;        // [S+1] query_start_loc; NULL means one query row per sequence
  int max_blocks;            // MB
  int bs_shift;              // block_size = 16 << bs_shift rows
  int max_ctx;
  int num_seqs;              // S
  int num_rows;              // S (decode) or Tq (prefill)
  int hq, hkv, num_blocks;
  int num_parts;             // partitions per row in the grid (1 = no split)
  int part_tokens;           // tokens per partition (multiple of 16)
  int out_kind;
  float scale_log2;          // scale * log2(e): scores are kept in the log2 domain
  bool stream_kv;            // decode K/V loads carry the non-temporal hint
  // Decode step extras (NULL when unused):
  const void* new_k;         // [S][Hkv][D] the step's K row of each sequence, written to
  const void* new_v;         //   position lens[s] - 1 and attended from these buffers
  int32_t* counters;         // [rows][Hq] arrivals per (row, first head of the group);
                             //   non-NULL: the last partition to finish merges the row
};

// Which sequence a query row belongs to.  Decode: row s is sequence s.
// Chunked prefill: the sequence whose query range [qsl[s], qsl[s+1]) holds
// the row.
__device__ __forceinline__ int row_seq(const AttnArgs& a, int row) {
  if (a.qsl == nullptr) return row;
  int lo = 0, hi = a.num_seqs - 1;  // largest s with qsl[s] <= row
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.qsl[mid] <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// The number of keys a query row attends.  Decode: keys [0, lens[s]).
// Chunked prefill: row i of sequence s's chunk sits at position
// lens[s] - qlen + i and attends keys [0, that position].  The result is
// clamped to what the table and max_ctx can address, so no read leaves the
// table row.
__device__ __forceinline__ int row_ctx(const AttnArgs& a, int row, int seq) {
  int ctx = a.lens[seq];
  if (a.qsl != nullptr) {
    const int qlen = a.qsl[seq + 1] - a.qsl[seq];
    ctx = ctx - qlen + (row - a.qsl[seq]) + 1;
  }
  const int cap = min(a.max_ctx, a.max_blocks << (4 + a.bs_shift));
  return max(0, min(ctx, cap));
}

// The kernels walk a context in tiles of 16 rows.  A block of
// 16 << bs_shift rows holds 1 << bs_shift of them: tile t of a sequence is in
// table entry t >> bs_shift, and the (block, KV head) slab of rows is
// contiguous, so the tile's index in units of 16 rows x head_dim is the one
// returned here.
__device__ __forceinline__ int64_t tile_index(const AttnArgs& a, int entry, int kvh, int t) {
  return ((static_cast<int64_t>(entry) * a.hkv + kvh) << a.bs_shift) +
         (t & ((1 << a.bs_shift) - 1));
}

__device__ __forceinline__ void row_context(const AttnArgs& a, int row, int& seq, int& ctx) {
  seq = row_seq(a, row);
  ctx = row_ctx(a, row, seq);
}

// Workgroups of the decode kernels.  Each owns one (query row, context
// partition, head group); the head group varies fastest along the grid.
// The tiles of all KV heads of one block are adjacent in the pool, so the
// workgroups that run together read neighbouring 4 KiB tiles of a few
// blocks, and their reads spread over every memory channel.  (With the head
// as the slow index, concurrent reads all sit at one offset modulo the
// block stride and crowd a few channels: on MI355X that costs about a
// quarter of the bandwidth.)
//
// A split decode launch (one row per sequence, several partitions) sizes
// its grid by the longest context, so shorter rows leave workgroups with no
// keys.  Those exit, but only once their first loads return, which under
// a full memory system takes microseconds: placed among the rows they
// would hold slots that later partitions wait for.  So the grid lists the
// used (row, partition) pairs first, row by row, and the empty workgroups
// after all of them.  Each wave finds its pair from the partition counts of
// all rows (a prefix sum over the context lengths, 256 rows per round of
// loads); `row` is -1 for an empty workgroup.  Past kCompactRowsMax rows the
// scan would cost every workgroup more dependent loads than the empty ones
// cost, so such launches keep the direct map (the library's partition
// choice splits only batches far smaller).

struct WgCoord {
  int row, part, hg;
};
constexpr int kCompactRowsMax = 1024;

__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(v, d);
    if (lane >= d) v += t;
  }
  return v;
}

__device__ __forceinline__ WgCoord wg_coord(const AttnArgs& a, int ngroups) {
  WgCoord c;
  const int bid = blockIdx.x;
  c.hg = bid % ngroups;
  const int idx = bid / ngroups;
  if (a.num_parts <= 1 || a.qsl != nullptr || a.num_rows > kCompactRowsMax) {
    c.part = idx % a.num_parts;
    c.row = idx / a.num_parts;
    return c;
  }
  const int lane = threadIdx.x & 63;
  const int cap = min(a.max_ctx, a.max_blocks << (4 + a.bs_shift));   // as row_ctx
  const int pt = a.part_tokens;
  int base = 0;   // partitions of the rows before this round
  for (int r0 = 0; r0 < a.num_rows; r0 += 256) {
    int n[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = r0 + 64 * j + lane;
      n[j] = r < a.num_rows ? a.lens[r] : -1;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // partitions of each row (a row with no keys still takes one, which
      // writes its zero output)
      const int cnt = n[j] < 0 ? 0 : max(1, (max(0, min(n[j], cap)) + pt - 1) / pt);
      const int incl = wave_incl_scan(cnt);
      // lane reads: the branch and the results are the same on every lane,
      // so they stay in scalar registers, as do the addresses derived from
      // them (read through a lane shuffle they would not)
      const int total = __builtin_amdgcn_readlane(incl, 63);
      if (idx < base + total) {
        const unsigned long long hit = __ballot(base + incl > idx);
        const int l = __ffsll(hit) - 1;
        c.row = r0 + 64 * j + l;
        c.part = idx - base - __builtin_amdgcn_readlane(incl - cnt, l);
        return c;
      }
      base += total;
    }
  }
  c.row = -1;
  c.part = 0;
  return c;
}

// Block-table entries of one wavefront's share of a partition.  Wave w of
// a workgroup of nw waves takes the partition's 16-row tiles w, w + nw,
// w + 2nw, ...; its k-th tile is tile `b0 + w + nw k` of the sequence, in
// table entry (b0 + w + nw k) >> bs_shift.  Lane i holds the entry for
// k = k0 + i, so one vector load covers 64 of the wave's tiles and each step
// reads its block id with a lane read, off the load path.  Tiles at or past
// `bmax` (the end of the partition or of the table row) read no entry.
struct TableChunk {
  int entry = -1;
  __device__ __forceinline__ void fetch(const int32_t* trow, int b0, int wave, int nw, int k0,
                                        int bmax, int bs_shift) {
    const int bi = wave + nw * (k0 + static_cast<int>(threadIdx.x & 63));
    entry = bi < bmax ? trow[(b0 + bi) >> bs_shift] : -1;
  }
  // Entry of the wave's tile k (k0 <= k < k0 + 64); k is wave-uniform.
  __device__ __forceinline__ int get(int k) const { return __builtin_amdgcn_readlane(entry, k & 63); }
};

__device__ __forceinline__ void store_out(const AttnArgs& a, int64_t idx, float v) {
  if (a.out_kind == kOutF32)
    static_cast<float*>(a.out)[idx] = v;
  else if (a.out_kind == kOutBF16)
    static_cast<uint16_t*>(a.out)[idx] = static_cast<uint16_t>(f32_to_bf16_bits(v));
  else
    static_cast<uint16_t*>(a.out)[idx] = f32_to_f16_bits(v);
}

// Merge of two (max, sum) softmax states in the log2 domain: returns the
// factors that rescale each side to the common max.  A side that has seen
// no key yet has max -inf and gets factor 0.
__device__ __forceinline__ void merge_factors(float m1, float m2, float& m, float& f1, float& f2) {
  m = fmaxf(m1, m2);
  const float ms = (m == kNegInf) ? 0.f : m;
  f1 = fast_exp2(m1 - ms);
  f2 = fast_exp2(m2 - ms);
}

// Index of the partial state of (query row, head, partition) in part_o (in
// units of D floats) and part_ml (pairs).  Partitions sit outside heads, so
// the heads a workgroup merges for one partition are adjacent: a
// grouped-query workgroup writes one contiguous run (8 heads x 128 floats)
// and one run of (max, sum) pairs, not one per head.
__device__ __forceinline__ int64_t part_slot(const AttnArgs& a, int64_t row, int h, int part) {
  return (row * a.num_parts + part) * a.hq + h;
}

// Canonical merge of the split-K partial states of one (row, head): with
// M = max_p m_p and f_p = 2^(m_p - M), L = sum_p l_p f_p taken in partition
// order p = 0, 1, ..., and O[d] = (sum over the first ceil(P / 2)
// partitions) + (sum over the rest), each half in partition order, with one
// fused multiply-add per term; the row is O / L (0 when L = 0).
// Every merger (the reduce kernel, the last workgroup of a row) runs these
// same steps, so all give the same bits for a fixed partition size.
struct PartMerge {
  float ms;   // M, or 0 when no partition saw a key
  float L;
};
// Loads of partial states.  Coherent: device-scope atomic loads, which read
// past the caches of this XCD (another workgroup of the same launch wrote
// them); otherwise plain loads (a later launch).  The value is the same.
template <bool Coherent>
__device__ __forceinline__ float load_part(const float* p) {
  if constexpr (Coherent)
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    return *p;
}
template <bool Coherent = false>
__device__ __forceinline__ PartMerge merge_ml(const AttnArgs& a, int64_t row, int h, int nparts) {
  const float* ml = a.part_ml + part_slot(a, row, h, 0) * 2;
  const int64_t st = 2 * static_cast<int64_t>(a.hq);   // floats between partitions' pairs
  float M = kNegInf;
  for (int p = 0; p < nparts; ++p) M = fmaxf(M, load_part<Coherent>(ml + p * st));
  PartMerge r;
  r.ms = (M == kNegInf) ? 0.f : M;
  r.L = 0.f;
  for (int p = 0; p < nparts; ++p)
    r.L = fmaf(load_part<Coherent>(ml + p * st + 1),
               fast_exp2(load_part<Coherent>(ml + p * st) - r.ms), r.L);
  return r;
}
template <bool Coherent = false>
__device__ __forceinline__ float merge_elem(const AttnArgs& a, int64_t row, int h, int nparts,
                                            const PartMerge& pm, int d, int D) {
  const float* ml = a.part_ml + part_slot(a, row, h, 0) * 2;
  const float* po = a.part_o + part_slot(a, row, h, 0) * D + d;
  const int64_t st = 2 * static_cast<int64_t>(a.hq);
  const int64_t so = static_cast<int64_t>(a.hq) * D;   // floats between partitions' rows
  // two halves of the partitions, each summed in order, then added
  const int half = (nparts + 1) >> 1;
  float O[2] = {0.f, 0.f};
#pragma unroll
  for (int g = 0; g < 2; ++g)
    for (int p = g * half; p < min(nparts, (g + 1) * half); ++p)
      O[g] = fmaf(load_part<Coherent>(po + p * so),
                  fast_exp2(load_part<Coherent>(ml + p * st) - pm.ms), O[g]);
  return pm.L > 0.f ? (O[0] + O[1]) / pm.L : 0.f;
}

// Last-arriver merge inside a decode kernel.  Each workgroup of a row whose
// context spans several partitions has written its partial state with
// device-scope atomic stores (finish_rows, when counters are set), which
// write through the caches of its XCD; the `stride` threads of the
// workgroup that wrote it (tid = 0 .. stride - 1) call this.  Each waits
// until its own stores are complete, `sync` (a barrier of those threads)
// puts every store before thread 0's device-scope count of the workgroup on
// the row's counter, and `bcast` hands thread 0's verdict to the others.
// The workgroup that brings the count to nparts resets the counter to 0 and
// merges the row's partitions (the canonical order above) for its heads
// [hbase, hbase + nheads), reading them with device-scope atomic loads that
// issue only once the count has returned.  Only the partial states cross
// workgroups, and only through such loads and stores, so no cache-wide
// write-back or invalidation is needed.  No workgroup waits for another.
// The counters must be zero when the launch starts; every launch leaves
// them zero.
template <typename Sync, typename Bcast>
__device__ __forceinline__ void merge_if_last(const AttnArgs& a, int row, int hbase, int nheads,
                                              int nparts, int D, int tid, int stride, Sync sync,
                                              Bcast bcast) {
  __builtin_amdgcn_s_waitcnt(0);   // this wave's partial-state stores are complete
  sync();
  int last = 0;
  if (tid == 0) {
    int32_t* ctr = a.counters + static_cast<int64_t>(row) * a.hq + hbase;
    const int old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = old == nparts - 1;
    if (last) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (!bcast(last)) return;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  for (int idx = tid; idx < nheads * D; idx += stride) {
    const int g = idx / D;
    const int d = idx % D;
    const PartMerge pm = merge_ml<true>(a, row, hbase + g, nparts);
    store_out(a, (static_cast<int64_t>(row) * a.hq + hbase + g) * D + d,
              merge_elem<true>(a, row, hbase + g, nparts, pm, d, D));
  }
}

// Final merge of a workgroup: NW wavefronts each left, per head row g, a
// softmax state (max m, sum l) and an unnormalised output row o[D] in LDS.
// Rescales them to the common max and either writes the normalised output
// (the row's context fits one partition) or the partition's partial state.
// Threads first, first + stride, ... share the elements.
template <int NW, int NH, int D>
__device__ __forceinline__ void finish_rows(const AttnArgs& a, const float (&sm_o)[NW][NH][D],
                                            const float (&sm_m)[NW][NH],
                                            const float (&sm_l)[NW][NH], int nheads, int row,
                                            int hbase, int part, int nparts, int first,
                                            int stride) {
  for (int idx = first; idx < nheads * D; idx += stride) {
    const int g = idx / D;
    const int d = idx % D;
    float M = sm_m[0][g];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, sm_m[w][g]);
    const float ms = (M == kNegInf) ? 0.f : M;
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = fast_exp2(sm_m[w][g] - ms);
      L += sm_l[w][g] * f;
      O += sm_o[w][g][d] * f;
    }
    const int64_t orow = static_cast<int64_t>(row) * a.hq + hbase + g;
    if (nparts <= 1) {
      store_out(a, orow * D + d, L > 0.f ? O / L : 0.f);
    } else if (a.counters != nullptr) {
      // merged in this launch by another workgroup: write through
      const int64_t pi = part_slot(a, row, hbase + g, part);
      __hip_atomic_store(a.part_o + pi * D + d, O, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (d == 0) {
        __hip_atomic_store(a.part_ml + pi * 2, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(a.part_ml + pi * 2 + 1, L, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
    } else {
      const int64_t pi = part_slot(a, row, hbase + g, part);
      a.part_o[pi * D + d] = O;
      if (d == 0) {
        a.part_ml[pi * 2] = M;
        a.part_ml[pi * 2 + 1] = L;
      }
    }
  }
}

}  // namespace pkv
