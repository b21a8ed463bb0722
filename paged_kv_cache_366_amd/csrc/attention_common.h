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

struct WgCoord {
  int row, part, hg;
};
__device__ __forceinline__ WgCoord wg_coord(int ngroups, int num_parts) {
  WgCoord c;
  const int bid = blockIdx.x;
  c.hg = bid % ngroups;
  const int rest = bid / ngroups;
  c.part = rest % num_parts;
  c.row = rest / num_parts;
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
