// Chunked prefill attention on the matrix cores (gfx950), 16-bit q and KV.
//
// Long prompts are processed in chunks that share a batch with decode steps
// (m.nxbn.cn §3.2; cnnetsun.cn "别再让GPU内存拖后腿了…" §4.1 turns chunking
// on).  Row i of sequence s's chunk of length qlen sits at absolute position
// P_i = context_lens[s] - qlen + i and attends keys [0, P_i] through the
// block table: per-block scores, one softmax over them, and the weighted sum
// of the value rows (cnnetsun.cn §3.1), with the chunk's own K/V already
// written to the cache.
//
// Layout.  A workgroup of 4 wavefronts owns 64 consecutive rows of one
// sequence's chunk for one query head; wavefront w takes rows 16w..16w+15.
// Every row of the workgroup reads the same keys, so K and V go through LDS
// in steps of two 16-row tiles (double-buffered, rows padded by 16 bytes so
// the 16 key rows a wavefront reads at one column fall in different banks)
// and all four wavefronts read them there.  Per tile and wavefront:
//   S^T [16 keys x 16 rows] = K [16 x D] . Q^T [D x 16]      (D/32 MFMA 16x16x32)
//   online softmax per row (column), lazily rescaled: the row maximum across
//   the four lane groups is taken only when some score outgrows the running
//   one by the slack; the row's weights stay in the lanes that hold them,
//   which is exactly the B operand of the next product;
//   O^T [D x 16 rows] += V^T [D x 16 keys] . P^T [16 keys x 16 rows]
//       (D/16 MFMA 16x16x32, weights as a 16-bit hi + lo pair: K = 32 is the
//       lane's 4 keys with the hi weights, then the same keys with the lo)
// Lane (m, g) reads the D/16 elements m*D/16.. of key rows 4g..4g+3 from
// LDS, so product j sees element m*D/16 + j; at the end the lane holds 32
// contiguous output elements of its row.
//
// Loads: the global loads of the steps two ahead are issued right after
// the barrier and land in registers while the wavefronts compute (two steps
// in flight measured 6% faster than one; three or four, slower); no branch
// guards them (a block outside the pool reads a fixed in-pool address), so
// the wait before the LDS store covers only that step's loads.
//
// Causality: a key t is used by row i when t <= P_i; rows past the chunk are
// idle, and a wavefront skips tiles past its last row's position; tiles
// wholly at or below the wavefront's first row position skip the test.  Key
// rows past the workgroup's last position (the unwritten tail of the last
// block) are stored to LDS as zeros, so no garbage enters the products; a
// table entry outside the pool makes its whole tile masked.
//
// Grid order: the query head is the fastest index, so (with a head count
// that is a multiple of 8) all tiles of one (sequence, head) go to the same
// XCD and share the K/V lines it caches in L2.
//
// Measured on MI355X (mixed step, four 512-row chunks): the loads, LDS
// stores and barriers alone take about 60% of the kernel's time, at about
// 6.6 TB/s of K/V delivered to the compute units; counters put the VALU at
// 43% and the matrix cores at 17% of their issue capacity, with on average
// half of the wave slots occupied as short row tiles finish first.  Wider
// workgroups, 32 rows per wavefront, wider steps, key partitions for the
// long row tiles and operand pairs formed without permutes each measured
// slower or within a few percent.
#include "attention_common.h"
#include "mfma_common.h"

namespace pkv {
namespace {

#ifndef PKV_PREFILL_WAVES
#define PKV_PREFILL_WAVES 4
#endif
constexpr int kPrefillWaves = PKV_PREFILL_WAVES;   // wavefronts (16 rows each) per workgroup
constexpr int kPrefillThreads = 64 * kPrefillWaves;
#ifndef PKV_PREFILL_DEPTH
#define PKV_PREFILL_DEPTH 2
#endif
#ifndef PKV_PREFILL_RTILES
#define PKV_PREFILL_RTILES 1
#endif
#ifndef PKV_PREFILL_GROUP
#define PKV_PREFILL_GROUP 2
#endif
// Tuning constants (the defaults measured best on MI355X):
constexpr int kDepth = PKV_PREFILL_DEPTH;     // steps whose global loads are in flight
constexpr int kGroup = PKV_PREFILL_GROUP;     // 16-key tiles per LDS step (one barrier)
constexpr int kRowTiles = PKV_PREFILL_RTILES; // 16-row tiles per wavefront
constexpr int kTileRows = kPrefillWaves * 16 * kRowTiles;   // query rows per workgroup

template <typename T, int D, int P, int R, int G0, bool STREAM>
__global__ __launch_bounds__(kPrefillThreads) void prefill_mfma_kernel(AttnArgs a, int max_tiles) {
  constexpr int NK = D / 32;              // QK products per block and row tile
  constexpr int NV = D / 16;              // PV products per block and row tile
  constexpr int VB = NV * 2;              // bytes of a lane's V chunk
  constexpr int ROWB = D * 2;             // bytes of a K/V row
  constexpr int LROW = ROWB + 16;         // LDS row stride
  constexpr int CHUNKS = ROWB / 16;       // 16-byte chunks per row
  constexpr int TILE_CHUNKS = 16 * CHUNKS;
  constexpr int NT = kPrefillThreads;
  // Blocks per LDS step: at least enough that every thread has a chunk.
  constexpr int G = (G0 * 2 * TILE_CHUNKS >= NT) ? G0 : NT / (2 * TILE_CHUNKS);
  constexpr int LPS = G * 2 * TILE_CHUNKS / NT;   // K+V chunks per thread per step
  static_assert(G * 2 * TILE_CHUNKS == NT * LPS, "a step's K and V split evenly over the threads");
  constexpr int WROWS = 16 * R;           // rows per wavefront
  constexpr int TROWS = kPrefillWaves * WROWS;
  using M = Mx<T>;

  // Workgroup -> (sequence, row tile, head), head fastest; within a
  // sequence the last row tiles (the most keys) are dispatched first.
  const int hq = a.hq;
  const int h = blockIdx.x % hq;
  const int rest = blockIdx.x / hq;
  const int part = rest % a.num_parts;   // key partition (split-K)
  const int rest2 = rest / a.num_parts;
  const int tile = max_tiles - 1 - rest2 % max_tiles;
  const int seq = rest2 / max_tiles;
  const int qs = a.qsl[seq];
  const int qlen = a.qsl[seq + 1] - qs;
  if (tile * TROWS >= qlen) return;
  const int kvh = h / (hq / a.hkv);
  const int cap = min(a.max_ctx, a.max_blocks << (4 + a.bs_shift));   // keys the table row can address
  const int base_pos = a.lens[seq] - qlen;             // position of the chunk's row 0

  const int wave = wave_uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;
  const int kg = lane >> 4;

  const int q0 = tile * TROWS + wave * WROWS;   // first row of this wave
  int qlast[R];                                 // last key of the lane's row in each row tile
  bool qlive[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int qi = q0 + 16 * r + r16;
    qlive[r] = qi < qlen;
    qlast[r] = qlive[r] ? min(base_pos + qi, cap - 1) : -1;
  }
  const int wrows = min(WROWS, qlen - q0);
  const int wlast = wrows > 0 ? min(base_pos + q0 + wrows - 1, cap - 1) : -1;
  const int wfirst = wrows > 0 ? min(base_pos + q0, cap - 1) : -1;   // first row's last key
  const int tlast = min(base_pos + min(qlen, (tile + 1) * TROWS) - 1, cap - 1);
  const int nblk = tlast >= 0 ? (tlast >> 4) + 1 : 0;
  // This workgroup's key tiles: those of its partition, up to the last key.
  const int ptiles = a.part_tokens >> 4;
  const int b_begin = part * ptiles;
  const int b_end = min(nblk, b_begin + ptiles);
  if (b_begin >= b_end) return;   // no row of the tile has keys in this partition

  // Q^T operands: row q0 + 16r + r16, elements 32kk + 8kg .. +7.
  u32x4 qop[R][NK];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int qi = q0 + 16 * r + r16;
      const int64_t qrow = (static_cast<int64_t>(qs + (qlive[r] ? qi : 0)) * hq + h) * D;
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(qp + qrow + 32 * kk + 8 * kg);
        qop[r][kk] = qlive[r] ? v : u32x4{0u, 0u, 0u, 0u};
      }
    }
  }

  __shared__ __align__(16) uint8_t sk[2][G * 16 * LROW];
  __shared__ __align__(16) uint8_t sv[2][G * 16 * LROW];

  const int32_t* trow = a.tables + static_cast<int64_t>(seq) * a.max_blocks;
  const uint8_t* kc = static_cast<const uint8_t*>(a.kc);
  const uint8_t* vc = static_cast<const uint8_t*>(a.vc);

  // Tile b of the context into registers: K chunks first, then V.  Rows past
  // the workgroup's last key, and every row of a block outside the pool,
  // become zeros.  P blocks are in flight: slot u of the ring holds block
  // b with b % P == u, so after unrolling every index is static.
  u32x4 ld[P][LPS];
  bool ld_ok[P][G];
  // Loads of the G blocks of step st: chunk c of the step is block c / (2
  // TILE_CHUNKS), K then V.  No branch around them and nothing consumes
  // them before the LDS store, so the wait there covers only that step's
  // loads and P steps really are in flight.  A block outside the pool (or
  // past the table) reads the same bytes of the pool's first tile instead;
  // the store turns it, and every row past the workgroup's last key, into
  // zeros.
  auto gload = [&](int st, u32x4 (&rg)[LPS], bool (&ok)[G]) {
    int64_t toff[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int b = b_begin + st * G + g;
      const int p = trow[min(b, b_end - 1) >> a.bs_shift];
      ok[g] = b < b_end && p >= 0 && p < a.num_blocks;
      toff[g] = ok[g] ? tile_index(a, p, kvh, b) * (16 * ROWB) : 0;
    }
#pragma unroll
    for (int i = 0; i < LPS; ++i) {
      const int c = threadIdx.x + NT * i;
      const int g = c / (2 * TILE_CHUNKS);
      const int rem = c % (2 * TILE_CHUNKS);
      int64_t off = toff[0];
#pragma unroll
      for (int k = 1; k < G; ++k) off = g == k ? toff[k] : off;
      rg[i] = load_kv<u32x4, STREAM>((rem < TILE_CHUNKS ? kc : vc) + off + (rem % TILE_CHUNKS) * 16);
    }
  };
  auto sstore = [&](int buf, const u32x4 (&rg)[LPS], int st, const bool (&ok)[G]) {
#pragma unroll
    for (int i = 0; i < LPS; ++i) {
      const int c = threadIdx.x + NT * i;
      const int g = c / (2 * TILE_CHUNKS);
      const int rem = c % (2 * TILE_CHUNKS);
      const int which = rem / TILE_CHUNKS;
      const int rc = rem % TILE_CHUNKS;
      const int row = rc / CHUNKS;
      bool okg = ok[0];
#pragma unroll
      for (int k = 1; k < G; ++k) okg = g == k ? ok[k] : okg;
      const bool use = okg && (b_begin + st * G + g) * 16 + row <= tlast;
      uint8_t* dst = (which == 0 ? sk[buf] : sv[buf]) + (g * 16 + row) * LROW + (rc % CHUNKS) * 16;
      *reinterpret_cast<u32x4*>(dst) = use ? rg[i] : u32x4{0u, 0u, 0u, 0u};
    }
  };

  float m[R], l[R];
  f32x4 acc[R][NV];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    m[r] = kNegInf;
    l[r] = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j) acc[r][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // One block: its tile from LDS buffer `buf`, for each of the wave's row
  // tiles.  The K operands and the V operand are read and built once and
  // serve every row tile.
  // `ok`: the block is in the pool (and in this workgroup's range); it sits
  // in slot g of the LDS step.
  auto compute = [&](int b, int buf, bool ok, int g) {
    const int kb = b * 16;
    if (!ok || kb > wlast) return;   // wave-uniform
    const int lrow0 = g * 16;   // the block's first row in the LDS step
    // ---- S^T = K . Q^T
    f32x4 s[R];
#pragma unroll
    for (int r = 0; r < R; ++r) s[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const u32x4 kop =
          *reinterpret_cast<const u32x4*>(sk[buf] + (lrow0 + r16) * LROW + (32 * kk + 8 * kg) * 2);
#pragma unroll
      for (int r = 0; r < R; ++r) s[r] = M::k32(kop, qop[r][kk], s[r]);
    }
    // ---- online softmax per row, lazily rescaled; P^T as hi + lo pairs.
    // Tiles wholly at or below the wave's first row position need no causal
    // mask (the key rows past the workgroup's last key, zeros in LDS, only
    // occur in tiles that reach past it).
    const bool whole = kb + 15 <= wfirst;
    u32x4 pcat[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float sc[4];
      float tmax = kNegInf;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = kb + 4 * kg + i;
        sc[i] = (whole || t <= qlast[r]) ? s[r][i] * a.scale_log2 : kNegInf;
        tmax = fmaxf(tmax, sc[i]);
      }
      // The running max of a row is shared by its four lane groups.  A lane
      // whose keys stay within the slack of it changes nothing; only when
      // some lane of the wave exceeds it are the row maxima taken across
      // the lane groups (the same value in all four) and the row rescaled.
      if (__any(tmax > m[r] + kRescaleSlack)) {   // rare after the first blocks
        tmax = max_xor32(max_xor16(tmax));
        const bool grow = tmax > m[r] + kRescaleSlack;
        const float mn = grow ? tmax : m[r];
        const float alpha = grow ? fast_exp2(m[r] - mn) : 1.f;
        m[r] = mn;
        l[r] *= alpha;
#pragma unroll
        for (int j = 0; j < NV; ++j) acc[r][j] *= alpha;
      }
      const float ms = (m[r] == kNegInf) ? 0.f : m[r];
      float pw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pw[i] = fast_exp2(sc[i] - ms);
        l[r] += pw[i];
      }
      const uint32_t h01 = M::pack(pw[0], pw[1]);
      const uint32_t h23 = M::pack(pw[2], pw[3]);
      // K = 32 of one product: the lane's 4 keys with the hi weights, then
      // the same 4 keys with the lo weights (the A operand repeats them)
      pcat[r] = u32x4{h01, h23, M::pack(pw[0] - M::lo(h01), pw[1] - M::hi(h01)),
                      M::pack(pw[2] - M::lo(h23), pw[3] - M::hi(h23))};
    }
    // ---- O^T += V^T . P^T
    u32x4 vrow[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      vrow[e] = load_bytes<VB>(sv[buf] + (lrow0 + 4 * kg + e) * LROW + r16 * VB);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const uint32_t v01 = pair_of(vrow[0], vrow[1], j);
      const uint32_t v23 = pair_of(vrow[2], vrow[3], j);
      const u32x4 vop = {v01, v23, v01, v23};
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r][j] = M::k32(vop, pcat[r], acc[r][j]);
    }
  };

  const int nstep = (b_end - b_begin + G - 1) / G;
  {   // (the loads read table entries of blocks b_begin .. b_end - 1 only)
#pragma unroll
    for (int u = 0; u < P; ++u) gload(u, ld[u], ld_ok[u]);
  }
  // Step st: its registers go to LDS buffer st & 1 (the other buffer may
  // still be read by slower waves for step st - 1), one barrier, then the
  // freed registers start loading step st + P.  Whole groups of P steps, so
  // no step is conditional (a step past the last block stores zeros and
  // computes nothing).
#pragma unroll 1
  for (int s0 = 0; s0 < nstep; s0 += P) {
#pragma unroll
    for (int u = 0; u < P; ++u) {
      const int st = s0 + u;
      bool ok[G];
#pragma unroll
      for (int g = 0; g < G; ++g) ok[g] = ld_ok[u][g];
      sstore(st & 1, ld[u], st, ok);
      __syncthreads();
      gload(st + P, ld[u], ld_ok[u]);
#pragma unroll
      for (int g = 0; g < G; ++g) compute(b_begin + st * G + g, st & 1, ok[g], g);
    }
  }

#pragma unroll
  for (int r = 0; r < R; ++r) {
    // Each lane summed the weights of its 4 keys per block; add the 4 groups.
    float lr = l[r];
    lr = sum_xor32(sum_xor16(lr));
    if (!qlive[r]) continue;
    // Partitions the row's own keys span (as the reduce counts them): one
    // means this workgroup (partition 0) writes the final row; more mean
    // each partition leaves its unnormalised output and (max, sum).
    const int rparts = a.num_parts > 1 ? (qlast[r] + a.part_tokens) / a.part_tokens : 1;
    if (part >= max(rparts, 1)) continue;
    const int64_t qrow = qs + q0 + 16 * r + r16;
    const int64_t grow = qrow * hq + h;
    if (rparts <= 1) {
      const float inv = lr > 0.f ? 1.f / lr : 0.f;
      // acc[r][j][i] is element NV*(4kg + i) + j of the row.
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NV; ++j)
          store_out(a, grow * D + NV * (4 * kg + i) + j, acc[r][j][i] * inv);
    } else {
      const int64_t slot = part_slot(a, qrow, h, part);
      float* po = a.part_o + slot * D;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NV; ++j) po[NV * (4 * kg + i) + j] = acc[r][j][i];
      if (kg == 0) {
        a.part_ml[slot * 2] = m[r];
        a.part_ml[slot * 2 + 1] = lr;
      }
    }
  }
}

template <typename T, bool NT>
pkv_status launch_t(const AttnArgs& a, int D, int max_tiles, hipStream_t st) {
  const int64_t wgs = static_cast<int64_t>(a.num_seqs) * max_tiles * a.num_parts * a.hq;
  if (wgs > 0x7fffffff / kPrefillThreads)
    return fail(PKV_ERR_UNSUPPORTED, "prefill: launch too large");
  dim3 grid(static_cast<unsigned>(wgs));
  if (D == 64)
    hipLaunchKernelGGL((prefill_mfma_kernel<T, 64, kDepth, kRowTiles, kGroup, NT>), grid, dim3(kPrefillThreads), 0, st,
                       a, max_tiles);
  else
    hipLaunchKernelGGL((prefill_mfma_kernel<T, 128, kDepth, kRowTiles, kGroup, NT>), grid, dim3(kPrefillThreads), 0, st,
                       a, max_tiles);
  PKV_LAUNCH_CHECK("chunked prefill (MFMA)");
  return PKV_OK;
}

}  // namespace

pkv_status launch_prefill_mfma(const AttnArgs& a, pkv_dtype q_dt, int D, int group,
                               int max_query_len, hipStream_t st) {
  if (max_query_len <= 0 || a.num_seqs <= 0) return PKV_OK;
  const int max_tiles = (max_query_len + kTileRows - 1) / kTileRows;
  // A workgroup serves one query head and one row tile: when every chunk
  // fits one row tile and no KV head serves several query heads, each K/V
  // tile is read by one workgroup only, so (under the streaming policy) its
  // loads carry the non-temporal hint; otherwise the other row tiles and
  // heads reuse it from L2.
  const bool stream = a.stream_kv && max_tiles == 1 && group == 1;
  if (q_dt == PKV_BF16)
    return stream ? launch_t<BF16, true>(a, D, max_tiles, st) : launch_t<BF16, false>(a, D, max_tiles, st);
  if (q_dt == PKV_F16)
    return stream ? launch_t<F16, true>(a, D, max_tiles, st) : launch_t<F16, false>(a, D, max_tiles, st);
  return fail(PKV_ERR_UNSUPPORTED, "MFMA prefill needs 16-bit q");
}

}  // namespace pkv
