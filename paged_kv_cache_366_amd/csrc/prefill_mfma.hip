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
// in steps of two 16-key tiles and all four wavefronts read them there.
// Per step and wavefront:
//   S^T [16 keys x 16 rows] = K [16 x D] . Q^T [D x 16], per tile
//       (D/32 MFMA 16x16x32; lane (r16, kg) holds keys 4kg..4kg+3 of row r16)
//   online softmax per row (column), lazily rescaled: the row maximum across
//   the four lane groups is taken only when some score outgrows the running
//   one by the slack; the lane's 8 weights (4 keys of each tile) are exactly
//   its B operand of the value product, so they never move between lanes;
//   O^T [D x 16 rows] += V^T [D x 32 keys] . P^T [32 keys x 16 rows]
//       (D/16 output blocks, each one MFMA 16x16x32 with the weights' bf16
//       (or f16) hi parts and one with the lo parts: an fp32-accurate sum)
// V^T comes straight out of LDS with gfx950's transpose read: two 8-byte
// reads per output block give the lane its 8 keys at one output element,
// in the key order of its weights, with no register permutes.  Lane
// (r16, kg) ends with elements 16j + 4kg .. +3 of its row for each block j.
//
// Loads: K and V move from global memory to LDS with gfx950's direct loads
// (no registers in between) into NST stages, so the loads of the next NST - 1
// steps are in flight while a step computes.  Three stages of head_dim 128
// take 48 KiB of LDS, which leaves room for three workgroups per compute
// unit; two take 32 KiB and leave room for four (the register cap below).
// The launch takes two when it has more workgroups than compute units and
// three otherwise: with fewer, each workgroup walks its keys alone and the
// deeper pipeline hides more of the load latency (long-document chunks
// unsplit, 128 workgroups: 441-446 us with three stages against 465-467
// with two), while with more, the fourth resident workgroup pays (mixed
// step, 1,024 workgroups: 84.6 against 86 us; long-document chunks split
// 4-way, 512 workgroups: 197.0 against 202.6 us; the prefix-cache
// admission prefill 268-288 against 288-290 us).  Head_dim 64 keeps three
// stages (24 KiB: registers, not LDS, bound its occupancy).
//
// Rows are unpadded and their 16-byte chunks XOR-swizzled by row, which
// keeps the rows read at one column in different banks.  Each wave waits for its own loads of a step,
// then one barrier (without the memory fence of __syncthreads, which would
// also wait for the steps still loading) makes every wave's loads visible.
// Rows past the workgroup's last key and rows of blocks outside the pool
// are zeroed by the wave that loaded them, after they land and before the
// barrier.
//
// Causality: a key t is used by row i when t <= P_i; rows past the chunk are
// idle, and a wavefront skips steps past its last row's position; steps
// wholly at or below the wavefront's first row position skip the test.  Key
// rows past the workgroup's last position (the unwritten tail of the last
// block) are stored to LDS as zeros, so no garbage enters the products; a
// table entry outside the pool makes its whole tile masked.
//
// Grid order: the query head is the fastest index, so (with a head count
// that is a multiple of 8) all tiles of one (sequence, head) go to the same
// XCD and share the K/V lines it caches in L2.  Sequences go longest
// context first and, within one, the last row tiles (the most keys) first:
// all of a compute unit's workgroups are resident together and older waves
// issue first, so the heaviest tiles lead instead of finishing alone.
//
// Measured on MI355X (mixed step, four 512-row chunks over 0..1536 cached
// tokens): the transposed value reads took the kernel from 140 to 109 us,
// the order by context length and four waves per SIMD to about 91 us, the
// direct loads to 86 us, two stages for large grids to 84.6 us.  What bounds it: without its arithmetic the same
// kernel (loads, LDS, barriers) still takes about 62 us, and with its
// arithmetic the longest row tiles (2,048 keys, 64 steps) finish last;
// 8-wave workgroups (half the K/V traffic) and key partitions (fp32 partial
// rows) both measured slower.
#include <atomic>

#include "attention_common.h"
#include "mfma_common.h"

namespace pkv {
namespace {

#ifndef PKV_PREFILL_WAVES
#define PKV_PREFILL_WAVES 4
#endif
constexpr int kPrefillWaves = PKV_PREFILL_WAVES;   // wavefronts (16 rows each) per workgroup
constexpr int kPrefillThreads = 64 * kPrefillWaves;
#ifndef PKV_PREFILL_RTILES
#define PKV_PREFILL_RTILES 1
#endif
#ifndef PKV_PREFILL_GROUP
#define PKV_PREFILL_GROUP 2
#endif
// Tuning constants (the defaults measured best on MI355X):
constexpr int kGroup = PKV_PREFILL_GROUP;     // 16-key tiles per LDS step (one barrier)
constexpr int kRowTiles = PKV_PREFILL_RTILES; // 16-row tiles per wavefront
constexpr int kTileRows = kPrefillWaves * 16 * kRowTiles;   // query rows per workgroup

// Registers for four waves per SIMD (at most 128 VGPRs), so that four
// workgroups fit a compute unit where the LDS allows it (two stages at
// head_dim 128, or head_dim 64).  Left to itself the compiler took 130 in
// an earlier form of the kernel, which leaves room for three.
#ifndef PKV_PREFILL_WPE
#define PKV_PREFILL_WPE 4
#endif
#define PKV_PREFILL_ATTR __attribute__((amdgpu_waves_per_eu(PKV_PREFILL_WPE)))
template <typename T, int D, int R, int G0, int NST>
__global__ __launch_bounds__(kPrefillThreads) PKV_PREFILL_ATTR void prefill_mfma_kernel(AttnArgs a, int max_tiles) {
  constexpr int NK = D / 32;              // QK products per block and row tile
  constexpr int NV = D / 16;              // PV products per block and row tile
  constexpr int ROWB = D * 2;             // bytes of a K/V row
  constexpr int CHUNKS = ROWB / 16;       // 16-byte chunks per row
  constexpr int G = G0;                   // 16-key tiles per step
  static_assert(G == 2, "a step is two 16-key tiles: the K = 32 of one value product");
  static_assert(NST == 2 || NST == 3, "two or three LDS stages");
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
  // Sequences are taken in order of context length, longest first (ties in
  // index order), so the row tiles with the most keys start first and their
  // waves are the oldest on their compute units (older waves issue first).
  // The rank is computed here by the workgroup, for up to kPrefillThreads
  // sequences; a larger batch keeps index order.
  int seq = rest2 / max_tiles;
  if (a.num_seqs <= kPrefillThreads) {
    __shared__ int s_seq;
    const int t = threadIdx.x;
    if (t < a.num_seqs) {
      const int lt = a.lens[t];
      int rank = 0;
      for (int u = 0; u < a.num_seqs; ++u) {
        const int lu = a.lens[u];
        rank += (lu > lt || (lu == lt && u < t)) ? 1 : 0;
      }
      if (rank == seq) s_seq = t;
    }
    __syncthreads();
    seq = wave_uniform(s_seq);
  }
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

  const int32_t* trow = a.tables + static_cast<int64_t>(seq) * a.max_blocks;
  const uint8_t* kc = static_cast<const uint8_t*>(a.kc);
  const uint8_t* vc = static_cast<const uint8_t*>(a.vc);

  // ---- K/V staging: direct global -> LDS loads into NST stages ----------
  // A stage holds one step (two 16-key tiles) of K and of V: 32 rows of
  // ROWB bytes each, unpadded.  One load instruction of a wave fills 1 KiB
  // (lane l's 16 bytes land at byte 16 l), i.e. RPL whole rows.  The
  // 16-byte chunk c of stage row r sits at chunk position c ^ (r % CHUNKS),
  // so rows read at one column fall in different banks.  Loads of the next
  // NST - 1 steps are in flight while a step computes, and they hold no
  // registers.
  constexpr int SROWS = G * 16;
  constexpr int STAGE = SROWS * ROWB;
  constexpr int RPL = 1024 / ROWB;                // rows per load instruction
  constexpr int LPO = SROWS / RPL;                // load instructions per operand and step
  // Per wave and operand: LDW instructions, by waves [0, LPO / LDW); with
  // more waves than instructions the rest load nothing.
  constexpr int LDW = LPO >= kPrefillWaves ? LPO / kPrefillWaves : 1;
  static_assert(LPO % LDW == 0 && (LPO >= kPrefillWaves ? LPO % kPrefillWaves == 0 : true),
                "loads split evenly over the waves");
  const bool loader = wave * LDW < LPO;          // wave-uniform
  constexpr int NLD = 2 * LDW;                    // vector memory instructions per loading wave and step
  __shared__ __align__(1024) uint8_t sk0[STAGE], sk1[STAGE], sk2[NST == 3 ? STAGE : 16];
  __shared__ __align__(1024) uint8_t sv0[STAGE], sv1[STAGE], sv2[NST == 3 ? STAGE : 16];

  // Lane constants.  Load k of this wave (per operand) fills stage rows
  // [RPL (wave LDW + k), +RPL); the lane's chunk comes from row
  // rl = that + lane / CHUNKS of the step, chunk (lane % CHUNKS) ^ (rl % CHUNKS).
  uint32_t loff[LDW];   // byte offset of the lane's chunk within its 16-row tile
#pragma unroll
  for (int k = 0; k < LDW; ++k) {
    const int rl = RPL * (wave * LDW + k) + lane / CHUNKS;
    loff[k] = (rl % 16) * ROWB + ((lane % CHUNKS) ^ (rl % CHUNKS)) * 16;
  }
  // K operand reads: row r16 (+16 for the second tile), chunk 4kk + kg.
  uint32_t koff[NK];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) koff[kk] = r16 * ROWB + ((4 * kk + kg) ^ (r16 % CHUNKS)) * 16;
  // V transpose reads: source row 4kg + (r16 >> 2), elements 16j + 4 (r16 & 3)
  // .. +3 = chunk 2j + ((r16 & 3) >> 1), half r16 & 1.
  uint32_t voff[NV];
  {
    const int vr = 4 * kg + (r16 >> 2);
#pragma unroll
    for (int j = 0; j < NV; ++j)
      voff[j] = vr * ROWB + ((2 * j + ((r16 & 3) >> 1)) ^ (vr % CHUNKS)) * 16 + (r16 & 1) * 8;
  }

  // Stage u's K and V bases (compile-time after unrolling).
  auto kst = [&](int u) -> uint8_t* { return u == 0 ? sk0 : u == 1 ? sk1 : sk2; };
  auto vst = [&](int u) -> uint8_t* { return u == 0 ? sv0 : u == 1 ? sv1 : sv2; };

  // Issue the loads of step st into stage u: the step's table entries, then
  // NLD instructions.  A block outside the pool or past the workgroup's range
  // loads the pool's first tile instead, so every step issues the same
  // count of loads (the waits below count them); such rows are zeroed after
  // they land, by the wave that loaded them.
  // Table entries come from a window of 64 in a vector register (lane i:
  // entry tv_base + i), read with a lane read: a load per step would have
  // to wait for every staging load issued before it.  The window moves (one
  // load, which does wait) when a step needs an entry past it.
  int tv_base = b_begin >> a.bs_shift;
  int tv = tv_base + lane < a.max_blocks ? trow[tv_base + lane] : -1;
  auto entry = [&](int e) {   // e: wave-uniform, not decreasing
    if (e >= tv_base + 64) {
      tv_base = e;
      tv = e + lane < a.max_blocks ? trow[e + lane] : -1;
    }
    return __builtin_amdgcn_readlane(tv, e - tv_base);
  };
  bool okst[NST][G];
  auto issue = [&](int st, int u) {
    int64_t toff[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int b = b_begin + st * G + g;
      const int p = entry(min(b, b_end - 1) >> a.bs_shift);
      okst[u][g] = b < b_end && p >= 0 && p < a.num_blocks;
      toff[g] = okst[u][g] ? tile_index(a, p, kvh, b) * (16 * ROWB) : 0;
    }
    if (!loader) return;
#pragma unroll
    for (int k = 0; k < LDW; ++k) {
      const int g = (RPL * (wave * LDW + k)) / 16;   // wave-uniform
      const int64_t t = g == 0 ? toff[0] : toff[1];
      load_to_lds16(kc + t + loff[k], kst(u) + 1024 * (wave * LDW + k));
      load_to_lds16(vc + t + loff[k], vst(u) + 1024 * (wave * LDW + k));
    }
  };
  // After this wave's loads of step st (stage u) have landed: zero the rows
  // it loaded that are past the workgroup's last key or in a block outside
  // the pool (wave-uniform test first).
  auto fixup = [&](int st, int u) {
    if (!loader || (okst[u][0] && okst[u][1] && (b_begin + st * G + G) * 16 - 1 <= tlast)) return;
#pragma unroll
    for (int k = 0; k < LDW; ++k) {
      const int rl = RPL * (wave * LDW + k) + lane / CHUNKS;
      const int g = rl / 16;
      const bool ok = g == 0 ? okst[u][0] : okst[u][1];
      if (!ok || (b_begin + st * G) * 16 + rl > tlast) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(kst(u) + 1024 * (wave * LDW + k) + 16 * lane) = z;
        *reinterpret_cast<u32x4*>(vst(u) + 1024 * (wave * LDW + k) + 16 * lane) = z;
      }
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

  // One step: its two 16-key tiles from stage u, for each of the wave's row
  // tiles.
  auto compute = [&](int st, int u) {
    const int kb = (b_begin + st * G) * 16;   // first key of the step
    bool use[G];
#pragma unroll
    for (int g = 0; g < G; ++g) use[g] = okst[u][g] && kb + 16 * g <= wlast;   // wave-uniform
    if (!use[0] && !use[1]) return;
    // ---- S^T = K . Q^T for each tile (a tile out of range has no scores)
    f32x4 s[G][R];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int r = 0; r < R; ++r) s[g][r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (!use[g]) continue;
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const u32x4 kop = *reinterpret_cast<const u32x4*>(kst(u) + 16 * g * ROWB + koff[kk]);
#pragma unroll
        for (int r = 0; r < R; ++r) s[g][r] = M::k32(kop, qop[r][kk], s[g][r]);
      }
    }
    // ---- online softmax per row over the step's 8 keys of this lane, lazily
    // rescaled; P^T as a hi and a lo operand.  When both tiles are in range
    // and wholly at or below the wave's first row position, no key needs the
    // causal test (wave-uniform).
    const bool all_whole = use[0] && use[1] && kb + 16 * G - 1 <= wfirst;
    u32x4 phi[R], plo[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float sc[G][4];
      if (all_whole) {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int i = 0; i < 4; ++i) sc[g][i] = s[g][r][i] * a.scale_log2;
      } else {
        // keys past the row's position, or of a tile out of range, get no weight
        const int lim = qlast[r] - kb - 4 * kg;   // key kb + 4kg + c is used when c <= lim
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            sc[g][i] = (use[g] && 16 * g + i <= lim) ? s[g][r][i] * a.scale_log2 : kNegInf;
      }
      float tmax = kNegInf;
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, sc[g][i]);
      // The running max of a row is shared by its four lane groups.  A lane
      // whose keys stay within the slack of it changes nothing; only when
      // some lane of the wave exceeds it are the row maxima taken across
      // the lane groups (the same value in all four) and the row rescaled.
      if (__any(tmax > m[r] + kRescaleSlack)) {   // rare after the first steps
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
      float pw[G][4];
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pw[g][i] = fast_exp2(sc[g][i] - ms);
          l[r] += pw[g][i];
        }
      uint32_t h[4], lo[4];
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          h[2 * g + i] = M::pack(pw[g][2 * i], pw[g][2 * i + 1]);
          lo[2 * g + i] = M::pack(pw[g][2 * i] - M::lo(h[2 * g + i]),
                                  pw[g][2 * i + 1] - M::hi(h[2 * g + i]));
        }
      phi[r] = u32x4{h[0], h[1], h[2], h[3]};
      plo[r] = u32x4{lo[0], lo[1], lo[2], lo[3]};
    }
    // ---- O^T += V^T . P^T, 16 output elements per product: the K = 32
    // slots of lane group kg are keys 4kg .. 4kg + 3 of the first tile, then
    // the same keys of the second; one product with the hi weights, one with
    // the lo.  Rows of a tile out of range hold finite values (zeros past
    // the workgroup's last key) and meet zero weights.
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const u32x2 v0 = lds_read_tr16(vst(u) + voff[j]);
      const u32x2 v1 = lds_read_tr16(vst(u) + 16 * ROWB + voff[j]);
      const u32x4 vop = {v0.x, v0.y, v1.x, v1.y};
#pragma unroll
      for (int r = 0; r < R; ++r) {
        acc[r][j] = M::k32(vop, phi[r], acc[r][j]);
        acc[r][j] = M::k32(vop, plo[r], acc[r][j]);
      }
    }
  };

  // vmcnt(n) alone (expcnt and lgkmcnt left at their maxima): with three
  // stages the loads of the next step stay in flight, with two none do.
  constexpr int kWaitOneStep =
      NST == 3 ? (NLD & 15) | ((NLD >> 4) << 14) | (7 << 4) | (15 << 8) : (7 << 4) | (15 << 8);
  static_assert(NLD < 64, "vmcnt range");
  // Barrier without the memory fence __syncthreads adds: that fence waits for
  // every load in flight, including the next steps' staging.  The empty asm
  // statements keep the compiler from moving memory accesses across it.
  auto barrier = [] {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  const int nstep = (b_end - b_begin + G - 1) / G;
  // (the loads read table entries of blocks b_begin .. b_end - 1 only)
  issue(0, 0);
  if constexpr (NST == 3) issue(1, 1);
  // Step st: wait for this wave's loads of step st (with three stages those
  // of step st + 1 stay in flight), zero its invalid rows, barrier (every
  // wave's loads of step st have landed and every wave is done with step
  // st - 1), start the loads of step st + NST - 1 into the stage step st - 1
  // used, compute step st.  Whole groups of NST steps, so every stage index
  // is static; steps past the last block load the first tile and compute
  // nothing.
#pragma unroll 1
  for (int s0 = 0; s0 < nstep; s0 += NST) {
#pragma unroll
    for (int u = 0; u < NST; ++u) {
      const int st = s0 + u;
      __builtin_amdgcn_s_waitcnt(kWaitOneStep);
      fixup(st, u);
      __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the zeros are in LDS
      barrier();
      issue(st + NST - 1, (u + NST - 1) % NST);
      compute(st, u);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);   // no load may land after the workgroup's LDS is released

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
      // acc[r][j][i] is element 16j + 4kg + i of the row.
#pragma unroll
      for (int j = 0; j < NV; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          store_out(a, grow * D + 16 * j + 4 * kg + i, acc[r][j][i] * inv);
    } else {
      const int64_t slot = part_slot(a, qrow, h, part);
      float* po = a.part_o + slot * D;
#pragma unroll
      for (int j = 0; j < NV; ++j)
        *reinterpret_cast<f32x4*>(po + 16 * j + 4 * kg) = acc[r][j];
      if (kg == 0) {
        a.part_ml[slot * 2] = m[r];
        a.part_ml[slot * 2 + 1] = lr;
      }
    }
  }
}

// Compute units of the current device, looked up once per device.
int current_compute_units() {
  constexpr int kDevices = 64;
  static std::atomic<int> cached[kDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < kDevices) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int c = 0;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (c > 0 && dev < kDevices) cached[dev].store(c, std::memory_order_relaxed);
  return c;
}

template <typename T>
pkv_status launch_t(const AttnArgs& a, int D, int max_tiles, hipStream_t st) {
  const int64_t wgs = static_cast<int64_t>(a.num_seqs) * max_tiles * a.num_parts * a.hq;
  if (wgs > 0x7fffffff / kPrefillThreads)
    return fail(PKV_ERR_UNSUPPORTED, "prefill: launch too large");
  dim3 grid(static_cast<unsigned>(wgs));
  if (D == 64) {
    hipLaunchKernelGGL((prefill_mfma_kernel<T, 64, kRowTiles, kGroup, 3>), grid,
                       dim3(kPrefillThreads), 0, st, a, max_tiles);
  } else {
    // two stages once the grid has more workgroups than compute units
    const int cus = current_compute_units();
    if (cus <= 0)
      return fail(PKV_ERR_DEVICE, "chunked prefill (MFMA): no device to size the launch for");
    if (wgs > cus)
      hipLaunchKernelGGL((prefill_mfma_kernel<T, 128, kRowTiles, kGroup, 2>), grid,
                         dim3(kPrefillThreads), 0, st, a, max_tiles);
    else
      hipLaunchKernelGGL((prefill_mfma_kernel<T, 128, kRowTiles, kGroup, 3>), grid,
                         dim3(kPrefillThreads), 0, st, a, max_tiles);
  }
  PKV_LAUNCH_CHECK("chunked prefill (MFMA)");
  return PKV_OK;
}

}  // namespace

int prefill_tile_rows() { return kTileRows; }

pkv_status launch_prefill_mfma(const AttnArgs& a, pkv_dtype q_dt, int D, int group,
                               int max_query_len, hipStream_t st) {
  if (max_query_len <= 0 || a.num_seqs <= 0) return PKV_OK;
  const int max_tiles = (max_query_len + kTileRows - 1) / kTileRows;
  // K/V go to LDS by direct loads with the default cache policy: the other
  // row tiles of a chunk, and the other query heads of a KV head, read the
  // same tiles, mostly at about the same time.
  (void)group;
  if (q_dt == PKV_BF16) return launch_t<BF16>(a, D, max_tiles, st);
  if (q_dt == PKV_F16) return launch_t<F16>(a, D, max_tiles, st);
  return fail(PKV_ERR_UNSUPPORTED, "MFMA prefill needs 16-bit q");
}

}  // namespace pkv
