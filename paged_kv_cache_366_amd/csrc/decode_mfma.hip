// Paged decode attention on the matrix cores, for query-head groups that
// share one KV head (grouped-query attention) and 16-bit queries; KV in the
// same 16-bit type, or int8 or 4-bit codes with per-(block, KV head) scales.
//
// Same computation as the wavefront kernel (cnnetsun.cn "别再让GPU内存拖后腿了…"
// §3.1: per-block scores, one softmax, weighted sum of value rows; int8 storage
// is the compression of §3.2).  With G query heads reading every K/V element,
// scoring and accumulation are dense products of a [G x D] query block with a
// [D x 16] key tile and of a [G x 16] weight block with a [16 x D] value tile,
// so they run on MFMA and the VALU keeps only the softmax and conversions.
//
// Per wavefront, one 16-token tile of one KV head:
//   scores^T [16 tok x 16 heads] = K [16 x D] . Q^T [D x 16]
//       v_mfma_f32_16x16x32 (bf16 or f16), D/32 of them.  Lane (t = l%16,
//       kg = l/16) loads 8 consecutive elements of key row t, which is the
//       A operand as it sits in memory; Q^T (B operand, lane = head l%16) stays
//       in registers.  Heads beyond G are zero rows.
//   The result leaves lane (h = l%16, kg) with the scores of head h for
//   tokens 4kg..4kg+3: the online softmax of head h (max across the four kg
//   lanes) needs two cross-lane steps, and those four weights are already the
//   B operand of the next product.
//   out^T [D x 16 heads] += V^T [D x 16 tok] . P^T [16 tok x 16 heads]
//       v_mfma_f32_16x16x16, D/16 of them.  Lane (m = l%16, kg) loads the
//       D/16 elements m*D/16.. of value rows 4kg..4kg+3 (four fully used
//       256-byte rows per load instruction) and regroups them with v_perm so
//       product j sees elements m*D/16 + j of those four rows.  The
//       accumulator of head h stays in lanes h, so the rescale by the softmax
//       correction is lane-local.
//   int8 keys: the contraction order over head_dim is free, so lane
//   (t, kg) reads 16 consecutive codes of key row t at byte 16kg + 64j
//   (j < D / 64) and product kk takes the half kk % 2 of load kk / 2; Q^T
//   takes the same elements.  Half as many key loads as one per product,
//   each covering half of every row it touches (about 6% faster).  Int8
//   products run in f16 whatever the q type: a code k, flipped to the byte
//   k + 128 and put under the high byte 0x64 by a byte permute, is the f16
//   value 1152 + k, and one packed f16 add per pair leaves k exactly (about
//   1.25 instructions per code, against 1.5 for a byte convert per code and
//   a pack into bf16, whose 7-bit mantissa cannot hold a code).  q enters
//   as f16 scaled by a power of two per head (its largest element to
//   [2^14, 2^15)), undone in the score scale.  The weights enter as f16
//   hi + lo pairs: the tile's value scale joins their exponent (log2 of it
//   added to the scores, so the running maximum covers it and a row's
//   largest weight sits at 2^7, far from f16's limits), and the sum of
//   weights takes each one times 1 / scale.
//   4-bit keys: the contraction order over head_dim is free, so lane
//   (t, kg) reads elements kg*D/4 .. +D/4-1 of key row t in one load (16
//   bytes at head_dim 128) and Q^T takes the same elements; 4-bit values
//   are read 4 (or 2) bytes per row.  Codes become 16-bit operands without
//   a convert: each nibble, XORed to c + 8 (or 7 - c), is byte-permuted
//   under a constant high byte, which spells the exact bf16 value 136 + c
//   in the low half of an operand pair and c - 135 in the high half (f16:
//   1032 + c and c - 1031, removed exactly by one packed add).  Key pairs
//   come out as elements (0,2), (4,6), (1,3), (5,7) of each 8, and q is
//   permuted to match once at load.  In bf16 the offsets stay in the
//   products: scores carry 136 x (sum of the head's q in low halves) - 135
//   x (sum in high halves), taken out with the score scale, and the value
//   accumulators 136 x (weights of even tokens) - 135 x (weights of odd
//   tokens), accumulated by one more product per tile against a constant
//   operand and subtracted at the end.  The opposite signs keep a common
//   component of q or of the weights from inflating the accumulators.
//   Weights enter the product as a bf16 (or f16) pair hi + lo, hi = p rounded
//   and lo = p - hi rounded, which keeps about 16 mantissa bits at the cost
//   of a second MFMA per product; decode is HBM-bound, so it is free.
// The workgroup's wavefronts take the partition's tiles round-robin and
// merge through LDS at the end.  Each wave issues the loads of its next
// tile before it computes the current one (two register buffers).  For
// 16-bit KV the second buffer costs a wave per SIMD (172 VGPRs: two
// workgroups per compute unit instead of three); with the grid sized to
// one round of resident workgroups that measured 4% faster (long-context
// GQA 257-260 -> 248 us) than loading two tiles and then computing both.
#include <type_traits>

#include "attention_common.h"
#include "mfma_common.h"

namespace pkv {
namespace {

// Wavefronts per workgroup, by storage width: four for 16-bit KV; two for
// int8 and 4-bit codes, whose small tiles leave each wave's loads
// latency-bound, so fewer waves per partition (more tiles each) measured
// faster (4-bit about 8%, int8 about 1.5%).
#ifndef PKV_MFMA_WAVES
#define PKV_MFMA_WAVES 4
#endif
#ifndef PKV_MFMA_WAVES_CODES
#define PKV_MFMA_WAVES_CODES 2
#endif
template <typename KT>
constexpr int mfma_waves() {
  return KT::bits == 16 ? PKV_MFMA_WAVES : PKV_MFMA_WAVES_CODES;
}
// Tiles per load group (a wave computes one group while the next is in
// flight), by storage width.
#ifndef PKV_MFMA_UNROLL16
#define PKV_MFMA_UNROLL16 1
#endif
// int8: two tiles per group (154 VGPRs, six workgroups per compute unit)
// measured about 1.3% faster than one at one round of workgroups; 4-bit:
// one (two measured 7% slower).
#ifndef PKV_MFMA_UNROLL_I8
#define PKV_MFMA_UNROLL_I8 2
#endif
#ifndef PKV_MFMA_UNROLL_CODES
#define PKV_MFMA_UNROLL_CODES 1
#endif
template <typename KT>
constexpr int mfma_unroll() {
  return KT::bits == 16 ? PKV_MFMA_UNROLL16 : KT::bits == 8 ? PKV_MFMA_UNROLL_I8 : PKV_MFMA_UNROLL_CODES;
}
// Whether a wave issues the next group's loads before computing the current
// one (two register buffers), by storage width.
#ifndef PKV_MFMA_PIPE16
#define PKV_MFMA_PIPE16 1
#endif
#ifndef PKV_MFMA_PIPE_CODES
#define PKV_MFMA_PIPE_CODES 1
#endif
template <typename KT>
constexpr bool mfma_pipe() {
  return KT::bits == 16 ? PKV_MFMA_PIPE16 != 0 : PKV_MFMA_PIPE_CODES != 0;
}
#ifndef PKV_MFMA_WPE16
#define PKV_MFMA_WPE16 1
#endif

template <typename QT, typename KT, int D, bool NTV>
__global__ __launch_bounds__(64 * mfma_waves<KT>())
__attribute__((amdgpu_waves_per_eu(KT::bits == 16 ? PKV_MFMA_WPE16 : 1))) void decode_mfma_kernel(
    AttnArgs a, int group) {
  constexpr int kWaves = mfma_waves<KT>();
  constexpr int kUnroll = mfma_unroll<KT>();
  static_assert(64 % kUnroll == 0, "the unroll must divide the table chunk");
  constexpr bool kInt4 = (KT::bits == 4);
  constexpr bool kInt8 = (KT::bits == 8);
  constexpr bool kScaled = kInt4 || kInt8;    // codes with per-tile scales
  constexpr int NK = D / 32;                  // QK products per tile
  constexpr int NV = D / 16;                  // PV products per tile (= elements per lane row)
  constexpr bool kWideK8 = kInt8;              // int8 keys: 16 codes per lane load
  constexpr int NKL = kInt4 ? 1 : kWideK8 ? NK / 2 : NK;   // K loads per lane and tile
  constexpr int KB = kInt4 ? D / 8 : kWideK8 ? 16 : 8 * KT::bytes;   // bytes of one lane's K load
  constexpr int VB = NV * KT::bits / 8;       // bytes of one lane's V chunk
  constexpr int ROW = D * KT::bits / 8;       // bytes of one token row
  constexpr int TILE = 16 * ROW;
  using M = Mx<QT>;
  // int8 codes run both products in f16 whatever the q type: a code byte
  // under the high byte 0x64 (or 0xE4) is an exact f16 value, so one byte
  // permute forms two operands (bf16's 7-bit mantissa cannot hold 8 bits)
  using MK = typename std::conditional<KT::bits == 8, Mx<F16>, Mx<QT>>::type;

  const int wave = wave_uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;   // head (B/D operand column) or token / dim row (A operand)
  const int kg = lane >> 4;

  const WgCoord wc = wg_coord(a, a.hkv);
  if (wc.row < 0) return;   // past every row's partitions
  const int part = wc.part;
  const int row = wc.row;
  const int kvh = wc.hg;
  const int hbase = kvh * group;

  // Table entries, q and the context length go out together.
  const int seq = row_seq(a, row);
  const int b0 = (part * a.part_tokens) >> 4;
  const int bmax = min(a.part_tokens >> 4, (a.max_blocks << a.bs_shift) - b0);
  const int32_t* trow = a.tables + static_cast<int64_t>(seq) * a.max_blocks;
  TableChunk tc;
  tc.fetch(trow, b0, wave, kWaves, 0, bmax, a.bs_shift);

  // Q^T operand: head r16, elements 32kk + 8kg .. +7 (4-bit keys:
  // kg*D/4 + 8kk .. +7, the elements that lane's key load holds).
  u32x4 qop[NK];
  // Offsets left in the operands and removed from the sums later: bf16
  // 4-bit codes, and int8 codes (below).
  constexpr bool kOffset = kInt4 && M::kOffset4;
  float kcorr = 0.f;                                // the offsets' share of every score
  float qinv = 1.f;                                 // int8: 2^-e, undoing q's f16 scaling
  if constexpr (kInt8) {
    // q as f16 operands: each head's row scaled by 2^e so that its largest
    // |element| lies in [2^14, 2^15) (exact: bf16 and f16 values have at
    // most 11 significant bits; only elements 2^28 or more below the row's
    // largest fall to f16 subnormals).  Scores are divided by 2^e again
    // through the score scale.
    const uint16_t* qp = static_cast<const uint16_t*>(a.q);
    const bool live = r16 < group;
    const int64_t qrow = (static_cast<int64_t>(row) * a.hq + hbase + (live ? r16 : 0)) * D;
    float qf[NK][8];
    float amax = 0.f;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const int e0 = 64 * (kk / 2) + 16 * kg + 8 * (kk % 2);   // the lane's 16-code key load
      u32x4 v = *reinterpret_cast<const u32x4*>(qp + qrow + e0);
      v = live ? v : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        qf[kk][2 * i] = M::lo(dw(v, i));
        qf[kk][2 * i + 1] = M::hi(dw(v, i));
        amax = fmaxf(amax, fmaxf(fabsf(qf[kk][2 * i]), fabsf(qf[kk][2 * i + 1])));
      }
    }
    amax = max_xor32(max_xor16(amax));   // the head's four lane groups
    const int e = amax > 0.f ? min(max(15 - __builtin_amdgcn_frexp_expf(amax), -126), 100) : 0;
    qinv = __builtin_amdgcn_ldexpf(1.f, -e);
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = MK::pack(__builtin_amdgcn_ldexpf(qf[kk][2 * i], e),
                        __builtin_amdgcn_ldexpf(qf[kk][2 * i + 1], e));
      qop[kk] = u32x4{w[0], w[1], w[2], w[3]};
    }
  } else {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q);
    const bool live = r16 < group;
    const int64_t qrow = (static_cast<int64_t>(row) * a.hq + hbase + (live ? r16 : 0)) * D;
    float qlo = 0.f, qhi = 0.f;   // q in low / high halves of the operand pairs
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const int e0 = kInt4 ? kg * (D / 4) + 8 * kk : 32 * kk + 8 * kg;
      u32x4 v = *reinterpret_cast<const u32x4*>(qp + qrow + e0);
      v = live ? v : u32x4{0u, 0u, 0u, 0u};
      if constexpr (kInt4) {
        // the element order of the unpacked 4-bit keys: (0,2), (4,6), (1,3), (5,7)
        qop[kk] = u32x4{__builtin_amdgcn_perm(v.y, v.x, 0x05040100u),
                        __builtin_amdgcn_perm(v.w, v.z, 0x05040100u),
                        __builtin_amdgcn_perm(v.y, v.x, 0x07060302u),
                        __builtin_amdgcn_perm(v.w, v.z, 0x07060302u)};
        if constexpr (kOffset) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            qlo += M::lo(dw(qop[kk], i));
            qhi += M::hi(dw(qop[kk], i));
          }
        }
      } else {
        qop[kk] = v;
      }
    }
    if constexpr (kOffset) {
      qlo = sum_xor32(sum_xor16(qlo));
      qhi = sum_xor32(sum_xor16(qhi));
      kcorr = M::kOffsetLo4 * qlo + M::kOffsetHi4 * qhi;
    }
  }

  const int ctx = row_ctx(a, row, seq);
  const int nparts = (ctx + a.part_tokens - 1) / a.part_tokens;
  if (part >= max(nparts, 1)) return;
  const int t0 = part * a.part_tokens;
  const int t1 = min(ctx, t0 + a.part_tokens);
  const int nb = ((t1 + 15) >> 4) - b0;
  const int nbw = nb > wave ? (nb - wave + kWaves - 1) / kWaves : 0;   // this wave's tiles

  float m = kNegInf, l = 0.f;
  f32x4 acc[NV];
  f32x4 wacc = {0.f, 0.f, 0.f, 0.f};   // bf16 4-bit: the offsets' share of acc
#pragma unroll
  for (int j = 0; j < NV; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint8_t* kc = static_cast<const uint8_t*>(a.kc);
  const uint8_t* vc = static_cast<const uint8_t*>(a.vc);
  // lane offsets inside a tile
  const int koff = r16 * ROW + (kInt4 || kWideK8 ? kg * KB : 8 * kg * KT::bytes);
  constexpr int KSTEP = kWideK8 ? 64 : 32 * KT::bytes;   // bytes between a lane's K loads
  const int voff = (4 * kg) * ROW + r16 * VB;                           // + e * ROW
  // A decode step that appends (new_k set, 16-bit K/V): position ctx - 1 is
  // the step's new token, whose K and V rows come from new_k and new_v; the
  // lanes that hold parts of that row read them there and, once the tile is
  // processed, write them to the token's slot in the cache.
  constexpr bool kCanAppend = KT::bits == 16;
  const bool append = kCanAppend && a.new_k != nullptr;
  const int64_t new_row = (static_cast<int64_t>(seq) * a.hkv + kvh) * ROW;

  // Tiles of K and V travel in groups of kUnroll through two register
  // buffers: the loads of the next group are issued before the current one
  // is computed, so each wave keeps a group in flight while it works.
  struct TileBuf {
    u32x4 kr[kUnroll][NKL], vr[kUnroll][4];
    int phys[kUnroll];
    int nrow[kUnroll];          // row of the step's new token in the tile, or -1
    int64_t tofs[kUnroll];
  };
  auto issue = [&](int k, TileBuf& tb) {
    if (k > 0 && (k & 63) == 0) tc.fetch(trow, b0, wave, kWaves, k, bmax, a.bs_shift);
    auto& kr = tb.kr;
    auto& vr = tb.vr;
    auto& phys = tb.phys;
    auto& nrow = tb.nrow;
    auto& tofs = tb.tofs;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      int p = -1;
      nrow[u] = -1;
      tofs[u] = 0;
      if (k + u < nbw) {
        p = tc.get(k + u);
        if (p < 0 || p >= a.num_blocks) p = -1;
      }
      phys[u] = p;
      if (p >= 0) {
        const int tt = b0 + wave + kWaves * (k + u);
        const int64_t toff = tile_index(a, p, kvh, tt) * TILE;
        tofs[u] = toff;
        if (append) {
          const int r = ctx - 1 - tt * 16;   // wave-uniform
          nrow[u] = (r >= 0 && r < 16) ? r : -1;
        }
        // Value loads cover whole rows; with NTV (the streaming load
        // policy) they carry the non-temporal hint, so tiles read once pass
        // through the caches without evicting what is reused.  Key loads
        // take parts of each row over several instructions and stay cached
        // (streaming them measured slower for every storage type).
        const bool knew = kCanAppend && nrow[u] == r16;
#pragma unroll
        for (int kk = 0; kk < NKL; ++kk) {
          const uint8_t* kp = knew ? static_cast<const uint8_t*>(a.new_k) + new_row +
                                         (koff - r16 * ROW) + kk * KSTEP
                                   : kc + toff + koff + kk * KSTEP;
          kr[u][kk] = load_kv_bytes<KB, false>(kp);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool vnew = kCanAppend && nrow[u] == 4 * kg + e;
          const uint8_t* vp = vnew ? static_cast<const uint8_t*>(a.new_v) + new_row + r16 * VB
                                   : vc + toff + voff + e * ROW;
          vr[u][e] = load_kv_bytes<VB, NTV>(vp);
        }
      }
    }
  };
  auto compute = [&](int k, TileBuf& tb) {
    auto& kr = tb.kr;
    auto& vr = tb.vr;
    auto& phys = tb.phys;
    auto& nrow = tb.nrow;
    auto& tofs = tb.tofs;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (k + u >= nbw) break;
      const int p = phys[u];
      const int tpos = (b0 + wave + kWaves * (k + u)) * 16;
      float kscale = 1.f, vscale = 1.f;
      if (kScaled && p >= 0) {
        kscale = a.ks[static_cast<int64_t>(p) * a.hkv + kvh];
        vscale = a.vs[static_cast<int64_t>(p) * a.hkv + kvh];
      }
      // ---- scores^T = K . Q^T
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        u32x4 kop;
        if constexpr (kInt4) {
          const uint32_t w = dw(kr[u][0], kk);
          const uint32_t lo = nib_lo(w, kFlipPairs), hi = nib_hi(w, kFlipPairs);
          kop = u32x4{M::fix4(magic_pair(M::kMagic4, lo, 0)), M::fix4(magic_pair(M::kMagic4, lo, 1)),
                      M::fix4(magic_pair(M::kMagic4, hi, 0)), M::fix4(magic_pair(M::kMagic4, hi, 1))};
        } else if constexpr (kInt8) {
          // exact f16 codes, two per permute and add (i8_pair)
          const u32x4& kw = kr[u][kk / 2];
          const int h2 = 2 * (kk % 2);
          const uint32_t w0 = dw(kw, h2) ^ 0x80808080u, w1 = dw(kw, h2 + 1) ^ 0x80808080u;
          kop = u32x4{i8_pair(w0, 0), i8_pair(w0, 1), i8_pair(w1, 0), i8_pair(w1, 1)};
        } else {
          kop = kr[u][kk];
        }
        s = MK::k32(kop, qop[kk], s);
      }
      // int8: the tile's value scale enters the weights through the exponent
      // (lv = log2 of the scale), so the running maximum covers it and the
      // largest weight of a row sits at 2^7, well inside f16's range; the
      // sum l takes each weight times 1 / scale.  A tile whose scale is 0
      // (or below the smallest normal float) holds zero values: its weights
      // count in l and its products get zero weights.
      const bool vok = !kInt8 || vscale >= 1.17549435e-38f;
      const float lv = (kInt8 && vok) ? __log2f(vscale) : 0.f;
      const float rv = (kInt8 && vok) ? __builtin_amdgcn_rcpf(vscale) : 1.f;
      const float sc = kscale * a.scale_log2 * qinv;
      const float nc = -kcorr * sc + lv;   // the offsets' share (4-bit) and log2 of the value scale (int8)
      float sv[4];
      float tmax = kNegInf;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool valid = (p >= 0) && (tpos + 4 * kg + i < t1);
        sv[i] = valid ? ((kOffset || kInt8) ? fmaf(s[i], sc, nc) : s[i] * sc) : kNegInf;
        tmax = fmaxf(tmax, sv[i]);
      }
      tmax = max_xor32(max_xor16(tmax));
      const bool grow = tmax > m + kRescaleSlack;
      if (__any(grow)) {   // rare after the first tiles: skips the accumulator rescale
        const float mn = grow ? tmax : m;
        const float alpha = grow ? fast_exp2(m - mn) : 1.f;
        m = mn;
        l *= alpha;
#pragma unroll
        for (int j = 0; j < NV; ++j) acc[j] *= alpha;
        if constexpr (kOffset) wacc *= alpha;
      }
      const float ms = (m == kNegInf) ? 0.f : m;
      float pv[4];
      if constexpr (kInt8) {
        const float ms7 = ms - 7.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pw = fast_exp2(sv[i] - ms7);
          l = fmaf(pw, rv, l);
          pv[i] = vok ? pw : 0.f;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pw = fast_exp2(sv[i] - ms);
          l += pw;
          pv[i] = pw * vscale;
        }
      }
      // ---- P^T operand as hi + lo pairs
      const uint32_t h01 = MK::pack(pv[0], pv[1]);
      const uint32_t h23 = MK::pack(pv[2], pv[3]);
      const u32x2 phi = {h01, h23};
      const u32x2 plo = {MK::pack(pv[0] - MK::lo(h01), pv[1] - MK::hi(h01)),
                         MK::pack(pv[2] - MK::lo(h23), pv[3] - MK::hi(h23))};
      // K = 32 of one product: the lane's 4 keys with the hi weights, then
      // the same 4 keys with the lo weights (the A operand repeats them)
      const u32x4 pcat = {phi.x, phi.y, plo.x, plo.y};
      // ---- out^T += V^T . P^T.  Value rows past the context (only in the
      // partly filled last block) may hold anything: they are zeroed (4-bit
      // and int8 codes always form finite operands and meet zero weights, so
      // they need no masking).
      u32x4 vrow[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) vrow[e] = vr[u][e];
      if (!kInt4 && !kInt8 && !(p >= 0 && tpos + 16 <= t1)) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool valid = (p >= 0) && (tpos + 4 * kg + e < t1);
          vrow[e] = valid ? vrow[e] : u32x4{0u, 0u, 0u, 0u};
        }
      }
      if constexpr (kInt4) {
        // rows 4kg..4kg+3 hold NV codes each (one dword, or its low half);
        // even rows take the low halves of the operand pairs, odd rows the
        // high halves.  x01[h][w] interleaves rows 0 and 1 byte by byte:
        // elements 4w + h and 4w + 2 + h (x23 the same for rows 2 and 3)
        constexpr int NW = NV / 4;
        uint32_t x01[2][NW], x23[2][NW];
        {
          const uint32_t l0 = nib_lo(vrow[0].x, kFlipLow), l1 = nib_lo(vrow[1].x, kFlipHigh);
          const uint32_t l2 = nib_lo(vrow[2].x, kFlipLow), l3 = nib_lo(vrow[3].x, kFlipHigh);
          const uint32_t h0 = nib_hi(vrow[0].x, kFlipLow), h1 = nib_hi(vrow[1].x, kFlipHigh);
          const uint32_t h2 = nib_hi(vrow[2].x, kFlipLow), h3 = nib_hi(vrow[3].x, kFlipHigh);
#pragma unroll
          for (int w = 0; w < NW; ++w) {
            const uint32_t sel = w ? 0x07030602u : 0x05010400u;
            x01[0][w] = __builtin_amdgcn_perm(l1, l0, sel);
            x01[1][w] = __builtin_amdgcn_perm(h1, h0, sel);
            x23[0][w] = __builtin_amdgcn_perm(l3, l2, sel);
            x23[1][w] = __builtin_amdgcn_perm(h3, h2, sel);
          }
        }
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          const int h = j & 1, w = j >> 2, pp = (j >> 1) & 1;
          const uint32_t v01 = M::fix4(magic_pair(M::kMagic4, x01[h][w], pp));
          const uint32_t v23 = M::fix4(magic_pair(M::kMagic4, x23[h][w], pp));
          acc[j] = M::k32(u32x4{v01, v23, v01, v23}, pcat, acc[j]);
        }
        if constexpr (kOffset) {
          constexpr uint32_t o = M::kOffsetPair4;
          wacc = M::k32(u32x4{o, o, o, o}, pcat, wacc);
        }
      } else if constexpr (kInt8) {
        // rows 4kg..4kg+3 hold NV codes each (NV / 4 dwords): a flip per
        // row dword, one permute interleaving two rows byte by byte, then
        // each operand pair (row 0's element j low, row 1's high) exact in
        // f16 by one permute and one packed add (i8_pair)
        constexpr int NW = NV / 4;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const uint32_t r0 = dw(vrow[0], w) ^ 0x80808080u, r1 = dw(vrow[1], w) ^ 0x80808080u;
          const uint32_t r2 = dw(vrow[2], w) ^ 0x80808080u, r3 = dw(vrow[3], w) ^ 0x80808080u;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint32_t sel = h ? 0x07030602u : 0x05010400u;
            const uint32_t x01 = __builtin_amdgcn_perm(r1, r0, sel);
            const uint32_t x23 = __builtin_amdgcn_perm(r3, r2, sel);
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
              const int j = 4 * w + 2 * h + pp;
              const uint32_t v01 = i8_pair(x01, pp);
              const uint32_t v23 = i8_pair(x23, pp);
              acc[j] = MK::k32(u32x4{v01, v23, v01, v23}, pcat, acc[j]);
            }
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          const uint32_t v01 = pair_of(vrow[0], vrow[1], j);
          const uint32_t v23 = pair_of(vrow[2], vrow[3], j);
          acc[j] = M::k32(u32x4{v01, v23, v01, v23}, pcat, acc[j]);
        }
      }
      if constexpr (kCanAppend) {
        if (nrow[u] >= 0) {   // the new token's rows to their slot (vector stores)
          uint8_t* kw = static_cast<uint8_t*>(const_cast<void*>(a.kc)) + tofs[u] + koff;
          uint8_t* vw = static_cast<uint8_t*>(const_cast<void*>(a.vc)) + tofs[u] + voff;
          if (nrow[u] == r16) {
#pragma unroll
            for (int kk = 0; kk < NKL; ++kk) store_bytes<KB>(kw + kk * KSTEP, kr[u][kk]);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (nrow[u] == 4 * kg + e) store_bytes<VB>(vw + e * ROW, vr[u][e]);
        }
      }
    }
  };
  if constexpr (mfma_pipe<KT>()) {
    TileBuf tb0, tb1;
    issue(0, tb0);
    for (int k = 0; k < nbw; k += 2 * kUnroll) {
      issue(k + kUnroll, tb1);   // tiles past the wave's last are not loaded
      compute(k, tb0);
      if (k + kUnroll >= nbw) break;
      issue(k + 2 * kUnroll, tb0);
      compute(k + kUnroll, tb1);
    }
  } else {
    for (int k = 0; k < nbw; k += kUnroll) {
      TileBuf tb;
      issue(k, tb);
      compute(k, tb);
    }
  }

  // Sum of each head's weights over its four lanes.
  l = sum_xor32(sum_xor16(l));

  __shared__ float sm_o[kWaves][16][D];
  __shared__ float sm_m[kWaves][16];
  __shared__ float sm_l[kWaves][16];
  // acc[j][i] of lane (h, kg) is element NV*(4kg + i) + j of head h's row.
  if constexpr (kOffset) {
#pragma unroll
    for (int j = 0; j < NV; ++j) acc[j] -= wacc;
  }
#pragma unroll
  for (int j = 0; j < NV; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) sm_o[wave][r16][NV * (4 * kg + i) + j] = acc[j][i];
  if (kg == 0) {
    sm_m[wave][r16] = m;
    sm_l[wave][r16] = l;
  }
  __syncthreads();
  finish_rows<kWaves, 16, D>(a, sm_o, sm_m, sm_l, group, row, hbase, part, nparts,
                             threadIdx.x, blockDim.x);
  // With counters, the last partition of a split row to finish merges it.
  if (a.counters != nullptr && nparts > 1) {
    __shared__ int sm_last;
    merge_if_last(a, row, hbase, group, nparts, D, threadIdx.x, blockDim.x,
                  [] { __syncthreads(); },
                  [&](int v) {
                    if (threadIdx.x == 0) sm_last = v;
                    __syncthreads();
                    return sm_last;
                  });
  }
}

// The kernel one launch runs: one workgroup of mfma_waves<KT>() waves per
// (partition, row, KV head).
struct MfmaKernel {
  const void* fn;
  int threads;
};

template <typename QT, typename KT>
MfmaKernel pick_qk(int D, bool nt) {
  constexpr int threads = 64 * mfma_waves<KT>();
  if (nt)
    return {D == 64 ? reinterpret_cast<const void*>(&decode_mfma_kernel<QT, KT, 64, true>)
                    : reinterpret_cast<const void*>(&decode_mfma_kernel<QT, KT, 128, true>),
            threads};
  return {D == 64 ? reinterpret_cast<const void*>(&decode_mfma_kernel<QT, KT, 64, false>)
                  : reinterpret_cast<const void*>(&decode_mfma_kernel<QT, KT, 128, false>),
          threads};
}

// Null fn for a q type the matrix-core path does not take.
MfmaKernel pick_mfma(pkv_dtype q_dt, pkv_dtype kv_dt, int D, bool nt) {
  if (q_dt == PKV_BF16)
    return kv_dt == PKV_I8   ? pick_qk<BF16, I8>(D, nt)
           : kv_dt == PKV_I4 ? pick_qk<BF16, I4>(D, nt)
                             : pick_qk<BF16, BF16>(D, nt);
  if (q_dt == PKV_F16)
    return kv_dt == PKV_I8   ? pick_qk<F16, I8>(D, nt)
           : kv_dt == PKV_I4 ? pick_qk<F16, I4>(D, nt)
                             : pick_qk<F16, F16>(D, nt);
  return {nullptr, 0};
}

}  // namespace

pkv_status launch_decode_mfma(const AttnArgs& a, pkv_dtype q_dt, pkv_dtype kv_dt, int D,
                              int group, hipStream_t st) {
  if (group > 16) return fail(PKV_ERR_UNSUPPORTED, "MFMA decode: group %d > 16", group);
  const MfmaKernel k = pick_mfma(q_dt, kv_dt, D, a.stream_kv != 0);
  if (k.fn == nullptr) return fail(PKV_ERR_UNSUPPORTED, "MFMA decode needs 16-bit q");
  AttnArgs args = a;
  int grp = group;
  void* params[] = {&args, &grp};
  const hipError_t e = hipLaunchKernel(k.fn, dim3(a.num_parts * a.num_rows * a.hkv),
                                       dim3(k.threads), params, 0, st);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(PKV_ERR_DEVICE, "paged attention (MFMA) launch failed: %s", hipGetErrorString(e));
  }
  PKV_LAUNCH_CHECK("paged attention (MFMA)");
  return PKV_OK;
}

pkv_status decode_mfma_occupancy(pkv_dtype q_dt, pkv_dtype kv_dt, int D, bool nt, int* wg_per_cu) {
  const MfmaKernel k = pick_mfma(q_dt, kv_dt, D, nt);
  if (k.fn == nullptr) return fail(PKV_ERR_UNSUPPORTED, "MFMA decode needs 16-bit q");
  int n = 0;
  const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k.fn, k.threads, 0);
  if (e != hipSuccess) return fail(PKV_ERR_DEVICE, "MFMA decode occupancy: %s", hipGetErrorString(e));
  *wg_per_cu = n;
  return PKV_OK;
}

}  // namespace pkv
