// Paged decode attention, wavefront path (any storage dtype, small head
// groups).  Also serves fp32 chunked prefill, one query row per workgroup.
// 4-bit codes are read 8 bytes per lane (16 codes), so a lane holds as many
// elements as with int8 and the register budget is the same.
//
// What it computes (cnnetsun.cn "别再让GPU内存拖后腿了…" §3.1): for each
// block of the sequence's table, the query's scores against that block's
// keys; one softmax over all scores after scaling; the blocks' value rows
// summed with those weights.  The softmax is taken online, block by block
// (running max and sum rescaled as the max grows), which gives the same
// result up to rounding without materialising the scores.
//
// Layout on gfx950.  A workgroup of 8 (or 16) wavefronts owns one (query
// row, context partition) and G query heads that share one KV head.
// One (block, KV head) tile of K is 16 rows x head_dim contiguous elements:
// 4 KiB at bf16 / head_dim 128, read as 16-byte chunks so one wavefront load
// instruction covers 1 KiB of consecutive bytes.  C = row_bytes / 16 lanes
// hold one token row, so a load covers 64 / C tokens and a tile takes C / 4
// loads.  Each lane dots its chunk with the matching slice of q, the C lanes
// of a row combine with DPP row operations, and every lane of the row ends
// with the token's score.  The lanes that hold token t's K chunk also load
// its V chunk, so the softmax weight never leaves its lanes: the PV product
// accumulates per lane, and rows, then wavefronts, are merged once at the
// end.  Wavefronts take blocks round-robin.  With streaming loads a wave
// loads a block's K and V into one set of registers and rotates them: the next block's K loads
// go out once the scores are taken, its V loads once the values are
// summed, so a tile stays in flight while the wave computes (2% faster at
// the 7B shape than loading each block after the previous one).  At bf16 /
// head_dim 128 the kernel takes 109 VGPRs (four waves per SIMD).  Pinning
// the widening of the value tiles next to the products (fewer registers,
// six waves per SIMD) measured slower.
// For 16-bit keys the score uses packed dot2 instructions on the raw pairs,
// and only the partly filled last block of a context pays for per-row
// masking.
//
// With NT (the caller's load policy, see AttnArgs::stream_kv) the K/V loads
// carry the non-temporal hint: a decode that reads every tile once streams
// them through the caches and leaves the lines that are reused (q, table
// entries, partial states) in place, about 10% faster at the 7B shape.
// Blocks shared by several sequences, and the keys every row of an fp32
// prefill chunk reads, are better served by cached loads.
//
// Workgroups are ordered with the head group fastest (see wg_coord): the
// KV-head tiles of one block are adjacent in the pool, so concurrent
// workgroups spread their reads over all memory channels.
#include <type_traits>

#include "attention_common.h"

// A multiply-add is fused only where the code says fmaf.  Left to the
// compiler, the fusing depends on how the loop around it is laid out, and the
// streaming and cached loop forms below would round differently.
#pragma clang fp contract(off)

namespace pkv {
namespace {

// Wavefronts per workgroup: 8, or 16 for a call that streams one head of
// 16-bit K/V (MHA decode over a pool larger than the caches) with partitions
// of at least kWideMinTokens.  Eight waves with 384-token partitions
// measured about 2% faster than four at the 7B shape; sixteen waves with
// 1,536-token partitions another 3% (the prologue and the merge amortise
// over more tiles, and most contexts fit one partition and write no partial
// state).  Sixteen waves lose with short partitions (1.5 tiles per wave at
// 384 tokens) and on cache-resident shared blocks, and would not fit the
// registers of a multi-head group.
#ifndef PKV_WAVE_WAVES
#define PKV_WAVE_WAVES 8
#endif
constexpr int kWavesDefault = PKV_WAVE_WAVES;
constexpr int kWavesWide = 16;
constexpr int kWideMinTokens = 1024;

// Dot product of one 16-byte chunk of 16-bit keys with the matching q
// chunk, both as packed pairs: v_dot2 forms the two exact products and adds
// them to the fp32 accumulator, two elements per instruction and no
// separate widening.
template <typename T> struct PackedDot { static constexpr bool ok = false; };
template <> struct PackedDot<BF16> {
  static constexpr bool ok = true;
  typedef __bf16 x2 __attribute__((ext_vector_type(2)));
  __device__ __forceinline__ static float step(uint32_t k, uint32_t q, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(x2, k), __builtin_bit_cast(x2, q), acc,
                                           false);
  }
};
template <> struct PackedDot<F16> {
  static constexpr bool ok = true;
  typedef _Float16 x2 __attribute__((ext_vector_type(2)));
  __device__ __forceinline__ static float step(uint32_t k, uint32_t q, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(x2, k), __builtin_bit_cast(x2, q), acc, false);
  }
};
template <typename T>
__device__ __forceinline__ float chunk_dot(const u32x4& k, const u32x4& q) {
  float acc = PackedDot<T>::step(k.x, q.x, 0.f);
  acc = PackedDot<T>::step(k.y, q.y, acc);
  acc = PackedDot<T>::step(k.z, q.z, acc);
  return PackedDot<T>::step(k.w, q.w, acc);
}

// Unpack one dword of stored values to floats (exact widening).
template <typename T> struct UnpackDw;
template <> struct UnpackDw<F32> {
  static constexpr int n = 1;
  __device__ __forceinline__ static void run(uint32_t w, float* x) { x[0] = __uint_as_float(w); }
};
template <> struct UnpackDw<BF16> {
  static constexpr int n = 2;
  __device__ __forceinline__ static void run(uint32_t w, float* x) { x[0] = bf16_lo(w); x[1] = bf16_hi(w); }
};
template <> struct UnpackDw<F16> {
  static constexpr int n = 2;
  __device__ __forceinline__ static void run(uint32_t w, float* x) { x[0] = f16_lo(w); x[1] = f16_hi(w); }
};
template <> struct UnpackDw<I8> {
  static constexpr int n = 4;
  __device__ __forceinline__ static void run(uint32_t w, float* x) {
#pragma unroll
    for (int k = 0; k < 4; ++k) x[k] = i8_at(w, k);
  }
};
template <> struct UnpackDw<I4> {
  static constexpr int n = 8;
  __device__ __forceinline__ static void run(uint32_t w, float* x) {
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = i4_at(w, k);
  }
};

__device__ __forceinline__ uint32_t dword(const u32x4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

template <typename QT, typename KT, int D, int G, bool NT, int NW>
__global__ __launch_bounds__(64 * NW) void decode_wave_kernel(AttnArgs a) {
  constexpr int kWaves = NW;
  // 4-bit codes are read as 8-byte chunks (16 codes, the register shape of
  // an int8 chunk); everything else as 16-byte chunks.
  constexpr int CB = KT::bits == 4 ? 8 : 16;    // bytes of one lane chunk
  constexpr int E = CB * 8 / KT::bits;          // elements per chunk
  constexpr int C = D / E;                      // lanes per token row
  constexpr int TPL = 64 / C;                   // tokens per wavefront load
  constexpr int NL = 16 / TPL;                  // loads per 16-token tile
  constexpr int TILE = 16 * D * KT::bits / 8;   // bytes of one (block, head) tile
  static_assert(C >= 4 && C <= 64 && NL >= 1, "unsupported head_dim / dtype");
  constexpr bool kScaled = (KT::bits <= 8);     // codes with per-tile scales

  const WgCoord wc = wg_coord(a, a.hq / G);
  if (wc.row < 0) return;   // past every row's partitions
  const int part = wc.part;
  const int row = wc.row;
  const int hbase = wc.hg * G;                        // first query head
  const int kvh = hbase / (a.hq / a.hkv);

  const int wave = wave_uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int c = lane % C;
  const int u = lane / C;

  // The table entries, q and the context length do not depend on each
  // other: their loads go out together.
  const int seq = row_seq(a, row);
  const int b0 = (part * a.part_tokens) >> 4;
  const int bmax = min(a.part_tokens >> 4, (a.max_blocks << a.bs_shift) - b0);
  const int32_t* trow = a.tables + static_cast<int64_t>(seq) * a.max_blocks;
  TableChunk tc;
  tc.fetch(trow, b0, wave, kWaves, 0, bmax, a.bs_shift);

  // q slice of every head of the group: elements [c*E, c*E + E), as
  // floats, or as the raw 16-byte chunk when keys and q share a 16-bit type.
  constexpr bool kPacked = PackedDot<KT>::ok && std::is_same<QT, KT>::value;
  float qf[G][E];
  u32x4 qpk[G];
  {
    const typename QT::raw* qp = static_cast<const typename QT::raw*>(a.q);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int64_t off = (static_cast<int64_t>(row) * a.hq + hbase + g) * D + c * E;
      if constexpr (kPacked) {
        qpk[g] = *reinterpret_cast<const u32x4*>(qp + off);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) qf[g][e] = load_elem<QT>(qp, off + e);
      }
    }
  }

  const int ctx = row_ctx(a, row, seq);
  const int nparts = (ctx + a.part_tokens - 1) / a.part_tokens;
  if (part >= max(nparts, 1)) return;
  // Arrival counter of the final merge (below).
  __shared__ int sm_arrived;
  if (threadIdx.x == 0) sm_arrived = 0;
  __syncthreads();

  const int t0 = part * a.part_tokens;
  const int t1 = min(ctx, t0 + a.part_tokens);
  const int nb = ((t1 + 15) >> 4) - b0;

  float m[G], l[G], o[G][E];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = kNegInf;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) o[g][e] = 0.f;
  }

  const uint8_t* kbase = static_cast<const uint8_t*>(a.kc) + lane * CB;
  const uint8_t* vbase = static_cast<const uint8_t*>(a.vc) + lane * CB;

  // One block: scores of this lane's tokens for every head, the online
  // softmax update, and the weighted sum of the value rows.  `masked` is set
  // only for the partly filled last block of the context: its rows past the
  // context may hold anything (NaN included), so they are zeroed, not just
  // given zero weight.  Whole blocks run without any per-row test.
  // One block in two halves: scores and the online softmax from the K tile
  // (leaving the block's weights in pw), then the weighted sum of the V
  // tile's rows.  The rotated loop below issues the next block's K loads
  // between the two.
  auto qk_softmax = [&](auto masked_tag, const u32x4 (&kr)[NL], int tpos, float ksc, float vsc,
                        float (&pw)[G][NL]) {
    constexpr bool masked = decltype(masked_tag)::value;
    float s[G][NL];
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const bool valid = !masked || (tpos + j * TPL + u < t1);
      float kx[E];
      if constexpr (!kPacked) Unpack<KT>::run(kr[j], kx);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float part_dot = 0.f;
        if constexpr (kPacked) {
          part_dot = chunk_dot<KT>(kr[j], qpk[g]);
        } else {
#pragma unroll
          for (int e = 0; e < E; ++e) part_dot = fmaf(qf[g][e], kx[e], part_dot);
        }
        const float dot = group_sum<C>(part_dot);
        s[g][j] = valid ? dot * (ksc * a.scale_log2) : kNegInf;
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float tmax = s[g][0];
#pragma unroll
      for (int j = 1; j < NL; ++j) tmax = fmaxf(tmax, s[g][j]);
      const float mn = fmaxf(m[g], tmax);
      const float ms = (mn == kNegInf) ? 0.f : mn;
      const float alpha = fast_exp2(m[g] - ms);
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        pw[g][j] = fast_exp2(s[g][j] - ms);
        psum += pw[g][j];
      }
      l[g] = fmaf(l[g], alpha, psum);
      m[g] = mn;
#pragma unroll
      for (int e = 0; e < E; ++e) o[g][e] *= alpha;
      if (kScaled) {
#pragma unroll
        for (int j = 0; j < NL; ++j) pw[g][j] *= vsc;   // per-block value scale
      }
    }
  };
  auto pv_sum = [&](auto masked_tag, const u32x4 (&vr)[NL], int tpos, const float (&pw)[G][NL]) {
    constexpr bool masked = decltype(masked_tag)::value;
    constexpr int ND = UnpackDw<KT>::n;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const bool valid = !masked || (tpos + j * TPL + u < t1);
#pragma unroll
      for (int d = 0; d < CB / 4; ++d) {
        float vx[ND];
        UnpackDw<KT>::run(dword(vr[j], d), vx);
#pragma unroll
        for (int i = 0; i < ND; ++i) {
          if (masked) vx[i] = valid ? vx[i] : 0.f;
#pragma unroll
          for (int g = 0; g < G; ++g) o[g][d * ND + i] = fmaf(pw[g][j], vx[i], o[g][d * ND + i]);
        }
      }
    }
  };
  auto block_step = [&](auto masked_tag, const u32x4 (&kr)[NL], const u32x4 (&vr)[NL], int tpos,
                        float ksc, float vsc) {
    float pw[G][NL];
    qk_softmax(masked_tag, kr, tpos, ksc, vsc, pw);
    pv_sum(masked_tag, vr, tpos, pw);
  };

  // A decode step that appends (new_k set, 16-bit or fp32 K/V): position
  // ctx - 1 is the step's new token, whose K and V rows come from new_k and
  // new_v; the lanes that hold that row read it there and, after the block
  // is processed, write it to its slot in the cache.
  constexpr bool kCanAppend = KT::bits >= 16;
  const bool append = kCanAppend && a.new_k != nullptr;
  const int64_t new_off = (static_cast<int64_t>(seq) * a.hkv + kvh) * D * KT::bytes + c * CB;

  // Loads of one block's K and V tiles; false for a table entry outside the
  // pool, which is skipped as if masked.  `toff` receives the tile's byte
  // offset and `nrow` the row of the step's new token in it (or -1).
  auto load_block = [&](int k, u32x4 (&kr)[NL], u32x4 (&vr)[NL], float& ksc, float& vsc,
                        int64_t& toff, int& nrow) {
    if (k > 0 && (k & 63) == 0) tc.fetch(trow, b0, wave, kWaves, k, bmax, a.bs_shift);
    const int p = tc.get(k);
    nrow = -1;
    if (p < 0 || p >= a.num_blocks) return false;
    const int tt = b0 + wave + kWaves * k;
    toff = tile_index(a, p, kvh, tt) * TILE;
    if (append) {
      const int r = ctx - 1 - tt * 16;   // wave-uniform
      nrow = (r >= 0 && r < 16) ? r : -1;
    }
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      if constexpr (CB == 16) {
        const uint8_t* kp = kbase + toff + j * 64 * CB;
        const uint8_t* vp = vbase + toff + j * 64 * CB;
        if (kCanAppend && nrow >= 0 && j * TPL + u == nrow) {
          kp = static_cast<const uint8_t*>(a.new_k) + new_off;
          vp = static_cast<const uint8_t*>(a.new_v) + new_off;
        }
        kr[j] = load_kv<u32x4, NT>(kp);
        vr[j] = load_kv<u32x4, NT>(vp);
      } else {
        const u32x2 k2 = load_kv<u32x2, NT>(kbase + toff + j * 64 * CB);
        const u32x2 v2 = load_kv<u32x2, NT>(vbase + toff + j * 64 * CB);
        kr[j] = u32x4{k2.x, k2.y, 0u, 0u};
        vr[j] = u32x4{v2.x, v2.y, 0u, 0u};
      }
    }
    ksc = vsc = 1.f;
    if (kScaled) {
      ksc = a.ks[static_cast<int64_t>(p) * a.hkv + kvh];
      vsc = a.vs[static_cast<int64_t>(p) * a.hkv + kvh];
    }
    return true;
  };

  // The same loads in two halves, for the rotated loop: the block's
  // position, scales and K tile; then its V tile.
  auto load_k = [&](int k, u32x4 (&kr)[NL], float& ksc, float& vsc, int64_t& toff, int& nrow) {
    if (k > 0 && (k & 63) == 0) tc.fetch(trow, b0, wave, kWaves, k, bmax, a.bs_shift);
    const int p = tc.get(k);
    nrow = -1;
    if (p < 0 || p >= a.num_blocks) return false;
    const int tt = b0 + wave + kWaves * k;
    toff = tile_index(a, p, kvh, tt) * TILE;
    if (append) {
      const int r = ctx - 1 - tt * 16;   // wave-uniform
      nrow = (r >= 0 && r < 16) ? r : -1;
    }
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      if constexpr (CB == 16) {
        const uint8_t* kp = kbase + toff + j * 64 * CB;
        if (kCanAppend && nrow >= 0 && j * TPL + u == nrow) kp = static_cast<const uint8_t*>(a.new_k) + new_off;
        kr[j] = load_kv<u32x4, NT>(kp);
      } else {
        const u32x2 k2 = load_kv<u32x2, NT>(kbase + toff + j * 64 * CB);
        kr[j] = u32x4{k2.x, k2.y, 0u, 0u};
      }
    }
    ksc = vsc = 1.f;
    if (kScaled) {
      ksc = a.ks[static_cast<int64_t>(p) * a.hkv + kvh];
      vsc = a.vs[static_cast<int64_t>(p) * a.hkv + kvh];
    }
    return true;
  };
  auto load_v = [&](u32x4 (&vr)[NL], int64_t toff, int nrow) {
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      if constexpr (CB == 16) {
        const uint8_t* vp = vbase + toff + j * 64 * CB;
        if (kCanAppend && nrow >= 0 && j * TPL + u == nrow) vp = static_cast<const uint8_t*>(a.new_v) + new_off;
        vr[j] = load_kv<u32x4, NT>(vp);
      } else {
        const u32x2 v2 = load_kv<u32x2, NT>(vbase + toff + j * 64 * CB);
        vr[j] = u32x4{v2.x, v2.y, 0u, 0u};
      }
    }
  };

  // The wave's blocks are partition blocks wave, wave + NW, wave + 2 NW,
  // ...; all are whole except possibly the partition's last block, which is
  // then the wave's last.
  const bool partial_tail = (t1 & 15) != 0;
  const int nwhole = nb - (partial_tail ? 1 : 0);
  const int kwhole = nwhole > wave ? (nwhole - wave + kWaves - 1) / kWaves : 0;
  const int kall = kwhole + ((partial_tail && (nb - 1) % kWaves == wave) ? 1 : 0);
  auto step = [&](int k, bool ok, const u32x4 (&kr)[NL], const u32x4 (&vr)[NL], float ksc,
                  float vsc) {
    if (!ok) return;
    const int tpos = (b0 + wave + kWaves * k) * 16;
    if (k < kwhole)
      block_step(std::false_type{}, kr, vr, tpos, ksc, vsc);
    else
      block_step(std::true_type{}, kr, vr, tpos, ksc, vsc);
  };
  // The new token's K or V row to its slot (vector stores), from the
  // registers that hold its tile.
  auto store_new = [&](const u32x4 (&r)[NL], void* cache, int64_t toff, int nrow) {
    if constexpr (kCanAppend) {
      if (nrow >= 0) {
        uint8_t* w = static_cast<uint8_t*>(cache) + lane * CB + toff;
#pragma unroll
        for (int j = 0; j < NL; ++j)
          if (j * TPL + u == nrow) *reinterpret_cast<u32x4*>(w + j * 64 * CB) = r[j];
      }
    }
  };
#ifndef PKV_WAVE_ROTATE
#define PKV_WAVE_ROTATE 1
#endif
  if constexpr (PKV_WAVE_ROTATE != 0 && NT) {
    // Rotated (streaming loads): the next block's K loads go out once this
    // block's scores are taken, its V loads once this block's values are
    // summed, into the same registers, so a wave keeps one tile in flight
    // while it computes.  With cached loads over cache-resident blocks (the
    // shared-prefix beams) it measured 7% slower, so those load each block
    // after the previous one.
    u32x4 kr[NL], vr[NL];
    float ksc = 1.f, vsc = 1.f;
    int64_t toff = 0;
    int nrow = -1;
    bool ok = false;
    if (kall > 0) {
      ok = load_k(0, kr, ksc, vsc, toff, nrow);
      if (ok) load_v(vr, toff, nrow);
    }
#pragma unroll 1
    for (int k = 0; k < kall; ++k) {
      const int tpos = (b0 + wave + kWaves * k) * 16;
      float pw[G][NL];
      if (ok) {
        if (k < kwhole)
          qk_softmax(std::false_type{}, kr, tpos, ksc, vsc, pw);
        else
          qk_softmax(std::true_type{}, kr, tpos, ksc, vsc, pw);
        store_new(kr, const_cast<void*>(a.kc), toff, nrow);
      }
      float ksc_n = 1.f, vsc_n = 1.f;
      int64_t toff_n = 0;
      int nrow_n = -1;
      const bool ok_n = k + 1 < kall && load_k(k + 1, kr, ksc_n, vsc_n, toff_n, nrow_n);
      if (ok) {
        if (k < kwhole)
          pv_sum(std::false_type{}, vr, tpos, pw);
        else
          pv_sum(std::true_type{}, vr, tpos, pw);
        store_new(vr, const_cast<void*>(a.vc), toff, nrow);
      }
      if (ok_n) load_v(vr, toff_n, nrow_n);
      ok = ok_n;
      ksc = ksc_n;
      vsc = vsc_n;
      toff = toff_n;
      nrow = nrow_n;
    }
  } else {
#pragma unroll 1
    for (int k = 0; k < kall; ++k) {
      u32x4 kr[NL], vr[NL];
      float ksc = 1.f, vsc = 1.f;
      int64_t toff = 0;
      int nrow = -1;
      const bool ok = load_block(k, kr, vr, ksc, vsc, toff, nrow);
      step(k, ok, kr, vr, ksc, vsc);
      if (ok) {
        store_new(kr, const_cast<void*>(a.kc), toff, nrow);
        store_new(vr, const_cast<void*>(a.vc), toff, nrow);
      }
    }
  }

  // Merge the token-row groups of the wavefront (lanes c, c+C, c+2C, ...).
#pragma unroll
  for (int off = C; off < 64; off <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float m2 = __shfl_xor(m[g], off);
      const float l2 = __shfl_xor(l[g], off);
      float mn, f1, f2;
      merge_factors(m[g], m2, mn, f1, f2);
      l[g] = fmaf(l[g], f1, l2 * f2);
#pragma unroll
      for (int e = 0; e < E; ++e) o[g][e] = fmaf(o[g][e], f1, __shfl_xor(o[g][e], off) * f2);
      m[g] = mn;
    }
  }

  // Merge the wavefronts through LDS.  Each wave leaves its state there and
  // counts itself in; the last to arrive merges all NW of them and writes,
  // the others end at once (no barrier: a wave with fewer blocks does not wait
  // for the slowest, and its slot frees for the next workgroup).
  __shared__ float sm_o[kWaves][G][D];
  __shared__ float sm_m[kWaves][G];
  __shared__ float sm_l[kWaves][G];
  if (u == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int e = 0; e < E; ++e) sm_o[wave][g][c * E + e] = o[g][e];
      if (lane == 0) {
        sm_m[wave][g] = m[g];
        sm_l[wave][g] = l[g];
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  int arrived = 0;
  if (lane == 0) arrived = atomicAdd(&sm_arrived, 1);
  arrived = __shfl(arrived, 0);
  if (arrived != kWaves - 1) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  finish_rows<kWaves, G, D>(a, sm_o, sm_m, sm_l, G, row, hbase, part, nparts, lane, 64);
  // With counters, the last partition of a split row to finish merges it.
  if (a.counters != nullptr && nparts > 1)
    merge_if_last(a, row, hbase, G, nparts, D, lane, 64, [] {},
                  [](int v) { return __shfl(v, 0); });
}

// Most query heads one workgroup serves.  Each head holds its q slice and an
// output chunk of E floats per lane, so the register file bounds the group:
// four heads of 16-bit or fp32 K/V, two of int8 or 4-bit codes (16 elements
// per lane) fit in 256 VGPRs without spilling to scratch; larger groups are
// split over several workgroups of the grid, which read the same K/V tiles
// at about the same time (the head group is the fastest grid index).
template <typename KT>
constexpr int max_wave_heads() {
  return KT::bits <= 8 ? 2 : 4;
}

// The kernel one launch runs: heads per workgroup are the largest of 4, 2
// and 1 that divides the group, capped by max_wave_heads; one head of
// streamed 16-bit K/V with partitions of at least kWideMinTokens runs the
// 16-wave kernel.
struct WaveKernel {
  const void* fn;
  int threads;
  int heads;   // query heads per workgroup
};

template <typename QT, typename KT, int D, bool NT>
WaveKernel pick_d(int group, int part_tokens) {
  int gw = 1;
  for (int c : {4, 2}) if (c <= max_wave_heads<KT>() && group % c == 0) { gw = c; break; }
  if (gw == 4) {
    if constexpr (max_wave_heads<KT>() >= 4)
      return {reinterpret_cast<const void*>(&decode_wave_kernel<QT, KT, D, 4, NT, kWavesDefault>),
              64 * kWavesDefault, 4};
  }
  if (gw == 2)
    return {reinterpret_cast<const void*>(&decode_wave_kernel<QT, KT, D, 2, NT, kWavesDefault>),
            64 * kWavesDefault, 2};
  if constexpr (KT::bits == 16 && NT) {
    if (part_tokens >= kWideMinTokens)
      return {reinterpret_cast<const void*>(&decode_wave_kernel<QT, KT, D, 1, NT, kWavesWide>),
              64 * kWavesWide, 1};
  }
  return {reinterpret_cast<const void*>(&decode_wave_kernel<QT, KT, D, 1, NT, kWavesDefault>),
          64 * kWavesDefault, 1};
}

template <typename QT, typename KT>
WaveKernel pick_qk(int D, int group, int part_tokens, bool nt) {
  if (!nt)
    return D == 64 ? pick_d<QT, KT, 64, false>(group, part_tokens)
                   : pick_d<QT, KT, 128, false>(group, part_tokens);
  return D == 64 ? pick_d<QT, KT, 64, true>(group, part_tokens)
                 : pick_d<QT, KT, 128, true>(group, part_tokens);
}

WaveKernel pick_wave(pkv_dtype q_dt, pkv_dtype kv_dt, int D, int group, int part_tokens, bool nt) {
  if (kv_dt == PKV_I8) {
    if (q_dt == PKV_BF16) return pick_qk<BF16, I8>(D, group, part_tokens, nt);
    if (q_dt == PKV_F16) return pick_qk<F16, I8>(D, group, part_tokens, nt);
    return pick_qk<F32, I8>(D, group, part_tokens, nt);
  }
  if (kv_dt == PKV_I4) {
    if (q_dt == PKV_BF16) return pick_qk<BF16, I4>(D, group, part_tokens, nt);
    if (q_dt == PKV_F16) return pick_qk<F16, I4>(D, group, part_tokens, nt);
    return pick_qk<F32, I4>(D, group, part_tokens, nt);
  }
  if (q_dt == PKV_BF16) return pick_qk<BF16, BF16>(D, group, part_tokens, nt);
  if (q_dt == PKV_F16) return pick_qk<F16, F16>(D, group, part_tokens, nt);
  return pick_qk<F32, F32>(D, group, part_tokens, nt);
}

}  // namespace

// Decode reads every K/V tile once, so its loads carry the non-temporal
// hint and stream through L2 (a.stream_kv); the fp32 prefill rows of one
// chunk read the same keys, so those loads are cached.
pkv_status launch_decode_wave(const AttnArgs& a, pkv_dtype q_dt, pkv_dtype kv_dt, int D,
                              int group, hipStream_t st) {
  const WaveKernel k = pick_wave(q_dt, kv_dt, D, group, a.part_tokens, a.stream_kv != 0);
  AttnArgs args = a;
  void* params[] = {&args};
  const hipError_t e = hipLaunchKernel(k.fn, dim3(a.num_parts * a.num_rows * (a.hq / k.heads)),
                                       dim3(k.threads), params, 0, st);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(PKV_ERR_DEVICE, "paged attention (wavefront) launch failed: %s", hipGetErrorString(e));
  }
  PKV_LAUNCH_CHECK("paged attention (wavefront)");
  return PKV_OK;
}

pkv_status decode_wave_occupancy(pkv_dtype q_dt, pkv_dtype kv_dt, int D, int group,
                                 int part_tokens, bool nt, int* wg_per_cu, int* heads_per_wg,
                                 int* min_part_tokens) {
  const WaveKernel k = pick_wave(q_dt, kv_dt, D, group, part_tokens, nt);
  *min_part_tokens = k.threads == 64 * kWavesWide ? kWideMinTokens : 0;
  int n = 0;
  const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k.fn, k.threads, 0);
  if (e != hipSuccess) return fail(PKV_ERR_DEVICE, "wavefront decode occupancy: %s", hipGetErrorString(e));
  *wg_per_cu = n;
  *heads_per_wg = k.heads;
  return PKV_OK;
}

}  // namespace pkv
