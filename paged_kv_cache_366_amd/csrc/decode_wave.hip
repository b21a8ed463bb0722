// Paged decode attention, wavefront path (any storage dtype, small head
// groups).  Also serves fp32 chunked prefill, one query row per workgroup.
//
// What it computes (cnnetsun.cn "别再让GPU内存拖后腿了…" §3.1): for each
// block of the sequence's table, the query's scores against that block's
// keys; one softmax over all scores after scaling; the blocks' value rows
// summed with those weights.  The softmax is taken online, block by block
// (running max and sum rescaled as the max grows), which gives the same
// result up to rounding without materialising the scores.
//
// Layout on gfx950.  A workgroup of 4 wavefronts owns one (query row, KV
// head, context partition) and the G query heads that share that KV head.
// One (block, KV head) tile of K is 16 rows x head_dim contiguous elements:
// 4 KiB at bf16 / head_dim 128, read as 16-byte chunks so one wavefront load
// instruction covers 1 KiB of consecutive bytes.  C = row_bytes / 16 lanes
// hold one token row, so a load covers 64 / C tokens and a tile takes C / 4
// loads.  Each lane dots its chunk with the matching slice of q, the C lanes
// of a row combine with DPP row operations, and every lane of the row ends
// with the token's score.  The lanes that hold token t's K chunk also load
// its V chunk, so the softmax weight never leaves its lanes: the PV product
// accumulates per lane, and rows, then wavefronts, are merged once at the
// end.  Wavefronts take blocks round-robin and keep two blocks of K and V
// (16 KiB) in flight each, which with several workgroups per CU keeps enough
// bytes outstanding to run HBM-bound.
#include "attention_common.h"

namespace pkv {
namespace {

constexpr int kWaves = 4;
constexpr int kUnroll = 2;

template <typename QT, typename KT, int D, int G>
__global__ __launch_bounds__(256) void decode_wave_kernel(AttnArgs a) {
  constexpr int EB = KT::bytes;
  constexpr int E = 16 / EB;           // elements per 16-byte chunk
  constexpr int C = D / E;             // lanes per token row
  constexpr int TPL = 64 / C;          // tokens per wavefront load
  constexpr int NL = 16 / TPL;         // loads per 16-token tile
  constexpr int TILE = 16 * D * EB;    // bytes of one (block, head) tile
  static_assert(C >= 4 && C <= 64 && NL >= 1, "unsupported head_dim / dtype");
  constexpr bool kInt8 = (EB == 1);

  const int part = blockIdx.x % a.num_parts;
  const int row = blockIdx.x / a.num_parts;
  const int hgroups = a.hq / G;                       // workgroups per row along y
  const int hbase = blockIdx.y * G;                   // first query head
  const int kvh = hbase / (a.hq / a.hkv);
  (void)hgroups;

  int seq, ctx;
  row_context(a, row, seq, ctx);
  const int nparts = (ctx + a.part_tokens - 1) / a.part_tokens;
  if (part >= max(nparts, 1)) return;

  const int t0 = part * a.part_tokens;
  const int t1 = min(ctx, t0 + a.part_tokens);
  const int b0 = t0 >> 4;
  const int nb = ((t1 + 15) >> 4) - b0;

  const int wave = wave_uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int c = lane % C;
  const int u = lane / C;

  // q slice of every head of the group: elements [c*E, c*E + E).
  float qf[G][E];
  {
    const typename QT::raw* qp = static_cast<const typename QT::raw*>(a.q);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int64_t off = (static_cast<int64_t>(row) * a.hq + hbase + g) * D + c * E;
#pragma unroll
      for (int e = 0; e < E; ++e) qf[g][e] = load_elem<QT>(qp, off + e);
    }
  }

  float m[G], l[G], o[G][E];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = kNegInf;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) o[g][e] = 0.f;
  }

  const int32_t* trow = a.tables + static_cast<int64_t>(seq) * a.max_blocks;
  const uint8_t* kbase = static_cast<const uint8_t*>(a.kc) + lane * 16;
  const uint8_t* vbase = static_cast<const uint8_t*>(a.vc) + lane * 16;

  for (int base = wave; base < nb; base += kWaves * kUnroll) {
    u32x4 kr[kUnroll][NL], vr[kUnroll][NL];
    int phys[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      const int bi = base + k * kWaves;
      int p = -1;
      if (bi < nb) {
        p = trow[b0 + bi];
        if (p < 0 || p >= a.num_blocks) p = -1;   // outside the pool: treated as masked
      }
      phys[k] = p;
      if (p >= 0) {
        const int64_t toff = (static_cast<int64_t>(p) * a.hkv + kvh) * TILE;
#pragma unroll
        for (int j = 0; j < NL; ++j) {
          kr[k][j] = *reinterpret_cast<const u32x4*>(kbase + toff + j * 1024);
          vr[k][j] = *reinterpret_cast<const u32x4*>(vbase + toff + j * 1024);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      const int bi = base + k * kWaves;
      if (bi >= nb) break;
      const int p = phys[k];
      const int tpos = (b0 + bi) * 16;
      float kscale = 1.f, vscale = 1.f;
      if (kInt8 && p >= 0) {
        kscale = a.ks[static_cast<int64_t>(p) * a.hkv + kvh];
        vscale = a.vs[static_cast<int64_t>(p) * a.hkv + kvh];
      }
      // scores of this lane's NL tokens for every head
      float s[G][NL];
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        float kx[E];
        Unpack<KT>::run(kr[k][j], kx);
        const int tok = tpos + j * TPL + u;
        const bool valid = (p >= 0) && tok < t1;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float part_dot = 0.f;
#pragma unroll
          for (int e = 0; e < E; ++e) part_dot = fmaf(qf[g][e], kx[e], part_dot);
          const float dot = group_sum<C>(part_dot);
          s[g][j] = valid ? dot * kscale * a.scale_log2 : kNegInf;
        }
      }
      float pw[G][NL];
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
        l[g] = l[g] * alpha + psum;
        m[g] = mn;
#pragma unroll
        for (int e = 0; e < E; ++e) o[g][e] *= alpha;
      }
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        float vx[E];
        Unpack<KT>::run(vr[k][j], vx);
        const int tok = tpos + j * TPL + u;
        const bool valid = (p >= 0) && tok < t1;
#pragma unroll
        for (int e = 0; e < E; ++e) vx[e] = valid ? vx[e] * vscale : 0.f;
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int e = 0; e < E; ++e) o[g][e] = fmaf(pw[g][j], vx[e], o[g][e]);
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
      l[g] = l[g] * f1 + l2 * f2;
#pragma unroll
      for (int e = 0; e < E; ++e) o[g][e] = o[g][e] * f1 + __shfl_xor(o[g][e], off) * f2;
      m[g] = mn;
    }
  }

  // Merge the wavefronts through LDS.
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
  __syncthreads();

  finish_rows<kWaves, G, D>(a, sm_o, sm_m, sm_l, G, row, hbase, part, nparts);
}

// Merge of the partitions of one (row, head): log-sum-exp rescaling of each
// partition's (max, sum, unnormalised output) to the common max.
__global__ __launch_bounds__(128) void reduce_kernel(AttnArgs a, int D) {
  const int h = blockIdx.x;
  const int row = blockIdx.y;
  int seq, ctx;
  row_context(a, row, seq, ctx);
  const int nparts = (ctx + a.part_tokens - 1) / a.part_tokens;
  if (nparts <= 1) return;  // written by the main kernel
  const int64_t orow = static_cast<int64_t>(row) * a.hq + h;
  const float* ml = a.part_ml + orow * a.num_parts * 2;
  float M = kNegInf;
  for (int p = 0; p < nparts; ++p) M = fmaxf(M, ml[2 * p]);
  const float ms = (M == kNegInf) ? 0.f : M;
  float L = 0.f;
  for (int p = 0; p < nparts; ++p) L += ml[2 * p + 1] * fast_exp2(ml[2 * p] - ms);
  const float* po = a.part_o + orow * a.num_parts * D;
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float O = 0.f;
    for (int p = 0; p < nparts; ++p) O += po[static_cast<int64_t>(p) * D + d] * fast_exp2(ml[2 * p] - ms);
    store_out(a, orow * D + d, L > 0.f ? O / L : 0.f);
  }
}

template <typename QT, typename KT, int D>
pkv_status launch_d(const AttnArgs& a, int group, hipStream_t st) {
  // Heads per workgroup: the whole group when it is 1, 2, 4 or 8, otherwise
  // the largest of those dividing it (each workgroup then re-reads the KV).
  int gw = 1;
  for (int c : {8, 4, 2}) if (group % c == 0) { gw = c; break; }
  dim3 grid(a.num_parts * a.num_rows, a.hq / gw);
  switch (gw) {
    case 1: hipLaunchKernelGGL((decode_wave_kernel<QT, KT, D, 1>), grid, dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((decode_wave_kernel<QT, KT, D, 2>), grid, dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL((decode_wave_kernel<QT, KT, D, 4>), grid, dim3(256), 0, st, a); break;
    default: hipLaunchKernelGGL((decode_wave_kernel<QT, KT, D, 8>), grid, dim3(256), 0, st, a); break;
  }
  PKV_LAUNCH_CHECK("paged attention (wavefront)");
  return PKV_OK;
}

template <typename QT, typename KT>
pkv_status launch_qk(const AttnArgs& a, int D, int group, hipStream_t st) {
  if (D == 64) return launch_d<QT, KT, 64>(a, group, st);
  return launch_d<QT, KT, 128>(a, group, st);
}

}  // namespace

pkv_status launch_decode_wave(const AttnArgs& a, pkv_dtype q_dt, pkv_dtype kv_dt, int D,
                              int group, hipStream_t st) {
  if (kv_dt == PKV_I8) {
    if (q_dt == PKV_BF16) return launch_qk<BF16, I8>(a, D, group, st);
    if (q_dt == PKV_F16) return launch_qk<F16, I8>(a, D, group, st);
    return launch_qk<F32, I8>(a, D, group, st);
  }
  if (q_dt == PKV_BF16) return launch_qk<BF16, BF16>(a, D, group, st);
  if (q_dt == PKV_F16) return launch_qk<F16, F16>(a, D, group, st);
  return launch_qk<F32, F32>(a, D, group, st);
}

pkv_status launch_reduce(const AttnArgs& a, int D, hipStream_t st) {
  hipLaunchKernelGGL(reduce_kernel, dim3(a.hq, a.num_rows), dim3(128), 0, st, a, D);
  PKV_LAUNCH_CHECK("partition reduce");
  return PKV_OK;
}

}  // namespace pkv
