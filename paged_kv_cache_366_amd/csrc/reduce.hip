// Partition reduce: merges the split-K partial results of decode (and of
// prefill rows whose keys span several partitions) into the final rows.
// Each partition left its maximum m_p and sum l_p of the exponentiated
// scores (log2 domain) and its unnormalised output o_p; with M = max m_p,
// L = sum l_p 2^(m_p - M), the row is sum o_p 2^(m_p - M) / L, which is the
// softmax over all of the row's keys (cnnetsun.cn "别再让GPU内存拖后腿了…"
// §3.1: one softmax over the scores of every page).
#include "attention_common.h"

namespace pkv {
namespace {

// One wavefront per (row, head), kReduceWaves per workgroup, head fastest.
// A row and head need only a few partitions' states: a whole workgroup per
// item left most of a split prefill's 65,536 items waiting in line (93 us
// against 31 us this way), and even the decode reduce runs faster (long-
// context GQA 5.9 -> 4.8 us bf16, 6.9 -> 5.3 us int8).  Lane p holds
// partition p's (max, sum) pair (p, p + 64, ... up to kRegParts pairs;
// later partitions are re-read), the row maximum is a wave reduction, and
// each lane turns its pairs into rescale factors once.  L and lane l's
// output elements (l, l + 64) are then summed in the canonical order of
// merge_ml / merge_elem, the factor of partition p read from its lane: the
// same bits as the last-arriver merge inside the decode kernels.
constexpr int kReduceWaves = 4;
constexpr int kRegParts = 4;
constexpr int kPre = 16;   // partitions whose outputs a lane loads ahead

__device__ __forceinline__ float lane_of(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

__global__ __launch_bounds__(64 * kReduceWaves) void reduce_kernel(AttnArgs a, int D,
                                                                         int items) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * kReduceWaves + wave_uniform(threadIdx.x >> 6);
  if (item >= items) return;
  const int h = item % a.hq;
  const int row = item / a.hq;
  int seq, ctx;
  row_context(a, row, seq, ctx);
  const int nparts = (ctx + a.part_tokens - 1) / a.part_tokens;
  if (nparts <= 1) return;  // written by the main kernel
  const float* ml = a.part_ml + part_slot(a, row, h, 0) * 2;
  const int64_t st = 2 * static_cast<int64_t>(a.hq);   // floats between partitions' pairs
  const float* po = a.part_o + part_slot(a, row, h, 0) * D + lane;
  const int64_t so = static_cast<int64_t>(a.hq) * D;   // floats between partitions' rows
  const int E = D >> 6;                                 // elements per lane (1 or 2)
  // The outputs of the first kPre partitions do not depend on the factors:
  // their loads go out before the (max, sum) pass.
  float ov[kPre][2];
#pragma unroll
  for (int i = 0; i < kPre; ++i)
#pragma unroll
    for (int e = 0; e < 2; ++e) ov[i][e] = (i < nparts && e < E) ? po[i * so + 64 * e] : 0.f;
  float mreg[kRegParts], lreg[kRegParts];
  float mx = kNegInf;
#pragma unroll
  for (int k = 0; k < kRegParts; ++k) {
    const int p = 64 * k + lane;
    mreg[k] = p < nparts ? ml[p * st] : kNegInf;
    lreg[k] = p < nparts ? ml[p * st + 1] : 0.f;
    mx = fmaxf(mx, mreg[k]);
  }
  for (int p = 64 * kRegParts + lane; p < nparts; p += 64) mx = fmaxf(mx, ml[p * st]);
  mx = group_max<64>(mx);
  const float ms = (mx == kNegInf) ? 0.f : mx;
  float fac[kRegParts];
#pragma unroll
  for (int k = 0; k < kRegParts; ++k) fac[k] = fast_exp2(mreg[k] - ms);
  const int half = (nparts + 1) >> 1;
  float L = 0.f;
  float O[2][2] = {{0.f, 0.f}, {0.f, 0.f}};   // [half][element]
  auto add_v = [&](int p, float f, const float (&v)[2]) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      if (e < E) {
        if (p < half)
          O[0][e] = fmaf(v[e], f, O[0][e]);
        else
          O[1][e] = fmaf(v[e], f, O[1][e]);
      }
    }
  };
  auto add = [&](int p, float f) {
    float v[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) v[e] = e < E ? po[p * so + 64 * e] : 0.f;
    add_v(p, f, v);
  };
  static_assert(kPre <= 64, "the prefetched partitions' factors sit in the first register");
#pragma unroll
  for (int i = 0; i < kPre; ++i) {
    if (i < nparts) {
      const float f = lane_of(fac[0], i);
      L = fmaf(lane_of(lreg[0], i), f, L);
      add_v(i, f, ov[i]);
    }
  }
#pragma unroll
  for (int k = 0; k < kRegParts; ++k) {
    const int n = min(64, nparts - 64 * k);
#pragma unroll 8
    for (int j = k == 0 ? kPre : 0; j < n; ++j) {
      const float f = lane_of(fac[k], j);
      L = fmaf(lane_of(lreg[k], j), f, L);
      add(64 * k + j, f);
    }
  }
  for (int p = 64 * kRegParts; p < nparts; ++p) {
    const float f = fast_exp2(ml[p * st] - ms);
    L = fmaf(ml[p * st + 1], f, L);
    add(p, f);
  }
#pragma unroll
  for (int e = 0; e < 2; ++e)
    if (e < E)
      store_out(a, (static_cast<int64_t>(row) * a.hq + h) * D + lane + 64 * e,
                L > 0.f ? (O[0][e] + O[1][e]) / L : 0.f);
}

}  // namespace

pkv_status launch_reduce(const AttnArgs& a, int D, hipStream_t st) {
  const int64_t items = static_cast<int64_t>(a.hq) * a.num_rows;
  if (items > 0x7fffffff) return fail(PKV_ERR_UNSUPPORTED, "partition reduce: too many rows");
  hipLaunchKernelGGL(reduce_kernel, dim3((items + kReduceWaves - 1) / kReduceWaves),
                     dim3(64 * kReduceWaves), 0, st, a, D, static_cast<int>(items));
  PKV_LAUNCH_CHECK("partition reduce");
  return PKV_OK;
}

}  // namespace pkv
