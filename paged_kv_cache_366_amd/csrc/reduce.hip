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

// Merge of the partitions of one (row, head): log-sum-exp rescaling of each
// partition's (max, sum, unnormalised output) to the common max.  One
// workgroup per (row, head), head fastest.  (One wavefront per (row, head),
// summing the partitions in a single lane chain, measured slower: 7.4 vs
// 7.0 µs at the 7B shape, 30 vs 15 µs with 64 partitions.)  The partitions' (max, sum)
// pairs are read by all threads at once and reduced across the workgroup;
// the rescale weights go to LDS; then groups of head_dim threads each sum a
// strided share of the partitions with independent, unrolled loads, and the
// groups are added in a fixed order (deterministic for a fixed partition
// size).
constexpr int kReduceThreads = 256;
constexpr int kReduceWeights = 1024;   // partitions whose weights are cached in LDS

__device__ __forceinline__ float wave_max(float v) { return group_max<64>(v); }
__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }

__global__ __launch_bounds__(kReduceThreads) void reduce_kernel(AttnArgs a, int D) {
  const int h = blockIdx.x % a.hq;
  const int row = blockIdx.x / a.hq;
  int seq, ctx;
  row_context(a, row, seq, ctx);
  const int nparts = (ctx + a.part_tokens - 1) / a.part_tokens;
  if (nparts <= 1) return;  // written by the main kernel
  const int64_t orow = static_cast<int64_t>(row) * a.hq + h;
  // partition p of this (row, head) is slot part_slot(a, row, h, p): the
  // slots of consecutive partitions are hq apart
  const float* ml = a.part_ml + part_slot(a, row, h, 0) * 2;
  const float* po = a.part_o + part_slot(a, row, h, 0) * D;
  const int64_t mls = 2 * static_cast<int64_t>(a.hq);   // floats between partitions' pairs
  const int64_t pos = static_cast<int64_t>(a.hq) * D;   // floats between partitions' rows
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  __shared__ float sw[kReduceWeights];
  __shared__ float red[2][kReduceThreads / 64];
  __shared__ float sacc[kReduceThreads];

  float mx = kNegInf;
  for (int p = tid; p < nparts; p += kReduceThreads) mx = fmaxf(mx, ml[p * mls]);
  mx = wave_max(mx);
  if (lane == 0) red[0][wave] = mx;
  __syncthreads();
  float M = red[0][0];
#pragma unroll
  for (int w = 1; w < kReduceThreads / 64; ++w) M = fmaxf(M, red[0][w]);
  const float ms = (M == kNegInf) ? 0.f : M;
  float ls = 0.f;
  for (int p = tid; p < nparts; p += kReduceThreads) {
    const float w = fast_exp2(ml[p * mls] - ms);
    if (p < kReduceWeights) sw[p] = w;
    ls += ml[p * mls + 1] * w;
  }
  ls = wave_sum(ls);
  if (lane == 0) red[1][wave] = ls;
  __syncthreads();
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < kReduceThreads / 64; ++w) L += red[1][w];

  const int groups = kReduceThreads / D;   // 2 for head_dim 128, 4 for 64
  const int g = tid / D;
  const int d = tid % D;
  float O = 0.f;
#pragma unroll 4
  for (int p = g; p < nparts; p += groups) {
    const float w = p < kReduceWeights ? sw[p] : fast_exp2(ml[p * mls] - ms);
    O += po[p * pos + d] * w;
  }
  sacc[tid] = O;
  __syncthreads();
  if (g == 0) {
    for (int k = 1; k < groups; ++k) O += sacc[k * D + d];
    store_out(a, orow * D + d, L > 0.f ? O / L : 0.f);
  }
}

}  // namespace

pkv_status launch_reduce(const AttnArgs& a, int D, hipStream_t st) {
  hipLaunchKernelGGL(reduce_kernel, dim3(a.hq * a.num_rows), dim3(kReduceThreads), 0, st, a, D);
  PKV_LAUNCH_CHECK("partition reduce");
  return PKV_OK;
}

}  // namespace pkv
