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

// One workgroup of head_dim threads per (row, head), head fastest.  The
// partitions' (max, sum) pairs are loaded once, in parallel, into LDS, where
// each partition's rescale factor f_p = 2^(m_p - M) is computed once; then
// every thread forms L and its element's O in the canonical partition order
// (merge_ml, merge_elem: the same steps, hence the same bits, as the
// last-arriver merge inside the decode kernels), its loads of the
// partitions' outputs independent of each other.
constexpr int kMaxCachedParts = 1024;   // partitions whose (max, sum, factor) sit in LDS

__global__ __launch_bounds__(128) void reduce_kernel(AttnArgs a, int D) {
  const int h = blockIdx.x % a.hq;
  const int row = blockIdx.x / a.hq;
  int seq, ctx;
  row_context(a, row, seq, ctx);
  const int nparts = (ctx + a.part_tokens - 1) / a.part_tokens;
  if (nparts <= 1) return;  // written by the main kernel
  const int d = threadIdx.x;
  const float* ml = a.part_ml + part_slot(a, row, h, 0) * 2;
  const int64_t st = 2 * static_cast<int64_t>(a.hq);   // floats between partitions' pairs
  __shared__ float s_m[kMaxCachedParts], s_l[kMaxCachedParts];
  __shared__ float s_red[2];
  float mx = kNegInf;
  for (int p = d; p < nparts; p += D) {
    const float mp = ml[p * st], lp = ml[p * st + 1];
    if (p < kMaxCachedParts) {
      s_m[p] = mp;
      s_l[p] = lp;
    }
    mx = fmaxf(mx, mp);
  }
  mx = group_max<64>(mx);
  if ((d & 63) == 0) s_red[d >> 6] = mx;
  __syncthreads();
  float M = s_red[0];
  if (D > 64) M = fmaxf(M, s_red[1]);
  const float ms = (M == kNegInf) ? 0.f : M;
  for (int p = d; p < min(nparts, kMaxCachedParts); p += D) s_m[p] = fast_exp2(s_m[p] - ms);
  __syncthreads();
  // L and O in partition order; f_p from LDS (or recomputed past the cache)
  auto factor = [&](int p) {
    return p < kMaxCachedParts ? s_m[p] : fast_exp2(ml[p * st] - ms);
  };
  auto lsum = [&](int p) { return p < kMaxCachedParts ? s_l[p] : ml[p * st + 1]; };
  float L = 0.f;
  for (int p = 0; p < nparts; ++p) L = fmaf(lsum(p), factor(p), L);
  const float* po = a.part_o + part_slot(a, row, h, 0) * D + d;
  const int64_t so = static_cast<int64_t>(a.hq) * D;   // floats between partitions' rows
  float O = 0.f;
#pragma unroll 8
  for (int p = 0; p < nparts; ++p) O = fmaf(po[p * so], factor(p), O);
  store_out(a, (static_cast<int64_t>(row) * a.hq + h) * D + d, L > 0.f ? O / L : 0.f);
}

}  // namespace

pkv_status launch_reduce(const AttnArgs& a, int D, hipStream_t st) {
  hipLaunchKernelGGL(reduce_kernel, dim3(a.hq * a.num_rows), dim3(D), 0, st, a, D);
  PKV_LAUNCH_CHECK("partition reduce");
  return PKV_OK;
}

}  // namespace pkv
