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

// One workgroup of 2 x head_dim threads per (row, head), head fastest.  The
// partitions' (max, sum) pairs are loaded once, in parallel, into LDS, where
// each partition's rescale factor f_p = 2^(m_p - M) is computed once; then
// thread (g, d) sums element d over half g of the partitions in order, and
// the two halves are added: the canonical order of merge_ml / merge_elem,
// so the same bits as the last-arriver merge inside the decode kernels.
// Each thread's loads of the partitions' outputs do not depend on the
// factors: the first kChunk of them are issued before the (max, sum) pass,
// and each later chunk before the previous one is summed, so a workgroup
// waits on memory about twice rather than once per unrolled batch.
constexpr int kMaxCachedParts = 1024;   // partitions whose (max, sum, factor) sit in LDS
constexpr int kChunk = 16;              // partition outputs a thread holds in flight

__global__ __launch_bounds__(256) void reduce_kernel(AttnArgs a, int D) {
  const int h = blockIdx.x % a.hq;
  const int row = blockIdx.x / a.hq;
  int seq, ctx;
  row_context(a, row, seq, ctx);
  const int nparts = (ctx + a.part_tokens - 1) / a.part_tokens;
  if (nparts <= 1) return;  // written by the main kernel
  const int tid = threadIdx.x;
  const int nt = 2 * D;
  const int g = tid / D;
  const int d = tid % D;
  const float* ml = a.part_ml + part_slot(a, row, h, 0) * 2;
  const int64_t st = 2 * static_cast<int64_t>(a.hq);   // floats between partitions' pairs
  const int half = (nparts + 1) >> 1;
  const float* po = a.part_o + part_slot(a, row, h, 0) * D + d;
  const int64_t so = static_cast<int64_t>(a.hq) * D;   // floats between partitions' rows
  const int p_begin = g * half;
  const int p_end = min(nparts, (g + 1) * half);
  float ov[kChunk];
  auto load_chunk = [&](int p0) {
#pragma unroll
    for (int i = 0; i < kChunk; ++i) ov[i] = p0 + i < p_end ? po[(p0 + i) * so] : 0.f;
  };
  load_chunk(p_begin);
  __shared__ float s_m[kMaxCachedParts], s_l[kMaxCachedParts];
  __shared__ float s_red[4];
  __shared__ float s_o[128];
  float mx = kNegInf;
  for (int p = tid; p < nparts; p += nt) {
    const float mp = ml[p * st], lp = ml[p * st + 1];
    if (p < kMaxCachedParts) {
      s_m[p] = mp;
      s_l[p] = lp;
    }
    mx = fmaxf(mx, mp);
  }
  mx = group_max<64>(mx);
  if ((tid & 63) == 0) s_red[tid >> 6] = mx;
  __syncthreads();
  float M = s_red[0];
  for (int w = 1; w < nt / 64; ++w) M = fmaxf(M, s_red[w]);
  const float ms = (M == kNegInf) ? 0.f : M;
  for (int p = tid; p < min(nparts, kMaxCachedParts); p += nt) s_m[p] = fast_exp2(s_m[p] - ms);
  __syncthreads();
  // f_p from LDS (or recomputed past the cache)
  auto factor = [&](int p) {
    return p < kMaxCachedParts ? s_m[p] : fast_exp2(ml[p * st] - ms);
  };
  auto lsum = [&](int p) { return p < kMaxCachedParts ? s_l[p] : ml[p * st + 1]; };
  // The sum L first (LDS only), while the output loads are in flight.
  float L = 0.f;
  if (g == 0) {
#pragma unroll 8
    for (int p = 0; p < nparts; ++p) L = fmaf(lsum(p), factor(p), L);
  }
  float O = 0.f;
  for (int p0 = p_begin; p0 < p_end; p0 += kChunk) {
    float cur[kChunk];
#pragma unroll
    for (int i = 0; i < kChunk; ++i) cur[i] = ov[i];
    if (p0 + kChunk < p_end) load_chunk(p0 + kChunk);
#pragma unroll
    for (int i = 0; i < kChunk; ++i)
      if (p0 + i < p_end) O = fmaf(cur[i], factor(p0 + i), O);
  }
  if (g == 1) s_o[d] = O;
  __syncthreads();
  if (g == 0) {
    store_out(a, (static_cast<int64_t>(row) * a.hq + h) * D + d,
              L > 0.f ? (O + s_o[d]) / L : 0.f);
  }
}

}  // namespace

pkv_status launch_reduce(const AttnArgs& a, int D, hipStream_t st) {
  hipLaunchKernelGGL(reduce_kernel, dim3(a.hq * a.num_rows), dim3(2 * D), 0, st, a, D);
  PKV_LAUNCH_CHECK("partition reduce");
  return PKV_OK;
}

}  // namespace pkv
