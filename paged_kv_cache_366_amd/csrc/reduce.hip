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

// One workgroup of head_dim threads per (row, head), head fastest; thread d
// merges element d in the canonical partition order (merge_ml, merge_elem),
// the same steps as the last-arriver merge inside the decode kernels.  The
// partitions' (max, sum) pairs are read by every thread (cache hits after
// the first), so no thread waits on another.
__global__ __launch_bounds__(128) void reduce_kernel(AttnArgs a, int D) {
  const int h = blockIdx.x % a.hq;
  const int row = blockIdx.x / a.hq;
  int seq, ctx;
  row_context(a, row, seq, ctx);
  const int nparts = (ctx + a.part_tokens - 1) / a.part_tokens;
  if (nparts <= 1) return;  // written by the main kernel
  const int d = threadIdx.x;
  const PartMerge pm = merge_ml(a, row, h, nparts);
  store_out(a, (static_cast<int64_t>(row) * a.hq + h) * D + d,
            merge_elem(a, row, h, nparts, pm, d, D));
}

}  // namespace

pkv_status launch_reduce(const AttnArgs& a, int D, hipStream_t st) {
  hipLaunchKernelGGL(reduce_kernel, dim3(a.hq * a.num_rows), dim3(D), 0, st, a, D);
  PKV_LAUNCH_CHECK("partition reduce");
  return PKV_OK;
}

}  // namespace pkv
