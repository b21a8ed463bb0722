// Launch shape of split attention launches (host C++, no device calls): the
// partition search and its C entry point pkv_decode_partition_for_capacity.
// The device-aware calls (pkv_decode_partition_tokens,
// pkv_prefill_partition_tokens) read the resident workgroups of the kernel
// a launch would pick and call the search from attention_api.hip.
#include "partition.h"

#include <algorithm>

#include "status.h"

namespace pkv {

int32_t partition_for_rounds(const int32_t* lens, const int64_t* weights, int64_t uniform,
                             int32_t num_seqs, int64_t resident, int32_t min_tokens) {
  auto weight = [&](int32_t s) { return weights ? weights[s] : uniform; };
  int32_t max_len = 0;
  for (int32_t s = 0; s < num_seqs; ++s)
    if (weight(s) > 0) max_len = std::max(max_len, lens[s]);
  const int64_t cap = (static_cast<int64_t>(max_len) + 15) / 16 * 16;   // one partition per context
  const int64_t lo = std::max<int64_t>(16, (static_cast<int64_t>(min_tokens) + 15) / 16 * 16);
  if (max_len == 0 || lo >= cap) return 0;
  // workgroups holding keys at partitions of p tokens; only falls as p grows,
  // so a bisection over multiples of 16 finds the least that fits
  auto wgs = [&](int64_t p) {
    int64_t n = 0;
    for (int32_t s = 0; s < num_seqs; ++s) n += (lens[s] + p - 1) / p * weight(s);
    return n;
  };
  const int64_t rounds = (wgs(cap) + resident - 1) / resident;
  const int64_t target = rounds * resident;
  int64_t a = lo / 16, b = cap / 16;   // wgs(16 b) <= target
  while (a < b) {
    const int64_t m = (a + b) / 2;
    if (wgs(16 * m) <= target) b = m; else a = m + 1;
  }
  return 16 * a < cap ? static_cast<int32_t>(16 * a) : 0;
}

}  // namespace pkv

extern "C" {

pkv_status pkv_decode_partition_for_capacity(const int32_t* context_lens, int32_t num_seqs,
                                             int32_t workgroups_per_partition,
                                             int64_t resident_workgroups, int32_t min_tokens,
                                             int32_t* partition_tokens) {
  const char* who = "decode_partition_for_capacity";
  if (!partition_tokens || (num_seqs > 0 && !context_lens))
    return pkv::fail(PKV_ERR_INVALID, "%s: NULL pointer", who);
  if (num_seqs < 0 || workgroups_per_partition <= 0 || resident_workgroups <= 0 || min_tokens < 0)
    return pkv::fail(PKV_ERR_INVALID, "%s: bad sizes (S=%d per-partition %d resident %lld min %d)",
                     who, num_seqs, workgroups_per_partition,
                     static_cast<long long>(resident_workgroups), min_tokens);
  for (int32_t s = 0; s < num_seqs; ++s)
    if (context_lens[s] < 0)
      return pkv::fail(PKV_ERR_INVALID, "%s: context_lens[%d] = %d", who, s, context_lens[s]);
  *partition_tokens = pkv::partition_for_rounds(context_lens, nullptr, workgroups_per_partition,
                                                num_seqs, resident_workgroups, min_tokens);
  return PKV_OK;
}

}  // extern "C"
