// Launch shape of split attention launches (host): how long the key
// partitions are.  Splitting a context into partitions whose partial
// softmax states merge into one ([cnnetsun] §3.1: one softmax over the
// scores of every page) is exact up to rounding for any length; the length
// only decides how many workgroups the launch has.
#pragma once
#include <cstdint>

namespace pkv {

// The shortest partition (a multiple of 16 tokens, at least min_tokens)
// whose workgroups fit in the whole rounds of `resident` workgroups that
// the launch needs without a split; 0 when no split fits (or there is
// nothing to split).  Sequence s, with lens[s] keys, contributes weights[s]
// workgroups per partition of its keys (`uniform` for every sequence when
// weights is null); partitions past a context's end hold no slot.  Sizes
// must be checked by the caller (lens >= 0, weights >= 0, resident > 0).
int32_t partition_for_rounds(const int32_t* lens, const int64_t* weights, int64_t uniform,
                             int32_t num_seqs, int64_t resident, int32_t min_tokens);

}  // namespace pkv
