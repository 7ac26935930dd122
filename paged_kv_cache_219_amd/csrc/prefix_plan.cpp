// Shared-prefix groups of a decode batch, derived from its block tables.
//
// Page "vLLM PagedAttention chuyên sâu: Phân mảnh bộ nhớ KV Cache, Prefill
// theo khối & Prefix Caching" (locionic.com), section "Cơ chế APC", item 2:
// a request whose prefix matches cached blocks links those physical blocks
// into its own table; the skymod.tech overview on vLLM: the samples of one
// prompt share the prompt's blocks.  Either way, sequences with a common
// prefix hold the same physical block ids at the start of their tables --
// this planner finds such runs of neighbouring sequences so that the decode
// kernel can read the shared pages once for all of them.
//
// Greedy, in batch order: a group starts at its first sequence (the leader)
// with the leader's whole blocks as the candidate prefix; the next sequence
// joins while the group has fewer than max_members members and the prefix
// it would leave (the leading block ids it has in common with the leader,
// within both contexts' whole blocks) is at least min_prefix tokens and keeps
// at least as many page reads saved: P' * n >= P * (n - 1) for a group of n
// members whose prefix shrinks from P to P'.  Groups of one are dropped.

#include <algorithm>
#include <cstdint>

#include "../../include/pa.h"

extern "C" int pa_prefix_plan(const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* context_lens, int32_t num_seqs, int32_t block_size,
                              int32_t max_members, int32_t min_prefix, int32_t* groups,
                              int32_t* seq_prefix_lens, int32_t* num_groups,
                              int32_t* max_prefix_len) {
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || block_size <= 0 || max_members < 1 ||
      max_members > PA_PREFIX_MAX_MEMBERS || min_prefix < 0 || !num_groups || !max_prefix_len)
    return PA_ERR_INVALID_ARG;
  if (num_seqs > 0 && (!block_tables || !context_lens || !groups || !seq_prefix_lens))
    return PA_ERR_INVALID_ARG;
  const int64_t cap = static_cast<int64_t>(max_blocks_per_seq) * block_size;
  for (int32_t s = 0; s < num_seqs; ++s)
    if (context_lens[s] < 0 || context_lens[s] > cap) return PA_ERR_INVALID_ARG;

  const int32_t floor_min = std::max(min_prefix, block_size);
  auto row = [&](int32_t s) { return block_tables + static_cast<int64_t>(s) * max_blocks_per_seq; };
  int32_t ng = 0, maxp = 0;
  int32_t s = 0;
  while (s < num_seqs) {
    const int32_t* lead = row(s);
    int32_t P = context_lens[s] / block_size * block_size;  // candidate prefix, tokens
    int32_t n = 1;
    while (s + n < num_seqs && n < max_members) {
      const int32_t t = s + n;
      const int32_t limit = std::min(P, context_lens[t] / block_size * block_size) / block_size;
      const int32_t* other = row(t);
      int32_t common = 0;
      while (common < limit && other[common] == lead[common]) ++common;
      const int32_t P2 = common * block_size;
      if (P2 < floor_min || static_cast<int64_t>(P2) * n < static_cast<int64_t>(P) * (n - 1))
        break;
      P = P2;
      ++n;
    }
    if (n >= 2 && P >= floor_min) {
      groups[3 * ng] = s;
      groups[3 * ng + 1] = n;
      groups[3 * ng + 2] = P;
      ++ng;
      maxp = std::max(maxp, P);
      for (int32_t i = 0; i < n; ++i) seq_prefix_lens[s + i] = P;
      s += n;
    } else {
      seq_prefix_lens[s] = 0;
      s += 1;
    }
  }
  *num_groups = ng;
  *max_prefix_len = maxp;
  return PA_OK;
}
