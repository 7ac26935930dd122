// Decode attention over a paged KV cache (gfx950): the kernels and the
// pa_decode / pa_decode_shared_prefix entry points.  The one-wave item body is
// in decode_core.h.

#include <mutex>

#include "decode_core.h"
#include "decode_mfma.h"

namespace {

// One wave (one 64-thread workgroup) per item.
template <typename T, int D, int G, bool PVB, int BS, bool NT>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void decode_kernel(
    T* __restrict__ out, Partials ws, const T* __restrict__ q, const T* __restrict__ kc,
    const T* __restrict__ vc, const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ context_lens, int32_t num_seqs, int32_t num_heads,
    int32_t num_kv_heads, int32_t num_parts, int32_t partition, float scale_log2,
    RangeSplit rs) {
  __shared__ __attribute__((aligned(16))) weight_t<PVB> p_lds[G * kTile];
  decode_item<T, D, G, PVB, BS, NT>(blockIdx.x, p_lds, out, ws, q, kc, vc, block_tables,
                                max_blocks, context_lens, num_seqs, num_heads, num_kv_heads,
                                num_parts, partition, scale_log2, rs);
}

// Shared-prefix pass (bf16, head_dim 128).  Prefix group i is `count`
// consecutive sequences starting at `first` whose block tables hold the same
// physical blocks for the first `prefix` tokens (a multiple of the block
// size) -- the samples of one prompt after a fork, or requests whose prompts
// matched the same cached blocks.  Those tokens' K/V pages are read once, from
// the first member's table, for the queries of every member, on the matrix
// cores (decode_mfma.h): one wave per (partition of the prefix, group, chunk
// of 32 queries, kv head), kv head fastest, the queries of a kv head ordered
// (member, head within the kv head's group) as the columns.  Each query's
// partial result goes to partial slot `part` of its (sequence, head) row, or
// straight to the output when the prefix is the sequence's whole context and
// fits one partition.
constexpr int kPrefixMembers = PA_PREFIX_MAX_MEMBERS;

template <bool NT>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void decode_prefix_mfma_kernel(
    uint16_t* __restrict__ out, Partials ws, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ groups,
    int32_t num_groups, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
    int32_t num_parts, int32_t prefix_parts, int32_t partition, float scale_log2) {
  constexpr int Q = 32;
  const int gq_heads = num_heads / num_kv_heads;
  const int nchunks = (kPrefixMembers * gq_heads + Q - 1) / Q;
  uint32_t li = blockIdx.x;
  const int g = static_cast<int>(li % static_cast<uint32_t>(num_kv_heads));
  li /= static_cast<uint32_t>(num_kv_heads);
  const int chunk = static_cast<int>(li % static_cast<uint32_t>(nchunks));
  li /= static_cast<uint32_t>(nchunks);
  const int gi = static_cast<int>(li % static_cast<uint32_t>(num_groups));
  const int part = static_cast<int>(li / static_cast<uint32_t>(num_groups));
  if (part >= prefix_parts) return;

  const int first = groups[3 * gi];
  const int count = min(min(groups[3 * gi + 1], kPrefixMembers), num_seqs - first);
  if (first < 0 || count <= 0) return;
  const int P = split_begin(groups[3 * gi + 2], min(context_lens[first], max_blocks * kBS));
  const int part_start = part * partition;
  const int nq = count * gq_heads;
  const int q0 = chunk * Q;
  if (part_start >= P || q0 >= nq) return;
  const int n_pre = (P + partition - 1) / partition;
  // (sequence, head) row of the chunk's local query i
  auto row_of = [&](int i) -> int64_t {
    const int gq = min(q0 + i, nq - 1);
    const int s = first + gq / gq_heads;
    return static_cast<int64_t>(s) * num_heads + g * gq_heads + gq % gq_heads;
  };
  const auto qrow = [&](int i) { return q + row_of(i) * kD; };
  const auto dest = [&](int i, int64_t& out_off, int64_t& part_row) {
    const int64_t row = row_of(i);
    const int s = first + (q0 + i) / gq_heads;
    const bool direct = n_pre == 1 && context_lens[s] <= P;
    out_off = direct ? row * kD : -1;
    part_row = direct ? -1 : row * num_parts + part;
  };
  const int32_t* bt_row = block_tables + static_cast<int64_t>(first) * max_blocks;
  const int end = min(part_start + partition, P);
  const int nq_chunk = min(Q, nq - q0);
  // up to 16 queries (8 samples of a multi-head prompt, or 4 with 4 heads per
  // kv head): half the columns (201 vs 204 us on 32 prompts x 8 samples)
  if (nq_chunk <= 16)
    mfma16_decode_range<NT, kGqaKeySteps, kGqaValueSteps>(out, ws, kc, vc, bt_row, num_kv_heads,
                                                          g, part_start, end, scale_log2,
                                                          nq_chunk, qrow, dest);
  else
    mfma_decode_range<NT>(out, ws, kc, vc, bt_row, num_kv_heads, g, part_start, end, scale_log2,
                          nq_chunk, qrow, dest);
}


// Prefix groups found on the device (PA_DECODE_FIND_SHARED): one wave per
// aligned run of kPrefixMembers sequences [first, first + kPrefixMembers).
// The run's first sequence leads; the next ones join in order while the
// leading block ids they share with the leader, within both contexts' whole
// blocks, make a prefix of at least min_prefix tokens and the page reads
// saved, prefix * (members - 1), do not fall: the host planner's rule
// (prefix_plan.cpp) within the run.  Writes the run's group (first, members,
// prefix tokens), or first = -1 when it forms none, and the prefix length of
// each of its sequences (0 outside the group).
__global__ __launch_bounds__(64) void find_groups_kernel(
    const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ context_lens, int32_t num_seqs, int32_t min_prefix,
    int32_t* __restrict__ groups, int32_t* __restrict__ seq_prefix_lens) {
  static_assert(kPrefixMembers == 8, "8 lanes per member, 8 members per wave");
  const int gi = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int first = gi * kPrefixMembers;
  const int n = min(kPrefixMembers, num_seqs - first);
  // whole blocks of each member's context (lane m holds member m's; a length
  // above the table row, a broken precondition, is cut to the row)
  const int my_whole = lane < n ? min(max(context_lens[first + lane], 0), max_blocks * kBS) / kBS : 0;
  const int whole0 = __builtin_amdgcn_readfirstlane(my_whole);
  // Leading block ids each member m >= 1 shares with the leader, all members
  // at once: lane 8 m + j compares positions j, j + 8, ... of member m's row
  // with the leader's, eight positions per pass (one round of loads).
  const int m = lane >> 3, j = lane & 7;
  const int whole_m = __shfl(my_whole, m, 64);  // every lane takes part in the exchange
  const int limit = m >= 1 && m < n ? min(whole0, whole_m) : 0;
  const int32_t* lead = block_tables + static_cast<int64_t>(first) * max_blocks;
  const int32_t* other = block_tables + static_cast<int64_t>(first + (m < n ? m : 0)) * max_blocks;
  int mine = limit;  // this lane's first mismatch (or the limit)
  for (int base = 0; __any(base < limit && mine == limit); base += 64) {
    int a[8], b[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int pos = base + j + 8 * k;
      a[k] = pos < limit ? lead[pos] : 0;
      b[k] = pos < limit ? other[pos] : 0;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int pos = base + j + 8 * k;
      if (mine == limit && pos < limit && a[k] != b[k]) mine = pos;
    }
    // the member's eight lanes have now compared every position below
    // base + 64: a mismatch among them is the member's first one
    int lo = mine;
    lo = min(lo, __shfl_xor(lo, 1, 64));
    lo = min(lo, __shfl_xor(lo, 2, 64));
    lo = min(lo, __shfl_xor(lo, 4, 64));
    if (lo < base + 64) mine = lo;  // every position below lo was compared equal
  }
  int lcp = mine;  // member m's common prefix with the leader, in blocks
  lcp = min(lcp, __shfl_xor(lcp, 1, 64));
  lcp = min(lcp, __shfl_xor(lcp, 2, 64));
  lcp = min(lcp, __shfl_xor(lcp, 4, 64));
  // the host planner's greedy rule, on the members' common prefixes in order
  const int floor_min = max(min_prefix, kBS);
  int P = whole0;  // candidate prefix, in blocks
  int count = 1;
  for (int mm = 1; mm < n; ++mm) {
    const int common = min(__shfl(lcp, 8 * mm, 64), P);
    if (common * kBS < floor_min ||
        static_cast<int64_t>(common) * count < static_cast<int64_t>(P) * (count - 1))
      break;
    P = common;
    ++count;
  }
  const bool grouped = count >= 2;  // a member joined: P * kBS >= floor_min
  if (lane == 0) {
    groups[3 * gi] = grouped ? first : -1;
    groups[3 * gi + 1] = grouped ? count : 0;
    groups[3 * gi + 2] = grouped ? P * kBS : 0;
  }
  if (lane < n) seq_prefix_lens[first + lane] = grouped && lane < count ? P * kBS : 0;
}

// Where a decode call's partitions go: `slots` partial slots per (sequence,
// head) row; the first pass covers tokens [starts[s], L) (from 0 when starts
// is null) in up to `parts` partitions written from slot part_base on.
struct Split {
  int32_t slots;
  int32_t parts;
  RangeSplit rs;
};

template <typename T, int D, int G, bool PVB, int BS, bool NT>
int launch_decode(void* out, const void* q, const void* kc, const void* vc, const int32_t* bt,
                  int32_t max_blocks, const int32_t* lens, int32_t B, int32_t H, int32_t KVH,
                  Split sp, int32_t partition, float scale_log2, void* ws, hipStream_t st) {
  const Partials p = carve(ws, B, H, D, sp.slots);
  const int64_t grid = static_cast<int64_t>(sp.parts) * KVH * B;
  // 4 or 8 query heads per kv head: on the matrix cores (decode_mfma.h).  With
  // 1 or 2 the one-wave body is as fast (both stream at the same rate) and
  // faster where sequences share pages through L2.
  if constexpr (BS == kBS && sizeof(T) == 2 && D == 128 && (G == 4 || G == 8)) {
    hipLaunchKernelGGL(decode_mfma_kernel<NT>, dim3(static_cast<uint32_t>(grid)), dim3(64), 0, st,
                       static_cast<uint16_t*>(out), p, static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(kc), static_cast<const uint16_t*>(vc), bt,
                       max_blocks, lens, B, H, KVH, sp.slots, partition, scale_log2, sp.rs);
  } else {
    hipLaunchKernelGGL((decode_kernel<T, D, G, PVB, BS, NT>), dim3(static_cast<uint32_t>(grid)), dim3(64),
                       0, st, static_cast<T*>(out), p, static_cast<const T*>(q),
                       static_cast<const T*>(kc), static_cast<const T*>(vc), bt, max_blocks, lens,
                       B, H, KVH, sp.slots, partition, scale_log2, sp.rs);
  }
  if (sp.slots > 1)
    hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3(static_cast<uint32_t>(B) * H), dim3(64),
                       0, st, static_cast<T*>(out), p, lens, H, sp.slots, partition, sp.rs,
                       max_blocks * BS);
  return pa_launch_status();
}

template <typename T, int D, int BS = kBS>
int dispatch_group(int G, void* out, const void* q, const void* kc, const void* vc,
                   const int32_t* bt, int32_t mb, const int32_t* lens, int32_t B, int32_t H,
                   int32_t KVH, Split sp, int32_t partition, float sl2, void* ws,
                   hipStream_t st, bool nt) {
  constexpr bool kBf = sizeof(T) == 2;
#define PA_LAUNCH(GG, PV)                                                                        \
  (nt ? launch_decode<T, D, GG, PV, BS, true>(out, q, kc, vc, bt, mb, lens, B, H, KVH, sp,        \
                                               partition, sl2, ws, st)                           \
      : launch_decode<T, D, GG, PV, BS, false>(out, q, kc, vc, bt, mb, lens, B, H, KVH, sp,       \
                                                partition, sl2, ws, st))
  switch (G) {
    case 1: return PA_LAUNCH(1, false);
    case 2: return PA_LAUNCH(2, false);
    case 4: return PA_LAUNCH(4, kBf);
    case 8: return PA_LAUNCH(8, kBf);
    default: return PA_ERR_UNSUPPORTED;
  }
#undef PA_LAUNCH
}

// dtype and head_dim dispatch for one block size
template <int BS>
int dispatch_block(int32_t dtype, int32_t head_dim, int G, void* out, const void* q,
                   const void* kc, const void* vc, const int32_t* bt, int32_t mb,
                   const int32_t* lens, int32_t B, int32_t H, int32_t KVH, Split sp,
                   int32_t partition, float sl2, void* ws, hipStream_t st, bool nt) {
  if (dtype == PA_BF16) {
    if (head_dim == 128)
      return dispatch_group<uint16_t, 128, BS>(G, out, q, kc, vc, bt, mb, lens, B, H, KVH, sp, partition, sl2, ws, st, nt);
    return dispatch_group<uint16_t, 64, BS>(G, out, q, kc, vc, bt, mb, lens, B, H, KVH, sp, partition, sl2, ws, st, nt);
  }
  if (head_dim == 128)
    return dispatch_group<float, 128, BS>(G, out, q, kc, vc, bt, mb, lens, B, H, KVH, sp, partition, sl2, ws, st, nt);
  return dispatch_group<float, 64, BS>(G, out, q, kc, vc, bt, mb, lens, B, H, KVH, sp, partition, sl2, ws, st, nt);
}


}  // namespace

namespace {

// The prefix pass works in partitions twice as long as the rest's: its
// workgroups then keep their copy pipeline full for longer (measured 4%
// faster on 8-sample groups with a 1024-token prefix than equal partitions;
// four times as long gained nothing more).
constexpr int kPrefixPartMult = 2;

// Partition of a shared prefix, in tokens, for the rest's partition `part`.
int32_t prefix_partition(int32_t part) {
  return static_cast<int32_t>(
      std::min<int64_t>(static_cast<int64_t>(part) * kPrefixPartMult, 0x40000000));
}

// Partial slots of a shared-prefix call: the prefix's partitions, then the
// rest's.
void shared_slots(int32_t max_context_len, int32_t max_prefix_len, int32_t part, int64_t& pre,
                  int64_t& rest) {
  pre = max_prefix_len > 0 ? parts_for(max_prefix_len, prefix_partition(part)) : 0;
  rest = parts_for(max_context_len, part);
}

int32_t unsplit_partition(int32_t partition, int32_t max_context_len) {
  if (partition != 0) return partition;
  return static_cast<int32_t>(((std::max(max_context_len, 1) + kTile - 1) / kTile) * kTile);
}


// The launches of a call with prefix groups (on the device, at `groups`,
// num_groups of them): the prefix pass over the groups' shared pages, then
// pass 1 over each sequence's rest (from seq_prefix_lens[s]) and the merge.
// pre and rest are the partial slots of the prefix and of the rest.
int shared_launch(void* out, const void* q, const void* kc, const void* vc, const int32_t* bt,
                  int32_t mb, const int32_t* lens, int32_t B, int32_t H, int32_t KVH,
                  int32_t part, int64_t pre, int64_t rest, const int32_t* groups,
                  int32_t num_groups, const int32_t* seq_prefix_lens, void* ws, float sl2,
                  hipStream_t st, bool nt) {
  const int G = H / KVH;
  const int64_t slots = pre + rest;
  const int64_t nchunks =  // 32 queries each
      (static_cast<int64_t>(kPrefixMembers) * G + 31) / 32;
  const bool split = num_groups > 0 && pre > 0;
  if (split) {
    const Partials p = carve(ws, B, H, 128, slots);
    const int64_t grid = pre * num_groups * nchunks * KVH;
    auto kernel = nt ? decode_prefix_mfma_kernel<true> : decode_prefix_mfma_kernel<false>;
    hipLaunchKernelGGL(kernel, dim3(static_cast<uint32_t>(grid)), dim3(64), 0, st,
                       static_cast<uint16_t*>(out), p, static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(kc), static_cast<const uint16_t*>(vc), bt,
                       mb, lens, groups, num_groups, B, H, KVH, static_cast<int32_t>(slots),
                       static_cast<int32_t>(pre), prefix_partition(part), sl2);
    const int rc = pa_launch_status();
    if (rc != PA_OK) return rc;
  }
  const Split sp{static_cast<int32_t>(slots), static_cast<int32_t>(rest),
                 {split ? seq_prefix_lens : nullptr, static_cast<int32_t>(pre),
                  prefix_partition(part)}};
  return dispatch_group<uint16_t, 128>(G, out, q, kc, vc, bt, mb, lens, B, H, KVH, sp, part,
                                       sl2, ws, st, nt);
}

// Workspace of a call that finds its prefix groups (PA_DECODE_FIND_SHARED):
// the partials of a prefix of up to max_context_len tokens and of the rest,
// then the groups found (3 int32 per run of kPrefixMembers sequences), then
// each sequence's prefix length.
struct FoundLayout {
  int32_t part, runs;
  int64_t pre, rest;
  size_t groups_off, lens_off, total;
};
FoundLayout found_layout(int32_t B, int32_t H, int32_t D, int32_t max_context_len,
                         int32_t partition) {
  FoundLayout f;
  f.part = unsplit_partition(partition, max_context_len);
  shared_slots(max_context_len, max_context_len / kBS * kBS, f.part, f.pre, f.rest);
  f.runs = (std::max(B, 0) + kPrefixMembers - 1) / kPrefixMembers;
  f.groups_off = align_up(ws_bytes(B, H, D, f.pre + f.rest));
  f.lens_off = f.groups_off + align_up(static_cast<size_t>(f.runs) * 3 * sizeof(int32_t));
  f.total = f.lens_off + static_cast<size_t>(std::max(B, 0)) * sizeof(int32_t);
  return f;
}

}  // namespace

extern "C" size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                            int32_t max_context_len, int32_t partition) {
  if (num_seqs <= 0 || num_heads <= 0 || head_dim <= 0) return 0;
  return ws_bytes(num_seqs, num_heads, head_dim, parts_for(max_context_len, partition));
}

extern "C" size_t pa_decode_workspace_bytes_flags(int32_t num_seqs, int32_t num_heads,
                                                  int32_t head_dim, int32_t max_context_len,
                                                  int32_t partition, int32_t flags) {
  if (!(flags & PA_DECODE_FIND_SHARED))
    return pa_decode_workspace_bytes(num_seqs, num_heads, head_dim, max_context_len, partition);
  if (num_seqs <= 0 || num_heads <= 0 || head_dim <= 0 || partition < 0 || max_context_len < 0)
    return 0;
  return found_layout(num_seqs, num_heads, head_dim, max_context_len, partition).total;
}

// pa_decode's checks and launches, on the workspace given.
static int decode_call(void* out, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                       const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                       int32_t num_blocks, float scale, int32_t partition,
                       int32_t max_context_len, void* workspace, size_t workspace_bytes,
                       int32_t dtype, int32_t flags, void* stream) {
  if (dtype != PA_F32 && dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  if (flags & ~(PA_DECODE_STREAM_KV | PA_DECODE_FIND_SHARED)) return PA_ERR_INVALID_ARG;
  const bool find = (flags & PA_DECODE_FIND_SHARED) != 0;
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0 ||
      num_blocks <= 0 || partition < 0 || max_context_len < 0)
    return PA_ERR_INVALID_ARG;
  if (num_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if ((block_size != 8 && block_size != 16 && block_size != 32 && block_size != 64) ||
      (head_dim != 64 && head_dim != 128))
    return PA_ERR_UNSUPPORTED;
  if (find && (dtype != PA_BF16 || head_dim != 128 || block_size != kBS))
    return PA_ERR_UNSUPPORTED;  // the prefix pass runs on the bf16 matrix-core body
  if (partition % kTile != 0) return PA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * block_size)
    return PA_ERR_INVALID_ARG;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return PA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_cache) |
       reinterpret_cast<uintptr_t>(v_cache)) & 15)
    return PA_ERR_INVALID_ARG;
  // One pass when unpartitioned: a single "partition" covering the longest
  // context, rounded up to whole tiles.
  int32_t part = partition;
  if (part == 0) part = static_cast<int32_t>(((std::max(max_context_len, 1) + kTile - 1) / kTile) * kTile);
  const int64_t parts = parts_for(max_context_len, part);
  if (parts > 0x7fffffff) return PA_ERR_INVALID_ARG;
  const size_t need = ws_bytes(num_seqs, num_heads, head_dim, parts);
  if (static_cast<int64_t>(parts) * num_kv_heads * num_seqs > 0x7fffffffLL)
    return PA_ERR_INVALID_ARG;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return PA_ERR_WORKSPACE;
  const int G = num_heads / num_kv_heads;
  const float sl2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool nt = (flags & PA_DECODE_STREAM_KV) != 0;
  if (find) {
    if (G != 1 && G != 2 && G != 4 && G != 8) return PA_ERR_UNSUPPORTED;
    const FoundLayout f =
        found_layout(num_seqs, num_heads, head_dim, max_context_len, partition);
    const int64_t nchunks = (static_cast<int64_t>(kPrefixMembers) * G + 31) / 32;
    if (f.pre + f.rest > 0x7fffffff || f.rest * num_kv_heads * num_seqs > 0x7fffffffLL ||
        f.pre * f.runs * nchunks * num_kv_heads > 0x7fffffffLL)
      return PA_ERR_INVALID_ARG;
    if (workspace == nullptr || workspace_bytes < f.total) return PA_ERR_WORKSPACE;
    uint8_t* base = static_cast<uint8_t*>(workspace);
    int32_t* groups = reinterpret_cast<int32_t*>(base + f.groups_off);
    int32_t* pre_lens = reinterpret_cast<int32_t*>(base + f.lens_off);
    hipLaunchKernelGGL(find_groups_kernel, dim3(static_cast<uint32_t>(f.runs)), dim3(64), 0, st,
                       block_tables, max_blocks_per_seq, context_lens, num_seqs,
                       static_cast<int32_t>(PA_FIND_SHARED_MIN_PREFIX), groups, pre_lens);
    const int rc = pa_launch_status();
    if (rc != PA_OK) return rc;
    return shared_launch(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq,
                         context_lens, num_seqs, num_heads, num_kv_heads, f.part, f.pre, f.rest,
                         groups, f.runs, pre_lens, workspace, sl2, st, nt);
  }
  const Split sp{static_cast<int32_t>(parts), static_cast<int32_t>(parts), {nullptr, 0, part}};
#define PA_DECODE_BS(BSZ)                                                                      \
  dispatch_block<BSZ>(dtype, head_dim, G, out, q, k_cache, v_cache, block_tables,              \
                      max_blocks_per_seq, context_lens, num_seqs, num_heads, num_kv_heads, sp, \
                      part, sl2, workspace, st, nt)
  switch (block_size) {
    case 8: return PA_DECODE_BS(8);
    case 32: return PA_DECODE_BS(32);
    case 64: return PA_DECODE_BS(64);
    default: return PA_DECODE_BS(16);
  }
#undef PA_DECODE_BS
}

extern "C" int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         int32_t num_blocks, float scale, int32_t partition,
                         int32_t max_context_len, void* workspace, size_t workspace_bytes,
                         int32_t dtype, int32_t flags, void* stream) {
  return decode_call(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                     num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                     partition, max_context_len, workspace, workspace_bytes, dtype, flags,
                     stream);
}

namespace {

// The partials of pa_decode_no_alloc: a file-scope device array, one copy per
// GPU, loaded with the library's code object and kept until the process ends.
// Host code uses only the per-device address hipGetSymbolAddress returns (the
// array's name on the host is a stand-in, not a device address).
static __device__ __align__(256) unsigned char scratch[PA_NO_ALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Address of this GPU's copy of the scratch array (looked up once per
// device, with that device current), or nullptr on failure.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" int pa_decode_no_alloc(void* out, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* block_tables,
                                  int32_t max_blocks_per_seq, const int32_t* context_lens,
                                  int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                  float scale, int32_t partition, int32_t max_context_len,
                                  int32_t dtype, int32_t flags, void* stream) {
  // The partials pa_decode would need (0 when no sequence can span two
  // partitions) must fit the array: a larger call is refused before any
  // device work.  Invalid arguments are reported by pa_decode's own checks.
  const size_t need = pa_decode_workspace_bytes_flags(num_seqs, num_heads, head_dim,
                                                      max_context_len, partition, flags);
  if (need > PA_NO_ALLOC_SCRATCH_BYTES) return PA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    ws = device_scratch();
    if (ws == nullptr) return PA_ERR_DEVICE;
  }
  return decode_call(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                     num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                     partition, max_context_len, ws, ws ? PA_NO_ALLOC_SCRATCH_BYTES : 0, dtype,
                     flags, stream);
}


extern "C" size_t pa_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_heads,
                                                          int32_t head_dim,
                                                          int32_t max_context_len,
                                                          int32_t max_prefix_len,
                                                          int32_t partition) {
  if (num_seqs <= 0 || num_heads <= 0 || head_dim <= 0 || partition < 0) return 0;
  int64_t pre, rest;
  shared_slots(max_context_len, max_prefix_len, unsplit_partition(partition, max_context_len), pre,
               rest);
  return ws_bytes(num_seqs, num_heads, head_dim, pre + rest);
}

extern "C" int pa_decode_shared_prefix(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t num_blocks, float scale, int32_t partition,
    int32_t max_context_len, const int32_t* prefix_groups, int32_t num_groups,
    const int32_t* seq_prefix_lens, int32_t max_prefix_len, void* workspace,
    size_t workspace_bytes, int32_t dtype, int32_t flags, void* stream) {
  if (dtype != PA_F32 && dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  if (flags & ~PA_DECODE_STREAM_KV) return PA_ERR_INVALID_ARG;
  const bool nt = (flags & PA_DECODE_STREAM_KV) != 0;
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0 ||
      num_blocks <= 0 || partition < 0 || max_context_len < 0 || num_groups < 0 ||
      max_prefix_len < 0)
    return PA_ERR_INVALID_ARG;
  if (num_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (dtype != PA_BF16 || block_size != kBS || head_dim != 128) return PA_ERR_UNSUPPORTED;
  const int G = num_heads / num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return PA_ERR_UNSUPPORTED;
  if (partition % kTile != 0 || max_prefix_len % kBS != 0 || max_prefix_len > max_context_len)
    return PA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * kBS)
    return PA_ERR_INVALID_ARG;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return PA_ERR_INVALID_ARG;
  const bool split = num_groups > 0 && max_prefix_len > 0;
  if (split && (!prefix_groups || !seq_prefix_lens)) return PA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_cache) |
       reinterpret_cast<uintptr_t>(v_cache)) & 15)
    return PA_ERR_INVALID_ARG;
  const int32_t part = unsplit_partition(partition, max_context_len);
  int64_t pre, rest;
  shared_slots(max_context_len, split ? max_prefix_len : 0, part, pre, rest);
  const int64_t slots = pre + rest;
  const int64_t nchunks = (static_cast<int64_t>(kPrefixMembers) * G + 31) / 32;  // 32 queries each
  if (slots > 0x7fffffff || rest * num_kv_heads * num_seqs > 0x7fffffffLL ||
      pre * num_groups * nchunks * num_kv_heads > 0x7fffffffLL)
    return PA_ERR_INVALID_ARG;
  const size_t need = ws_bytes(num_seqs, num_heads, head_dim, slots);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return PA_ERR_WORKSPACE;
  const float sl2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  return shared_launch(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                       num_seqs, num_heads, num_kv_heads, part, pre, rest, prefix_groups,
                       split ? num_groups : 0, seq_prefix_lens, workspace, sl2,
                       static_cast<hipStream_t>(stream), nt);
}
