// A mixed batch -- prefill chunks beside single decode tokens -- in one launch
// (gfx950).
//
// Page "vLLM PagedAttention chuyên sâu: Phân mảnh bộ nhớ KV Cache, Prefill
// theo khối & Prefix Caching" (locionic.com), sections "Chunked Prefill" and
// "Cơ chế của Chunked Prefill": the scheduler interleaves prefill chunks with
// the decode steps of other requests, so one batch holds both; the summary
// page on vLLM (tr.news.hada.io): requests join the batch as they arrive and
// finished sequences leave it (continuous batching).  One launch serves the whole batch:
//  * workgroups [0, prefill workgroups) run the chunked-prefill workgroup of
//    prefill_core.h (matrix cores, 128 query rows of one (sequence, head));
//  * the rest run four decode items each, one per wave, with pa_decode's
//    bodies: the one-wave body of decode_core.h for 1 or 2 query heads per kv
//    head, the matrix-core body of decode_mfma.h for 4 or 8.  An item is a
//    (partition, decode sequence, kv head) as in pa_decode, and decode
//    sequences longer than one partition are merged afterwards by pa_decode's
//    second pass (the only other launch).
// The long prefill workgroups are dispatched first and the short decode items
// fill the chip behind them, so neither part waits for the other's tail.

#include "decode_core.h"
#include "decode_mfma.h"
#include "prefill_core.h"

namespace {

constexpr int kMixedWaves = 4;

template <int G, bool NT>
__global__ __launch_bounds__(kMixedWaves * 64, 2) void mixed_step_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ qsl, const int32_t* __restrict__ context_lens,
    int32_t num_prefill_seqs, uint32_t prefill_wgs, int32_t num_qtiles,
    int64_t num_prefill_tokens, int32_t num_decode_seqs, int32_t decode_partition,
    int32_t decode_parts, Partials ws, int32_t num_heads, int32_t num_kv_heads,
    float scale_log2) {
  constexpr bool PVB = G >= 4;
  __shared__ StepBuf buf[kRing];
  __shared__ __attribute__((aligned(16))) weight_t<PVB> p_lds[kMixedWaves][G >= 4 ? 1 : G * kTile];
  if (blockIdx.x < prefill_wgs) {
    prefill_tile<kMixedWaves>(blockIdx.x, buf, out, q, kc, vc, block_tables, max_blocks, qsl,
                                 context_lens, num_prefill_seqs, num_heads, num_kv_heads,
                                 num_qtiles, scale_log2);
    return;
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t item = (blockIdx.x - prefill_wgs) * kMixedWaves + wave;
  const int64_t row0 = num_prefill_tokens * num_heads * kD;  // first decode query row
  // items: kv head fastest, then decode sequence, then partition
  const int32_t* bt = block_tables + static_cast<int64_t>(num_prefill_seqs) * max_blocks;
  const RangeSplit rs{nullptr, 0, decode_partition};
  if constexpr (G >= 4)
    mfma_decode_item<NT>(item, out + row0, ws, q + row0, kc, vc, bt, max_blocks,
                     context_lens + num_prefill_seqs, num_decode_seqs, num_heads, num_kv_heads,
                     decode_parts, decode_partition, scale_log2, rs);
  else
    decode_item<uint16_t, kD, G, PVB, kBS, NT>(item, p_lds[wave], out + row0, ws, q + row0, kc, vc, bt,
                                      max_blocks, context_lens + num_prefill_seqs,
                                      num_decode_seqs, num_heads, num_kv_heads, decode_parts,
                                      decode_partition, scale_log2, rs);
}

// Decode partition used for a requested one (0: one partition covering the
// longest decode context).
int32_t mixed_partition(int32_t partition, int32_t max_decode_context) {
  if (partition != 0) return partition;
  return static_cast<int32_t>((std::max(max_decode_context, 1) + kTile - 1) / kTile * kTile);
}

}  // namespace

extern "C" size_t pa_mixed_step_workspace_bytes(int32_t num_decode_seqs, int32_t num_heads,
                                                int32_t head_dim, int32_t max_decode_context,
                                                int32_t partition) {
  if (num_decode_seqs <= 0 || num_heads <= 0 || head_dim <= 0 || partition < 0) return 0;
  return ws_bytes(num_decode_seqs, num_heads, head_dim,
                  parts_for(max_decode_context, mixed_partition(partition, max_decode_context)));
}

extern "C" int pa_mixed_step(void* out, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* query_start_loc, const int32_t* context_lens,
                             int32_t num_prefill_seqs, int32_t num_prefill_tokens,
                             int32_t max_query_len, int32_t num_decode_seqs,
                             int32_t max_decode_context, int32_t num_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, int32_t num_blocks,
                             float scale, int32_t partition, void* workspace,
                             size_t workspace_bytes, int32_t dtype, int32_t flags,
                             void* stream) {
  if (dtype != PA_BF16 && dtype != PA_F32) return PA_ERR_UNSUPPORTED;
  if (num_prefill_seqs < 0 || num_prefill_tokens < 0 || max_query_len < 0 ||
      num_decode_seqs < 0 || max_decode_context < 0 || num_heads <= 0 || num_kv_heads <= 0 ||
      max_blocks_per_seq <= 0 || num_blocks <= 0 || partition < 0 || partition % kTile != 0)
    return PA_ERR_INVALID_ARG;
  if (num_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (flags & ~PA_DECODE_STREAM_KV) return PA_ERR_INVALID_ARG;
  if (dtype != PA_BF16 || head_dim != kD || block_size != kBS) return PA_ERR_UNSUPPORTED;
  const int G = num_heads / num_kv_heads;
  const bool nt = (flags & PA_DECODE_STREAM_KV) != 0;
  if (G != 1 && G != 2 && G != 4 && G != 8) return PA_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(max_decode_context) > static_cast<int64_t>(max_blocks_per_seq) * kBS)
    return PA_ERR_INVALID_ARG;
  if (num_prefill_seqs > 0 && max_query_len == 0 && num_prefill_tokens != 0)
    return PA_ERR_INVALID_ARG;
  if (num_prefill_seqs + num_decode_seqs == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens ||
      (num_prefill_seqs > 0 && !query_start_loc))
    return PA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(out) |
       reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache)) & 15)
    return PA_ERR_INVALID_ARG;
  constexpr int kRows = kMixedWaves * 32;
  const int64_t qtiles = (static_cast<int64_t>(max_query_len) + kRows - 1) / kRows;
  const int64_t units = static_cast<int64_t>(num_heads) * num_prefill_seqs;
  const int64_t pf_wgs = qtiles > 0 ? (units + kXcds - 1) / kXcds * kXcds * qtiles : 0;
  const int32_t dec_part = mixed_partition(partition, max_decode_context);
  const int64_t dec_parts = num_decode_seqs > 0 ? parts_for(max_decode_context, dec_part) : 1;
  const int64_t items = dec_parts * num_decode_seqs * num_kv_heads;
  const int64_t dec_wgs = (items + kMixedWaves - 1) / kMixedWaves;
  if (pf_wgs + dec_wgs > 0x7fffffffLL || dec_parts > 0x7fffffffLL) return PA_ERR_INVALID_ARG;
  const size_t need = num_decode_seqs > 0 ? ws_bytes(num_decode_seqs, num_heads, kD, dec_parts) : 0;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return PA_ERR_WORKSPACE;
  const Partials p = carve(workspace, num_decode_seqs, num_heads, kD, dec_parts);
  const float sl2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  const dim3 grid(static_cast<uint32_t>(pf_wgs + dec_wgs)), block(kMixedWaves * 64);
  hipStream_t st = static_cast<hipStream_t>(stream);
#define PA_MIXED_LAUNCH(GG)                                                                      \
  hipLaunchKernelGGL((nt ? mixed_step_kernel<GG, true> : mixed_step_kernel<GG, false>), grid,   \
                     block, 0, st, static_cast<uint16_t*>(out),                                  \
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cache),    \
                     static_cast<const uint16_t*>(v_cache), block_tables, max_blocks_per_seq,   \
                     query_start_loc, context_lens, num_prefill_seqs,                            \
                     static_cast<uint32_t>(pf_wgs), static_cast<int32_t>(qtiles),                \
                     static_cast<int64_t>(num_prefill_tokens), num_decode_seqs, dec_part,        \
                     static_cast<int32_t>(dec_parts), p, num_heads, num_kv_heads, sl2)
  switch (G) {
    case 1: PA_MIXED_LAUNCH(1); break;
    case 2: PA_MIXED_LAUNCH(2); break;
    case 4: PA_MIXED_LAUNCH(4); break;
    default: PA_MIXED_LAUNCH(8); break;
  }
#undef PA_MIXED_LAUNCH
  if (dec_parts > 1) {
    const int64_t row0 = static_cast<int64_t>(num_prefill_tokens) * num_heads * kD;
    hipLaunchKernelGGL((decode_merge_kernel<uint16_t, kD>),
                       dim3(static_cast<uint32_t>(num_decode_seqs) * num_heads), dim3(64), 0, st,
                       static_cast<uint16_t*>(out) + row0, p,
                       context_lens + num_prefill_seqs, num_heads,
                       static_cast<int32_t>(dec_parts), dec_part,
                       RangeSplit{nullptr, 0, dec_part}, max_blocks_per_seq * kBS);
  }
  return pa_launch_status();
}
