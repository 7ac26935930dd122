// Chunked prefill over a paged KV cache on gfx950 matrix cores: the kernel and
// the pa_prefill_chunk entry point.  The workgroup body is in prefill_core.h.

#include "prefill_pingpong.h"

namespace {

constexpr int kWaves = 4;
constexpr int kRowsPerWG = kWaves * 32;

// 128 query rows of one (sequence, head) per workgroup (prefill_core.h); three
// workgroups share a CU.
template <int W>
__global__ __launch_bounds__(W * 64, 3) void prefill_chunk_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ qsl, const int32_t* __restrict__ context_lens, int32_t num_seqs,
    int32_t num_heads, int32_t num_kv_heads, int32_t num_qtiles, float scale_log2) {
  __shared__ StepBuf buf[kRing];
  prefill_tile<W>(blockIdx.x, buf, out, q, kc, vc, block_tables, max_blocks, qsl,
                      context_lens, num_seqs, num_heads, num_kv_heads, num_qtiles, scale_log2);
}

// 256 query rows of one (sequence, head) per workgroup, two groups of 4 waves
// taking turns on the matrix cores (prefill_pingpong.h).  One workgroup per
// CU: 8 waves of up to 256 registers and 96 KB of LDS.
__global__ __launch_bounds__(kWavesPP * 64, 1) void prefill_chunk_pp_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ qsl, const int32_t* __restrict__ context_lens, int32_t num_seqs,
    int32_t num_heads, int32_t num_kv_heads, int32_t num_qtiles, float scale_log2) {
  __shared__ StepBuf ring[kRingPP];
  prefill_tile_pp(blockIdx.x, ring, out, q, kc, vc, block_tables, max_blocks, qsl, context_lens,
                  num_seqs, num_heads, num_kv_heads, num_qtiles, scale_log2);
}

}  // namespace

extern "C" int pa_prefill_chunk(void* out, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* block_tables,
                                int32_t max_blocks_per_seq, const int32_t* query_start_loc,
                                const int32_t* context_lens, int32_t num_seqs,
                                int32_t max_query_len, int32_t num_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                float scale, int32_t dtype, void* stream) {
  if (dtype != PA_BF16 && dtype != PA_F32) return PA_ERR_UNSUPPORTED;
  if (num_seqs < 0 || max_query_len < 0 || num_heads <= 0 || num_kv_heads <= 0 ||
      max_blocks_per_seq <= 0 || num_blocks <= 0)
    return PA_ERR_INVALID_ARG;
  if (num_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (num_kv_heads > (1 << 19)) return PA_ERR_INVALID_ARG;  // a cache block's bytes fit 31 bits
  if (dtype != PA_BF16 || head_dim != kD || block_size != kBS) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0 || max_query_len == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !query_start_loc || !context_lens)
    return PA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(out) |
       reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache)) & 15)
    return PA_ERR_INVALID_ARG;
  const int64_t units = static_cast<int64_t>(num_heads) * num_seqs;
  const float sl2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  if (max_query_len > kRowsPerWG) {  // chunks longer than one 128-row tile
    const int64_t qtiles = (static_cast<int64_t>(max_query_len) + kRowsPP - 1) / kRowsPP;
    const int64_t grid = (units + kXcds - 1) / kXcds * kXcds * qtiles;
    if (grid > 0x7fffffffLL) return PA_ERR_INVALID_ARG;
    hipLaunchKernelGGL(prefill_chunk_pp_kernel, dim3(static_cast<uint32_t>(grid)),
                       dim3(kWavesPP * 64), 0, static_cast<hipStream_t>(stream),
                       static_cast<uint16_t*>(out), static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(k_cache), static_cast<const uint16_t*>(v_cache),
                       block_tables, max_blocks_per_seq, query_start_loc, context_lens, num_seqs,
                       num_heads, num_kv_heads, static_cast<int32_t>(qtiles), sl2);
    return pa_launch_status();
  }
  const int64_t qtiles = (static_cast<int64_t>(max_query_len) + kRowsPerWG - 1) / kRowsPerWG;
  const int64_t grid = (units + kXcds - 1) / kXcds * kXcds * qtiles;
  if (grid > 0x7fffffffLL) return PA_ERR_INVALID_ARG;
  hipLaunchKernelGGL((prefill_chunk_kernel<kWaves>), dim3(static_cast<uint32_t>(grid)),
                     dim3(kWaves * 64), 0,
                     static_cast<hipStream_t>(stream), static_cast<uint16_t*>(out),
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cache),
                     static_cast<const uint16_t*>(v_cache), block_tables, max_blocks_per_seq,
                     query_start_loc, context_lens, num_seqs, num_heads, num_kv_heads,
                     static_cast<int32_t>(qtiles), sl2);
  return pa_launch_status();
}
