// Chunked prefill over a paged KV cache on gfx950 matrix cores.
//
// Page "vLLM PagedAttention chuyên sâu: Phân mảnh bộ nhớ KV Cache, Prefill
// theo khối & Prefix Caching" (locionic.com), sections "Chunked Prefill" and
// "Cơ chế của Chunked Prefill": a long prompt is processed in chunks, in
// order, each chunk's KV accumulating in paged blocks; prefill is the
// compute-heavy phase.  A chunk of n_q queries against L cached-plus-chunk
// tokens is a dense contraction, so it runs on MFMA
// (v_mfma_f32_16x16x32_bf16, fp32 accumulation).
//
// Causal alignment: query i of the chunk sits at position L - n_q + i and
// attends to positions 0 .. L - n_q + i.
//
// Formulation (per wave: 16 query rows of one head):
//   S^T = K Q^T   A = 16 tokens x 32 dims of K (one 1 KB run of the x-packed
//                 key page), B = 32 dims x 16 queries (registers)
//   O^T += V^T P^T   A = 16 dims x 32 tokens of V (d-major value page),
//                 B = P^T straight from the S^T accumulators.
// With the accumulator layout of a 16x16 MFMA (lane i holds column i%16, rows
// 4*(i/16)..+3) every lane owns one query column, so the online softmax state
// of a query lives in the four lanes i%16 == q and the 32-token P^T operand
// is assembled in registers: slot k of lane group g is token 4g+k (k<4) of the
// first page and 16+4g+(k-4) of the second; V^T uses the same token order.

#include "pa_device.h"

namespace {

constexpr int kBS = 16;
constexpr int kD = 128;
constexpr int kWavesPerWG = 4;
constexpr int kRowsPerWave = 16;

__device__ __forceinline__ pa::bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(pa::bf16x8_t, v); }

__device__ __forceinline__ pa::f32x4_t mfma16(uint4 a, uint4 b, pa::f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ float xgroup_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  return fmaxf(v, __shfl_xor(v, 32, 64));
}
__device__ __forceinline__ float xgroup_sum(float v) {
  v += __shfl_xor(v, 16, 64);
  return v + __shfl_xor(v, 32, 64);
}

// grid (ceil(max_query_len / 64), num_heads, num_seqs), 256 threads.
__global__ __launch_bounds__(256) void prefill_chunk_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ qsl, const int32_t* __restrict__ context_lens, int32_t num_heads,
    int32_t num_kv_heads, float scale_log2) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = blockIdx.y;
  const int s = blockIdx.z;
  const int g = h / (num_heads / num_kv_heads);
  const int q0 = qsl[s];
  const int n_q = qsl[s + 1] - q0;
  const int L = context_lens[s];
  const int row_a = blockIdx.x * (kWavesPerWG * kRowsPerWave) + wave * kRowsPerWave;
  if (row_a >= n_q) return;
  const int first_pos = L - n_q;  // position of query row 0

  const int qc = lane & 15;  // this lane's query column
  const int grp = lane >> 4;
  const int my_row = min(row_a + qc, n_q - 1);  // rows past the chunk mirror the last one
  const int my_pos = first_pos + my_row;
  const int last_pos = first_pos + min(row_a + kRowsPerWave, n_q) - 1;
  const int first_row_pos = first_pos + row_a;

  // Q^T operand: lane (qc, grp) holds dims 32*kk + 8*grp .. +7 of its query.
  uint4 qreg[4];
  {
    const uint16_t* qrow = q + (static_cast<int64_t>(q0 + my_row) * num_heads + h) * kD;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      qreg[kk] = *reinterpret_cast<const uint4*>(qrow + 32 * kk + 8 * grp);
  }

  const int32_t* bt_row = block_tables + static_cast<int64_t>(s) * max_blocks;
  const int64_t page = static_cast<int64_t>(kBS) * kD;
  const int64_t blk_stride = static_cast<int64_t>(num_kv_heads) * page;
  const int64_t head_off = static_cast<int64_t>(g) * page;

  pa::f32x4_t o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = pa::f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int kv_end = last_pos + 1;  // tokens 0 .. last_pos are needed
  for (int t0 = 0; t0 < kv_end; t0 += 2 * kBS) {
    int phys[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int lb = t0 / kBS + p;
      phys[p] = lb * kBS < kv_end ? bt_row[lb] : -1;
    }
    // ---- S^T for two pages
    pa::f32x4_t sacc[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      sacc[p] = pa::f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (phys[p] >= 0) {
        const uint16_t* kp = kc + phys[p] * blk_stride + head_off;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          // chunk c = 4*kk + grp of token qc: byte run (c*16 + qc) * 16
          const uint4 a = *reinterpret_cast<const uint4*>(kp + ((4 * kk + grp) * kBS + qc) * 8);
          sacc[p] = mfma16(a, qreg[kk], sacc[p]);
        }
      }
    }
    // ---- mask + online softmax (lane's query column)
    const bool need_mask = t0 + 2 * kBS - 1 > first_row_pos || t0 + 2 * kBS > L;
    float sv[8];
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + 16 * p + 4 * grp + r;
        float x = sacc[p][r] * scale_log2;
        if (need_mask && (t > my_pos || t >= L || phys[p] < 0)) x = -INFINITY;
        sv[4 * p + r] = x;
      }
    float mt = sv[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mt = fmaxf(mt, sv[i]);
    mt = xgroup_max(mt);
    const float m_new = fmaxf(m_run, mt);
    // a query with every token so far masked keeps m = -inf; guard the rescale
    const float alpha = m_new == -INFINITY ? 1.f : pa::fast_exp2(m_run - m_new);
    float pv[8];
    float lsum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pv[i] = m_new == -INFINITY ? 0.f : pa::fast_exp2(sv[i] - m_new);
      lsum += pv[i];
    }
    l_run = l_run * alpha + lsum;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] *= alpha;
    // P^T operand: slots 0..3 = page 0 tokens 4grp..+3, 4..7 = page 1 tokens 4grp..+3
    uint4 pb;
    pb.x = pa::pack_bf16x2(pv[0], pv[1]);
    pb.y = pa::pack_bf16x2(pv[2], pv[3]);
    pb.z = pa::pack_bf16x2(pv[4], pv[5]);
    pb.w = pa::pack_bf16x2(pv[6], pv[7]);

    // ---- O^T += V^T P^T over 8 tiles of 16 dims
    const bool tail = t0 + 2 * kBS > L;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int d = 16 * dt + qc;
      uint2 v0 = make_uint2(0, 0), v1 = make_uint2(0, 0);
      if (phys[0] >= 0)
        v0 = *reinterpret_cast<const uint2*>(vc + phys[0] * blk_stride + head_off + d * kBS + 4 * grp);
      if (phys[1] >= 0)
        v1 = *reinterpret_cast<const uint2*>(vc + phys[1] * blk_stride + head_off + d * kBS + 4 * grp);
      if (tail) {
        // zero value elements of tokens at or past L (the cache may hold NaN)
        uint32_t w[4] = {v0.x, v0.y, v1.x, v1.y};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tb = t0 + 16 * (i >> 1) + 4 * grp + 2 * (i & 1);
          const uint32_t mk = (tb < L ? 0x0000ffffu : 0u) | (tb + 1 < L ? 0xffff0000u : 0u);
          w[i] &= mk;
        }
        v0 = make_uint2(w[0], w[1]);
        v1 = make_uint2(w[2], w[3]);
      }
      const uint4 a = make_uint4(v0.x, v0.y, v1.x, v1.y);
      o[dt] = mfma16(a, pb, o[dt]);
    }
  }

  const float lt = xgroup_sum(l_run);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (row_a + qc < n_q) {
    uint16_t* orow = out + (static_cast<int64_t>(q0 + row_a + qc) * num_heads + h) * kD;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      uint2 w;
      w.x = pa::pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv);
      w.y = pa::pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv);
      *reinterpret_cast<uint2*>(orow + 16 * dt + 4 * grp) = w;
    }
  }
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
  if (dtype != PA_BF16 || head_dim != kD || block_size != kBS) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0 || max_query_len == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !query_start_loc || !context_lens)
    return PA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(out) |
       reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache)) & 15)
    return PA_ERR_INVALID_ARG;
  if (num_seqs > 65535 || num_heads > 65535) return PA_ERR_INVALID_ARG;
  const int rows = kWavesPerWG * kRowsPerWave;
  const uint32_t gx = static_cast<uint32_t>((static_cast<int64_t>(max_query_len) + rows - 1) / rows);
  const float sl2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  hipLaunchKernelGGL(prefill_chunk_kernel, dim3(gx, num_heads, num_seqs), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<uint16_t*>(out),
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cache),
                     static_cast<const uint16_t*>(v_cache), block_tables, max_blocks_per_seq,
                     query_start_loc, context_lens, num_heads, num_kv_heads, sl2);
  return pa_launch_status();
}
