// Chunked prefill over a paged KV cache on gfx950 matrix cores.
//
// Page "vLLM PagedAttention chuyên sâu: Phân mảnh bộ nhớ KV Cache, Prefill
// theo khối & Prefix Caching" (locionic.com), sections "Chunked Prefill" and
// "Cơ chế của Chunked Prefill": a long prompt is processed in chunks, in
// order, each chunk's KV accumulating in paged blocks; prefill is the
// compute-heavy phase.  A chunk of n_q queries against L cached-plus-chunk
// tokens is a dense contraction, so it runs on MFMA
// (v_mfma_f32_32x32x16_bf16, fp32 accumulation).
//
// Causal alignment: query i of the chunk sits at position L - n_q + i and
// attends to positions 0 .. L - n_q + i.
//
// Work decomposition.  A workgroup of 4 waves owns 128 consecutive query rows
// of one (sequence, head); each wave owns 32 of them.  The workgroup walks the
// keys/values in steps of 32 tokens (two 16-token pages): each step's K and V
// pages are copied once, cooperatively, into a ring of four LDS step buffers
// with direct-to-LDS loads issued three steps ahead of use, then every wave
// computes, in transposed form so no operand needs a shuffle,
//   S^T[32 tokens x 32 queries] = K Q^T    (8 MFMAs over head_dim 128)
//   O^T[128 dims x 32 queries] += V^T P^T  (8 MFMAs)
// With the 32x32 accumulator layout (lane l holds column l%32, rows
// 8*(j/4) + 4*(l/32) + j%4 for j = 0..15), each lane owns one query column:
// the online softmax of a query lives in lanes q and q+32, and the bf16 P^T
// operand is built in registers from the lane's own scores.  V^T's operand
// uses the same token order.  O is rescaled only when a query's running max
// grows by more than 2^8 (the exponentials then stay below 2^8, far inside
// fp32 and bf16 range; the final O / l is unchanged).
//
// Workgroups are mapped so the q-tiles of one (sequence, head) run on the same
// XCD at the same time: its K/V pages come from HBM once and are served to the
// other q-tiles from that XCD's L2.

#include "page_ring.h"

namespace {

using pa::ring::kBS;
using pa::ring::kD;
using pa::ring::kPageElems;
using pa::ring::kPages;
using pa::ring::kRing;
using pa::ring::kStep;
using pa::ring::StepBuf;
using pa::ring::vhalf;
constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;
constexpr int kRowsPerWG = kWaves * kRowsPerWave;
constexpr uint32_t kXcds = 8;
constexpr float kLazyRescale = 8.f;   // log2 units

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ pa::f32x16_t mfma32(uint4 a, uint4 b, pa::f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ float swap32_max(float v) { return fmaxf(v, __shfl_xor(v, 32, 64)); }

// grid (ceil(max_query_len / 128) * num_heads * num_seqs rounded up to 8), 256 threads.
__global__ __launch_bounds__(256, 2) void prefill_chunk_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ qsl, const int32_t* __restrict__ context_lens, int32_t num_seqs,
    int32_t num_heads, int32_t num_kv_heads, int32_t num_qtiles, float scale_log2) {
  __shared__ StepBuf buf[kRing];

  // XCD-aware order: logical = (seq, head, q-tile) with q-tile fastest, and XCD
  // x runs the x-th contiguous slice, so a (seq, head)'s q-tiles share an L2.
  const uint32_t per_xcd = gridDim.x / kXcds;
  const uint32_t li = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  const int qt = num_qtiles - 1 - static_cast<int>(li % num_qtiles);  // long q-tiles first
  const uint32_t sh = li / num_qtiles;
  const int h = static_cast<int>(sh % static_cast<uint32_t>(num_heads));
  const int s = static_cast<int>(sh / static_cast<uint32_t>(num_heads));
  if (s >= num_seqs) return;  // grid padding (whole workgroup)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = h / (num_heads / num_kv_heads);
  const int q0 = qsl[s];
  const int n_q = qsl[s + 1] - q0;
  const int L = context_lens[s];
  const int wg_row0 = qt * kRowsPerWG;
  if (wg_row0 >= n_q) return;  // whole workgroup idle
  const int first_pos = L - n_q;                  // position of chunk row 0
  const int wg_last = first_pos + min(wg_row0 + kRowsPerWG, n_q) - 1;
  const int nsteps = wg_last / kStep + 1;         // steps covering tokens 0 .. wg_last

  const int row0 = wg_row0 + wave * kRowsPerWave;
  const bool wave_active = row0 < n_q;
  const int qn = lane & 31;   // this lane's query column
  const int hh = lane >> 5;   // which half of the accumulator rows
  const int my_row = min(row0 + qn, n_q - 1);
  const int my_pos = first_pos + my_row;
  const int wave_last = first_pos + min(row0 + kRowsPerWave, n_q) - 1;
  const int wave_first = first_pos + row0;

  // Q^T operand: lane (qn, hh) holds dims 16*kk + 8*hh .. +7 of its query row.
  uint4 qreg[8];
  {
    const uint16_t* qrow = q + (static_cast<int64_t>(q0 + my_row) * num_heads + h) * kD + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qreg[kk] = *reinterpret_cast<const uint4*>(qrow + 16 * kk);
    // Consume the query registers here: otherwise their load waits land in
    // the step loop, where (loads retiring in order) they would also drain
    // every step copy in flight.
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      asm volatile("" : "+v"(qreg[kk].x), "+v"(qreg[kk].y), "+v"(qreg[kk].z), "+v"(qreg[kk].w));
  }

  const int32_t* bt_row = block_tables + static_cast<int64_t>(s) * max_blocks;
  const int64_t blk_stride = static_cast<int64_t>(num_kv_heads) * kPageElems;
  const int64_t head_off = static_cast<int64_t>(g) * kPageElems;

  // Pages past the last needed token load logical block 0 instead (always
  // valid): their scores are masked, and their values must just be finite.
  auto issue = [&](int step) {
    const int lb = step * kPages + (wave >> 1);
    pa::ring::issue_step(buf[step % kRing], kc, vc, bt_row[lb * kBS <= wg_last ? lb : 0],
                         blk_stride, head_off, wave, lane);
  };
  // Values of tokens at or past L in the step's last page: zero them in LDS
  // (the cache may hold NaN there, and 0 * NaN would reach every query).
  auto zero_tail = [&](int step) {
    StepBuf& B = buf[step % kRing];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int row = tid + 256 * r;      // (page, dim) row, 2 units each
      const int page = row >> 7, d = row & 127;
      const int tok0 = (step * kPages + page) * kBS;
      uint4* vr = &B.v[page * 256 + d * 2];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int keep = L - (tok0 + 8 * half);
        if (keep < 8) {
          uint4& w4 = vr[vhalf(d, half)];
          uint32_t w[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
          for (int i = 0; i < 4; ++i)
            w[i] &= (2 * i < keep ? 0x0000ffffu : 0u) | (2 * i + 1 < keep ? 0xffff0000u : 0u);
          w4 = make_uint4(w[0], w[1], w[2], w[3]);
        }
      }
    }
  };

  pa::f32x16_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pa::f32x16_t{};
  float m_run = -INFINITY, l_run = 0.f;

  for (int st = 0; st < kRing - 1 && st < nsteps; ++st) issue(st);

  for (int step = 0; step < nsteps; ++step) {
    const StepBuf& B = buf[step % kRing];
    // wait for this wave's copies of this step (later steps may stay in
    // flight), then for everyone's
    pa::ring::wait_step(min(kRing - 2, nsteps - 1 - step));
    const int t0 = step * kStep;
    if (t0 + kStep > L) {  // the step holding the sequence's last token
      zero_tail(step);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
    // the buffer written next was last read in the previous step, which every
    // wave has finished (barrier above)
    if (step + kRing - 1 < nsteps) issue(step + kRing - 1);

    if (wave_active && t0 <= wave_last) {
      // ---- S^T = K Q^T
      pa::f32x16_t sa = pa::f32x16_t{};
      const int m = lane & 31;  // token row of the K operand
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int c = 2 * kk + hh;
        const uint4 a0 = B.k[((m >> 4) * 16 + c) * 16 + pa::ring::kslot(c, m & 15)];
        sa = mfma32(a0, qreg[kk], sa);
      }
      // ---- online softmax over this lane's 16 tokens (query qn).  Token of
      // element j: t0 + 8*(j/4) + 4*hh + j%4.
      float x[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) x[j] = sa[j];
      if (t0 + kStep - 1 > wave_first || t0 + kStep > L) {  // diagonal or tail step
        const int lim = min(my_pos, L - 1) - t0 - 4 * hh;   // keep offsets <= lim
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int off = 8 * (j >> 2) + (j & 3);
          if (off > lim) x[j] = -INFINITY;
        }
      }
      float mx = fmaxf(x[0], x[1]);
#pragma unroll
      for (int j = 2; j < 16; j += 2) mx = fmaxf(mx, fmaxf(x[j], x[j + 1]));
      mx = swap32_max(mx) * scale_log2;  // scale > 0: max commutes with it
      // Lazy rescale, wave-uniform: only when some query's max grew by > 2^8.
      if (__any(mx > m_run + kLazyRescale)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = pa::fast_exp2(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] *= alpha;
        m_run = m_new;
      }
      const float neg_m = m_run == -INFINITY ? 0.f : -m_run;
      uint32_t pw[8];
      float ls = 0.f;
#pragma unroll
      for (int j = 0; j < 16; j += 2) {
        const float p0 = pa::fast_exp2(fmaf(x[j], scale_log2, neg_m));
        const float p1 = pa::fast_exp2(fmaf(x[j + 1], scale_log2, neg_m));
        ls += p0 + p1;
        pw[j >> 1] = pa::pack_bf16x2(p0, p1);
      }
      l_run += ls;
      // P^T operands, one per page: page pg's 16 tokens are the lane's
      // elements 8*pg .. 8*pg+7 (tokens 4hh..+3 and 8+4hh..+3 of that page).
      // ---- O^T += V^T P^T
#pragma unroll
      for (int pg = 0; pg < kPages; ++pg) {
        const uint4 pb = make_uint4(pw[4 * pg], pw[4 * pg + 1], pw[4 * pg + 2], pw[4 * pg + 3]);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const int d = dt * 32 + (lane & 31);
          // tokens 4hh..+3 (half 0, byte 8*hh) and 8+4hh..+3 (half 1, byte 8*hh)
          const uint2* r0 = reinterpret_cast<const uint2*>(&B.v[pg * 256 + d * 2 + vhalf(d, 0)]);
          const uint2* r1 = reinterpret_cast<const uint2*>(&B.v[pg * 256 + d * 2 + vhalf(d, 1)]);
          const uint2 lo = r0[hh], hi = r1[hh];
          o[dt] = mfma32(make_uint4(lo.x, lo.y, hi.x, hi.y), pb, o[dt]);
        }
      }
    }
  }

  if (!wave_active) return;
  const float lt = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (row0 + qn < n_q) {
    uint16_t* orow = out + (static_cast<int64_t>(q0 + row0 + qn) * num_heads + h) * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        uint2 w;
        w.x = pa::pack_bf16x2(o[dt][4 * jg] * inv, o[dt][4 * jg + 1] * inv);
        w.y = pa::pack_bf16x2(o[dt][4 * jg + 2] * inv, o[dt][4 * jg + 3] * inv);
        *reinterpret_cast<uint2*>(orow + dt * 32 + 8 * jg + 4 * hh) = w;
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
  const int64_t qtiles = (static_cast<int64_t>(max_query_len) + kRowsPerWG - 1) / kRowsPerWG;
  const int64_t wgs = qtiles * num_heads * num_seqs;
  const int64_t grid = (wgs + kXcds - 1) / kXcds * kXcds;
  if (grid > 0x7fffffffLL) return PA_ERR_INVALID_ARG;
  const float sl2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  hipLaunchKernelGGL(prefill_chunk_kernel, dim3(static_cast<uint32_t>(grid)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<uint16_t*>(out),
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cache),
                     static_cast<const uint16_t*>(v_cache), block_tables, max_blocks_per_seq,
                     query_start_loc, context_lens, num_seqs, num_heads, num_kv_heads,
                     static_cast<int32_t>(qtiles), sl2);
  return pa_launch_status();
}
