// Chunked prefill over a paged KV cache on gfx950 matrix cores: the body of
// one workgroup, shared by the prefill and mixed-batch kernels.
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
// pages are copied once, cooperatively, into a ring of three LDS step buffers
// with direct-to-LDS loads issued two steps ahead of use, then every wave
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

#pragma once

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
constexpr uint32_t kXcds = 8;
constexpr float kLazyRescale = 8.f;   // log2 units

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ pa::f32x16_t mfma32(uint4 a, uint4 b, pa::f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ float swap32_max(float v) { return fmaxf(v, __shfl_xor(v, 32, 64)); }

// Workgroup `bid` of a grid of ceil(num_heads * num_seqs / 8) * 8 *
// num_qtiles, W * 64 threads.  W waves per workgroup, NB blocks of 32 query
// rows per wave (every K and V operand read from LDS feeds NB matrix products).
// The body of one workgroup; `bid` takes the place of the block index.
template <int W, int NB>
__device__ __forceinline__ void prefill_tile(
    uint32_t bid, StepBuf (&buf)[kRing], uint16_t* __restrict__ out,
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ qsl, const int32_t* __restrict__ context_lens, int32_t num_seqs,
    int32_t num_heads, int32_t num_kv_heads, int32_t num_qtiles, float scale_log2) {
  constexpr int kRowsPerWave = 32 * NB;
  constexpr int kRowsPerWG = W * kRowsPerWave;

  const int tid = threadIdx.x;
  const int lane = tid & 63;

  // Order of work.  A unit is one (sequence, head); its q-tiles share the
  // unit's K/V pages.  Units run longest first (when there are at most 64
  // sequences, every workgroup ranks them by their number of steps; heads of
  // a sequence are equal), so the longest workgroups do not start last and
  // leave the chip idle behind them.  Unit u runs on XCD u % 8 and its q-tiles
  // are consecutive there (dispatch sends workgroup b to XCD b % 8), so they
  // are in flight together and read the unit's pages from HBM once, through
  // that XCD's L2.
  const uint32_t xcd = bid % kXcds, k = bid / kXcds;
  const uint32_t u = (k / num_qtiles) * kXcds + xcd;
  const int qt = num_qtiles - 1 - static_cast<int>(k % num_qtiles);  // long q-tiles first
  if (u >= static_cast<uint32_t>(num_seqs) * num_heads) return;  // grid padding
  const int h = static_cast<int>(u % static_cast<uint32_t>(num_heads));
  const int rank = static_cast<int>(u / static_cast<uint32_t>(num_heads));
  int s = rank;
  if (num_seqs <= 64) {
    int work = -1;
    if (lane < num_seqs) {
      const int Li = context_lens[lane], nqi = qsl[lane + 1] - qsl[lane];
      work = 0;
      for (int t = 0; t < num_qtiles && t * kRowsPerWG < nqi; ++t)
        work += (Li - nqi + min((t + 1) * kRowsPerWG, nqi) - 1) / kStep + 1;
    }
    int my_rank = 0;
    for (int j = 0; j < num_seqs; ++j) {
      const int wj = __builtin_amdgcn_readlane(work, j);
      my_rank += (wj > work) || (wj == work && j < lane);
    }
    s = __builtin_ctzll(__ballot(lane < num_seqs && my_rank == rank));
  }

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
  const int qn = lane & 31;   // this lane's query column within a block
  const int hh = lane >> 5;   // which half of the accumulator rows
  const int wave_last = first_pos + min(row0 + kRowsPerWave, n_q) - 1;
  const int wave_first = first_pos + row0;
  int my_pos[NB];

  // Q^T operands: lane (qn, hh) holds dims 16*kk + 8*hh .. +7 of its query
  // row in each block.
  uint4 qreg[NB][8];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int my_row = min(row0 + 32 * b + qn, n_q - 1);
    my_pos[b] = first_pos + my_row;
    const uint16_t* qrow = q + (static_cast<int64_t>(q0 + my_row) * num_heads + h) * kD + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qreg[b][kk] = *reinterpret_cast<const uint4*>(qrow + 16 * kk);
  }
  // Consume the query registers here: otherwise their load waits land in the
  // step loop, where (loads retiring in order) they would also drain every
  // step copy in flight.
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      asm volatile("" : "+v"(qreg[b][kk].x), "+v"(qreg[b][kk].y), "+v"(qreg[b][kk].z),
                   "+v"(qreg[b][kk].w));

  const int32_t* bt_row = block_tables + static_cast<int64_t>(s) * max_blocks;
  const int64_t blk_stride = static_cast<int64_t>(num_kv_heads) * kPageElems;
  const int64_t head_off = static_cast<int64_t>(g) * kPageElems;

  // Pages past the last needed token load logical block 0 instead (always
  // valid): their scores are masked, and their values must just be finite.
  auto issue = [&](int step) {
    const int lb = step * kPages + pa::ring::page_of<W>(wave);
    pa::ring::issue_step<W>(buf[step % kRing], kc, vc, bt_row[lb * kBS <= wg_last ? lb : 0],
                            blk_stride, head_off, wave, lane);
  };
  // Values of tokens at or past L in the step's last page: zero them in LDS
  // (the cache may hold NaN there, and 0 * NaN would reach every query).
  auto zero_tail = [&](int step) {
    StepBuf& B = buf[step % kRing];
#pragma unroll
    for (int r = 0; r < 512 / (W * 64); ++r) {
      const int row = tid + W * 64 * r;   // (page, dim) row, 2 units each
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

  pa::f32x16_t o[NB][4];
  float m_run[NB], l_run[NB], neg_m[NB];  // neg_m: -m_run, or 0 while m_run is -inf
#pragma unroll
  for (int b = 0; b < NB; ++b) {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[b][i] = pa::f32x16_t{};
    m_run[b] = -INFINITY;
    l_run[b] = 0.f;
    neg_m[b] = 0.f;
  }

  // Row m of the K operand (and of S^T) holds token krow(m) of the step: m
  // with bits 2 and 3 swapped.  Then the 16 accumulator rows of lane (q, hh)
  // -- rows 8*(j/4) + 4*hh + j%4 -- are tokens 16*(j/8) + 8*hh + j%8, i.e.
  // 8 consecutive tokens of each page, exactly the k-slots 8*hh..8*hh+7 of
  // the PV product's P^T operand; so the matching V^T operand is one 16-byte
  // half row of the d-major value page.
  const int m_row = lane & 31;
  const int ktok = (m_row & 0x13) | ((m_row & 4) << 1) | ((m_row & 8) >> 1);

  auto step_compute = [&](int step) {
    const StepBuf& B = buf[step % kRing];
    const int t0 = step * kStep;
    // ---- S^T = K Q^T, each K operand feeding every block
    pa::f32x16_t sa[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) sa[b] = pa::f32x16_t{};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int c = 2 * kk + hh;
      const uint4 a0 = B.k[((ktok >> 4) * 16 + c) * 16 + pa::ring::kslot(c, ktok & 15)];
#pragma unroll
      for (int b = 0; b < NB; ++b) sa[b] = mfma32(a0, qreg[b][kk], sa[b]);
    }
    // ---- online softmax per block: lane (qn, hh) element j is token
    // t0 + 16*(j/8) + 8*hh + j%8 of query row 32*b + qn
    uint4 pb[NB][kPages];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float x[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) x[j] = sa[b][j];
      if (t0 + kStep - 1 > wave_first + 32 * b || t0 + kStep > L) {  // diagonal or tail step
        const int lim = min(my_pos[b], L - 1) - t0 - 8 * hh;         // keep offsets <= lim
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int off = 16 * (j >> 3) + (j & 7);
          if (off > lim) x[j] = -INFINITY;
        }
      }
      float mx = fmaxf(x[0], x[1]);
#pragma unroll
      for (int j = 2; j < 16; j += 2) mx = fmaxf(mx, fmaxf(x[j], x[j + 1]));
      // Lazy rescale, wave-uniform: only when some query's score exceeds its
      // reference by more than 2^8 (scale > 0: max commutes with it).  Only
      // then are the two halves of each query column combined.
      if (__any(mx * scale_log2 > m_run[b] + kLazyRescale)) {
        const float m_new = fmaxf(m_run[b], swap32_max(mx) * scale_log2);
        const float alpha = pa::fast_exp2(m_run[b] - m_new);
        l_run[b] *= alpha;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[b][i] *= alpha;
        m_run[b] = m_new;
        neg_m[b] = m_new == -INFINITY ? 0.f : -m_new;
      }
      uint32_t pw[8];
      float ls = 0.f;
#pragma unroll
      for (int j = 0; j < 16; j += 2) {
        const float p0 = pa::fast_exp2(fmaf(x[j], scale_log2, neg_m[b]));
        const float p1 = pa::fast_exp2(fmaf(x[j + 1], scale_log2, neg_m[b]));
        ls += p0 + p1;
        pw[j >> 1] = pa::pack_bf16x2(p0, p1);
      }
      l_run[b] += ls;
      // P^T operands, one per page: elements 8*pg .. 8*pg+7 are tokens
      // 8*hh .. 8*hh+7 of page pg.
#pragma unroll
      for (int pg = 0; pg < kPages; ++pg)
        pb[b][pg] = make_uint4(pw[4 * pg], pw[4 * pg + 1], pw[4 * pg + 2], pw[4 * pg + 3]);
    }
    // ---- O^T += V^T P^T, each V operand feeding every block
#pragma unroll
    for (int pg = 0; pg < kPages; ++pg) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const int d = dt * 32 + (lane & 31);
        const uint4 va = B.v[pg * 256 + d * 2 + vhalf(d, hh)];
#pragma unroll
        for (int b = 0; b < NB; ++b) o[b][dt] = mfma32(va, pb[b][pg], o[b][dt]);
      }
    }
  };

  for (int st = 0; st < kRing - 1 && st < nsteps; ++st) issue(st);
  for (int step = 0; step < nsteps; ++step) {
    // wait for this wave's copies of this step (later steps may stay in
    // flight), then for everyone's
    pa::ring::wait_step<kRing, W>(min(kRing - 2, nsteps - 1 - step));
    if (step * kStep + kStep > L) {  // the step holding the sequence's last token
      zero_tail(step);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
    // the buffer written next was last read in the previous step, which every
    // wave has finished (barrier above)
    if (step + kRing - 1 < nsteps) issue(step + kRing - 1);
    if (wave_active && step * kStep <= wave_last) step_compute(step);
  }

  if (!wave_active) return;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const float lt = l_run[b] + __shfl_xor(l_run[b], 32, 64);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int row = row0 + 32 * b + qn;
    if (row < n_q) {
      uint16_t* orow = out + (static_cast<int64_t>(q0 + row) * num_heads + h) * kD;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int jg = 0; jg < 4; ++jg) {
          uint2 w;
          w.x = pa::pack_bf16x2(o[b][dt][4 * jg] * inv, o[b][dt][4 * jg + 1] * inv);
          w.y = pa::pack_bf16x2(o[b][dt][4 * jg + 2] * inv, o[b][dt][4 * jg + 3] * inv);
          *reinterpret_cast<uint2*>(orow + dt * 32 + 8 * jg + 4 * hh) = w;
        }
    }
  }
}

}  // namespace
