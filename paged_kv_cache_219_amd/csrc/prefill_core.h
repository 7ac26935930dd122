// Chunked prefill over a paged KV cache on gfx950 matrix cores: the body of
// one 128-row workgroup, shared by the prefill and mixed-batch kernels, and
// the helpers the 256-row ping-pong body (prefill_pingpong.h) also uses.
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
// Work decomposition.  A workgroup of W waves owns 32 W consecutive query rows
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
// uses the same token order.  O is rescaled only when a query's weight would
// exceed 2^8 against its reference (the exponentials then stay below 2^8, far
// inside fp32 and bf16 range; the final O / l is unchanged).
//
// The vector instructions per step are kept few, since a wave issues about
// one instruction every four to six cycles: copy and LDS addresses are
// per-lane constants plus a scalar per step, the block ids a wave copies are
// preloaded into its lanes, the row sums come from v_dot2 on the bf16
// weights (the values the products use), and the need to move a reference is
// read from those sums instead of from a row maximum.
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
constexpr float kMaxLaneSum = 256.f;  // 2^kLazyRescale
constexpr uint32_t kStepBytes = sizeof(StepBuf);  // 16 KB
constexpr uint32_t kVBytes = kStepBytes / 2;      // values follow the keys
constexpr uint32_t kOnesBf16x2 = 0x3f803f80u;     // two bf16 1.0

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ pa::f32x16_t mfma32(uint4 a, uint4 b, pa::f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ float swap32_max(float v) { return fmaxf(v, __shfl_xor(v, 32, 64)); }

__device__ __forceinline__ float max3(float a, float b, float c) {
  return __builtin_fmaxf(__builtin_fmaxf(a, b), c);
}

// Maximum of a lane's 16 scores.
__device__ __forceinline__ float max16(const float (&x)[16]) {
  return max3(max3(max3(x[0], x[1], x[2]), max3(x[3], x[4], x[5]), max3(x[6], x[7], x[8])),
              max3(x[9], x[10], x[11]), max3(max3(x[12], x[13], x[14]), x[15], x[15]));
}

// Zero the bf16 elements of a 16-byte value chunk whose token index (0..7
// within the chunk) is >= keep.
__device__ __forceinline__ uint4 keep_tokens(uint4 v, int keep) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] &= (2 * i < keep ? 0x0000ffffu : 0u) | (2 * i + 1 < keep ? 0xffff0000u : 0u);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// 16-byte direct-to-LDS load from the scalar base `sbase` plus the lane's
// 32-bit byte offset; lane i's bytes land at LDS address lds + 16 i.  The
// five wait states cover a scalar base written by a vector instruction.
__device__ __forceinline__ void dma16_sbase(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 4\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}

// Per-lane constants of one wave's work on the LDS ring: where its share of a
// step's copy comes from and lands, and where its MFMA operands sit in a step
// buffer.  A W-wave workgroup copies a step as 8 runs of 64 16-byte units
// (1 KB) of keys and 8 of values; wave w copies runs w * 8/W .. (w+1) * 8/W - 1,
// all within page page_of<W>(w) of the step.
template <int W>
struct RingLane {
  static constexpr int kRuns = 8 / W;
  uint32_t k_src[kRuns], v_src[kRuns];  // byte offsets within the source page
  uint32_t k_lo, k_hi, v_ln;            // operand byte offsets within a step buffer
  __device__ __forceinline__ RingLane(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < kRuns; ++i) {
      const int pos = (64 * (kRuns * wave + i) + lane) & 255;  // unit within the page
      const int c = pos >> 4, d = pos >> 1;
      k_src[i] = static_cast<uint32_t>((c * 16 + pa::ring::kslot(c, pos & 15)) * 16);
      v_src[i] = static_cast<uint32_t>((d * 2 + vhalf(d, pos & 1)) * 16);
    }
    // Row m of the K operand holds token krow(m) of the step (bits 2 and 3 of
    // m swapped), so the 16 accumulator rows of lane (q, hh) are 8
    // consecutive tokens of each page: the k-slots of the P^T operand.  Key
    // chunk c = 2 kk + hh of token t sits in unit (t / 16) 256 + 16 c +
    // (t % 16 ^ (c & 8)); the value half of dim d = 32 dt + m for tokens
    // 8 hh .. 8 hh + 7 of page pg in unit 256 pg + 2 d + (hh ^ bit 3 of d).
    const int m = lane & 31, hh = lane >> 5;
    const int ktok = (m & 0x13) | ((m & 4) << 1) | ((m & 8) >> 1);
    k_lo = static_cast<uint32_t>(((ktok >> 4) * 256 + 16 * hh + (ktok & 15)) * 16);
    k_hi = static_cast<uint32_t>(((ktok >> 4) * 256 + 16 * hh + ((ktok & 15) ^ 8)) * 16);
    v_ln = kVBytes + static_cast<uint32_t>((2 * m + (hh ^ ((m >> 3) & 1))) * 16);
  }
  // K operand kk (chunks 2 kk + hh) of the step buffer at `b`
  __device__ __forceinline__ uint4 k_op(const char* b, int kk) const {
    return *reinterpret_cast<const uint4*>(b + (kk < 4 ? k_lo : k_hi) + 512 * kk);
  }
  // V^T operand (page pg, dims 32 dt ..) of the step buffer at `b`
  __device__ __forceinline__ uint4 v_op(const char* b, int pg, int dt) const {
    return *reinterpret_cast<const uint4*>(b + v_ln + 4096 * pg + 1024 * dt);
  }
};

// Online softmax of one 32-token step for one lane (16 scores of its query
// column, x[i] = token 16 (i / 8) + 8 hh + i % 8 of the step): bf16 weights
// against the column's reference, the lane's sum of them, and the lazy move
// of the reference.  o are the column's output accumulators.
struct OnlineSoftmax {
  float m_run = -INFINITY, l_run = 0.f, neg_m = 0.f;  // neg_m: -m_run, or 0 while it is -inf
  bool have_ref = false;                              // wave-uniform

  __device__ __forceinline__ void weights(const float (&x)[16], float scale_log2,
                                          uint32_t (&pw)[8], float& ls) const {
    float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const float p0 = pa::fast_exp2(fmaf(x[i], scale_log2, neg_m));
      const float p1 = pa::fast_exp2(fmaf(x[i + 1], scale_log2, neg_m));
      pw[i >> 1] = pa::pack_bf16x2(p0, p1);
      if (i & 2) ls1 = pa::dot2_bf16(pw[i >> 1], kOnesBf16x2, ls1);
      else ls0 = pa::dot2_bf16(pw[i >> 1], kOnesBf16x2, ls0);
    }
    ls = ls0 + ls1;
  }

  // Weights of a step into pw; adds their sum to l_run.  The reference of a
  // column moves only when one of its weights would exceed 2^8 -- seen as a
  // lane's sum of 16 weights above 2^8, so no row maximum is needed on the
  // common path -- or before the first reference is set (wave-uniform
  // decision).  Then the two halves of each column combine their maxima, O and
  // l are rescaled, and the weights are recomputed.
  __device__ __forceinline__ void step(const float (&x)[16], float scale_log2, uint32_t (&pw)[8],
                                       pa::f32x16_t (&o)[4]) {
    float ls;
    weights(x, scale_log2, pw, ls);
    if (!have_ref || __any(!(ls <= kMaxLaneSum))) {
      const float m_new = fmaxf(m_run, swap32_max(max16(x)) * scale_log2);
      const float alpha = pa::fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] *= alpha;
      m_run = m_new;
      neg_m = m_new == -INFINITY ? 0.f : -m_new;
      have_ref = true;
      weights(x, scale_log2, pw, ls);
    }
    l_run += ls;
  }
};

// Workgroup `bid` of a grid of ceil(num_heads * num_seqs / 8) * 8 *
// num_qtiles, W * 64 threads (num_qtiles = ceil(max chunk / (32 W))).  The
// body of one workgroup; `bid` takes the place of the block index.
template <int W>
__device__ __forceinline__ void prefill_tile(
    uint32_t bid, StepBuf (&buf)[kRing], uint16_t* __restrict__ out,
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ qsl, const int32_t* __restrict__ context_lens, int32_t num_seqs,
    int32_t num_heads, int32_t num_kv_heads, int32_t num_qtiles, float scale_log2) {
  constexpr int kRowsPerWG = W * 32;
  using RL = RingLane<W>;

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
  // a length above the table row (a broken precondition) is cut to it
  const int L = min(context_lens[s], max_blocks * kBS);
  const int wg_row0 = qt * kRowsPerWG;
  if (wg_row0 >= n_q) return;  // whole workgroup idle
  const int first_pos = L - n_q;                  // position of chunk row 0
  const int wg_last = first_pos + min(wg_row0 + kRowsPerWG, n_q) - 1;
  const int nsteps = wg_last / kStep + 1;         // steps covering tokens 0 .. wg_last

  const int row0 = wg_row0 + wave * 32;
  const bool wave_active = row0 < n_q;
  const int qn = lane & 31;   // this lane's query column
  const int hh = lane >> 5;   // which half of the accumulator rows
  const int wave_last = first_pos + min(row0 + 32, n_q) - 1;
  const int wave_first = first_pos + row0;
  const int my_row = min(row0 + qn, n_q - 1);
  const int my_pos = first_pos + my_row;

  // Q^T operand: lane (qn, hh) holds dims 16 kk + 8 hh .. + 7 of its row.
  uint4 qreg[8];
  {
    const uint16_t* qrow = q + (static_cast<int64_t>(q0 + my_row) * num_heads + h) * kD + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qreg[kk] = *reinterpret_cast<const uint4*>(qrow + 16 * kk);
  }

  // Block ids of this wave's page of each step, preloaded into lanes: lane i
  // holds step i's and step 64 + i's.  Pages past the last needed token name
  // logical block 0 (always valid): their scores are masked and their values
  // weighted by 0.
  const int32_t* bt_row = block_tables + static_cast<int64_t>(s) * max_blocks;
  const int pw_page = pa::ring::page_of<W>(wave);
  auto page_index = [&](int st) {
    const int lb = st * kPages + pw_page;
    return st < nsteps && lb * kBS <= wg_last ? lb : 0;
  };
  const int ids_lo = bt_row[page_index(lane)];
  const int ids_hi = bt_row[page_index(lane + 64)];
  // Consume the query registers and block ids before the copies are issued:
  // the compiler does not count the copies (inline asm), so a wait for these
  // loads placed at their first use would drain every copy in flight.
#pragma unroll
  for (int kk = 0; kk < 8; ++kk)
    asm volatile("" : "+v"(qreg[kk].x), "+v"(qreg[kk].y), "+v"(qreg[kk].z), "+v"(qreg[kk].w));
  asm volatile("" ::"v"(ids_lo), "v"(ids_hi));

  const RL rl(wave, lane);
  const int64_t page_bytes = static_cast<int64_t>(kPageElems) * 2;
  const int64_t blk_bytes = static_cast<int64_t>(num_kv_heads) * page_bytes;
  const int64_t head_bytes = static_cast<int64_t>(g) * page_bytes;
  const uint32_t ring_lds = pa::ring::lds_addr(&buf[0]);
  const char* lds = reinterpret_cast<const char*>(&buf[0]);
  const char* kc_b = reinterpret_cast<const char*>(kc);
  const char* vc_b = reinterpret_cast<const char*>(vc);
  auto issue = [&](int step) {
    const int phys = step < 64    ? __builtin_amdgcn_readlane(ids_lo, step)
                     : step < 128 ? __builtin_amdgcn_readlane(ids_hi, step - 64)
                                  : bt_row[page_index(step)];
    const int64_t src = static_cast<int64_t>(phys) * blk_bytes + head_bytes;
    const uint32_t dst = ring_lds + static_cast<uint32_t>(step % kRing) * kStepBytes;
#pragma unroll
    for (int i = 0; i < RL::kRuns; ++i) {
      const uint32_t u0 = 64u * static_cast<uint32_t>(RL::kRuns * wave + i);
      dma16_sbase(kc_b + src, rl.k_src[i], dst + 16 * u0);
      dma16_sbase(vc_b + src, rl.v_src[i], dst + kVBytes + 16 * u0);
    }
  };

  pa::f32x16_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pa::f32x16_t{};
  OnlineSoftmax sm;

  auto step_compute = [&](int step) {
    const char* b = lds + static_cast<uint32_t>(step % kRing) * kStepBytes;
    const int t0 = step * kStep;
    // ---- S^T = K Q^T
    pa::f32x16_t sa = pa::f32x16_t{};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) sa = mfma32(rl.k_op(b, kk), qreg[kk], sa);
    // ---- online softmax: lane (qn, hh) element i is token
    // t0 + 16 (i / 8) + 8 hh + i % 8 of query row row0 + qn
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = sa[i];
    const bool tail = t0 + kStep > L;
    if (t0 + kStep - 1 > wave_first || tail) {  // diagonal or tail step
      const int lim = min(my_pos, L - 1) - t0 - 8 * hh;  // keep offsets <= lim
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (16 * (i >> 3) + (i & 7) > lim) x[i] = -INFINITY;
    }
    uint32_t pw[8];
    sm.step(x, scale_log2, pw, o);
    // ---- O^T += V^T P^T; values of tokens at or past L may be anything
    // (0 * NaN): zeroed in registers
#pragma unroll
    for (int pg = 0; pg < kPages; ++pg) {
      const uint4 pb = make_uint4(pw[4 * pg], pw[4 * pg + 1], pw[4 * pg + 2], pw[4 * pg + 3]);
      const int keep = L - (t0 + 16 * pg + 8 * hh);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        uint4 va = rl.v_op(b, pg, dt);
        if (tail && keep < 8) va = keep_tokens(va, keep);
        o[dt] = mfma32(va, pb, o[dt]);
      }
    }
  };

  for (int st = 0; st < kRing - 1 && st < nsteps; ++st) issue(st);
  for (int step = 0; step < nsteps; ++step) {
    // wait for this wave's copies of this step (later steps may stay in
    // flight), then for everyone's
    pa::ring::wait_step<kRing, W>(min(kRing - 2, nsteps - 1 - step));
    // the buffer written next was last read in the previous step, which every
    // wave has finished (barrier above)
    if (step + kRing - 1 < nsteps) issue(step + kRing - 1);
    if (wave_active && step * kStep <= wave_last) step_compute(step);
  }

  if (!wave_active) return;
  const float lt = sm.l_run + __shfl_xor(sm.l_run, 32, 64);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const int row = row0 + qn;
  if (row < n_q) {
    uint16_t* orow = out + (static_cast<int64_t>(q0 + row) * num_heads + h) * kD;
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
