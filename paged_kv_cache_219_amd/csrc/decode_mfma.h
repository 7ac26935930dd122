// Decode of several query rows against one kv head's paged K/V on the matrix
// cores, one wave, no LDS (gfx950; bf16, head_dim 128, 16-token blocks).
//
// Page "vLLM PagedAttention chuyên sâu: Phân mảnh bộ nhớ KV Cache, Prefill
// theo khối & Prefix Caching" (locionic.com), section "Cơ chế PagedAttention":
// look up the physical blocks in the block table, gather K and V, attend.
//
// With n (up to 32) query rows on one kv head -- the samples of a prompt over
// their shared prefix (mfma_decode_range), or the 4 or 8 query heads of a
// grouped-query group (mfma16_decode_range, the same scheme on 16 columns
// with 16 x 16 x 32 instructions) -- a 32-token step is a small dense
// contraction, computed in the same transposed form as the chunked-prefill
// kernel:
//   S^T[32 tokens x 32 columns] = K Q^T    (8 x v_mfma_f32_32x32x16_bf16)
//   O^T[128 dims x 32 columns] += V^T P^T  (8 more)
// Column q is query row q (columns past n compute a copy of the last row and
// are never written).  Both matrix operands that change per step come
// straight from global memory into registers in operand layout: lane (m, hh)
// of the K operand loads the 16-byte key chunk 2 kk + hh of token krow(m) --
// one load per MFMA -- and lane (m, hh) of the V^T operand loads tokens
// 8 hh .. 8 hh + 7 of value row m of the d-major page.  There is no LDS
// staging, no barrier and almost no VALU work per byte; the wave keeps the
// next step's keys and values in flight while it computes, and many waves per
// CU keep HBM busy.
//
// Softmax per column, as in prefill: each lane owns 16 scores of one column,
// the two lanes of a column exchange maxima only when a score exceeds the
// column's reference by more than 2^8 (then the reference moves and O and l
// are rescaled); the weights are 2^(s * scale - reference).
#pragma once

#include "decode_core.h"
#include "prefill_core.h"

namespace {

// Attention of query rows 0..nq-1 (nq <= 32) over tokens [part_start,
// part_end) of one block-table row, kv head g.  qrow_of(i) is row i's query
// (128 bf16); dest_of(i, out_off, part_row) says where its result goes: the
// output row at element offset out_off (>= 0), or partial row part_row (>= 0)
// of the workspace.  part_start is a multiple of 16.
template <bool NT, typename QRow, typename Dest>
__device__ __forceinline__ void mfma_decode_range(
    uint16_t* __restrict__ out, Partials ws, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ bt_row, int32_t num_kv_heads,
    int g, int part_start, int part_end, float scale_log2, int nq, QRow qrow_of, Dest dest_of) {
  const int lane = threadIdx.x & 63;
  const int qn = lane & 31;  // this lane's column
  const int hh = lane >> 5;  // which half of the accumulator rows
  const int nsteps = (part_end - part_start + kStep - 1) / kStep;
  const int npages = (part_end - part_start + kBS - 1) / kBS;
  const int lb0 = part_start / kBS;

  // Q^T operand: dims 16 kk + 8 hh .. +7 of this lane's column's query
  uint4 qreg[8];
  {
    const uint16_t* qrow = qrow_of(min(qn, nq - 1)) + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qreg[kk] = *reinterpret_cast<const uint4*>(qrow + 16 * kk);
  }
  int ids = bt_row[lb0 + min(lane, npages - 1)];  // block ids of the first 64 pages
  auto page = [&](int pi) -> int {                // block id of page pi of the range
    return pi < 64 ? __builtin_amdgcn_readlane(ids, pi) : bt_row[lb0 + pi];
  };

  const int64_t blk_stride = static_cast<int64_t>(num_kv_heads) * kPageElems;
  const int64_t head_off = static_cast<int64_t>(g) * kPageElems;
  // Row m of the K operand holds token krow(m) of the step (bits 2 and 3 of m
  // swapped), so that the 16 accumulator rows of lane (q, hh) are tokens
  // 16 (j / 8) + 8 hh + j % 8 -- 8 consecutive tokens of each page, the
  // k-slots of the P^T operand.
  const int m_row = lane & 31;
  const int ktok = (m_row & 0x13) | ((m_row & 4) << 1) | ((m_row & 8) >> 1);
  const int kofs = ((2 * 0 + hh) * kBS + (ktok & 15)) * 8;  // chunk hh of token ktok, kk = 0

  // two key buffers: the keys of step s + 2 are fetched as soon as step s's
  // scores are done, so they have a step and a half to arrive
  uint4 kreg0[8], kreg1[8], vreg[2][4];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) kreg0[kk] = kreg1[kk] = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int pg = 0; pg < 2; ++pg)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) vreg[pg][dt] = make_uint4(0, 0, 0, 0);

  // Pages past the end are not loaded: their keys' scores are masked and
  // their weights are 0 against finite stale values.
  auto load_k = [&](int step, int ofs, uint4 (&kreg)[8]) {
    const int pi = 2 * step + (ktok >> 4);
    const int phys0 = page(2 * step);
    const int phys1 = 2 * step + 1 < npages ? page(2 * step + 1) : phys0;
    const int phys = (ktok >> 4) ? phys1 : phys0;
    if (pi < npages) {
      const uint16_t* base = kc + phys * blk_stride + head_off + ofs;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)  // chunk 2 kk + hh
        kreg[kk] = pa::ld16_kv<NT>(base + kk * 2 * kBS * 8);
    }
  };
  auto load_v = [&](int step, int ofs) {
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
      if (2 * step + pg < npages) {
        const uint16_t* base = vc + page(2 * step + pg) * blk_stride + head_off + ofs;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)  // value row dt * 32 + m_row, tokens 8 hh ..
          vreg[pg][dt] = pa::ld16_kv<NT>(base + dt * 32 * kBS);
      }
    }
  };

  pa::f32x16_t o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = pa::f32x16_t{};
  float m_run = -INFINITY, l_run = 0.f, neg_m = 0.f;

  const int vofs = m_row * kBS + 8 * hh;
  load_k(0, kofs, kreg0);
  load_v(0, vofs);
  if (nsteps > 1) load_k(1, kofs, kreg1);
  auto body = [&](int step, uint4 (&kreg)[8]) {
    const int t0 = part_start + step * kStep;
    const bool more = step + 1 < nsteps;
    // ---- S^T = K Q^T
    pa::f32x16_t sa = pa::f32x16_t{};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) sa = mfma32(kreg[kk], qreg[kk], sa);
    if (step + 2 < nsteps) {  // this key buffer is free again: fetch step + 2's keys
      int ofs = kofs;
      asm volatile("" : "+v"(ofs) : "v"(sa[15]));
      load_k(step + 2, ofs, kreg);
    }
    // ---- softmax of this lane's 16 scores (tokens t0 + 16 (j / 8) + 8 hh + j % 8)
    float x[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = sa[j];
    const bool tail = t0 + kStep > part_end;
    if (tail) {
      const int lim = part_end - 1 - t0 - 8 * hh;
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (16 * (j >> 3) + (j & 7) > lim) x[j] = -INFINITY;
    }
    float mx = fmaxf(x[0], x[1]);
#pragma unroll
    for (int j = 2; j < 16; j += 2) mx = fmaxf(mx, fmaxf(x[j], x[j + 1]));
    if (__any(mx * scale_log2 > m_run + kLazyRescale)) {
      const float m_new = fmaxf(m_run, swap32_max(mx) * scale_log2);
      const float alpha = pa::fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
      m_run = m_new;
      neg_m = m_new == -INFINITY ? 0.f : -m_new;
    }
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
    // values of tokens past the end may be anything (0 * NaN): zero them
    if (tail) {
#pragma unroll
      for (int pg = 0; pg < 2; ++pg) {
        const int keep = part_end - (t0 + 16 * pg + 8 * hh);
        if (keep < 8) {
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) vreg[pg][dt] = mask_chunk<uint16_t>(vreg[pg][dt], keep);
        }
      }
    }
    // ---- O^T += V^T P^T
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
      const uint4 pb = make_uint4(pw[4 * pg], pw[4 * pg + 1], pw[4 * pg + 2], pw[4 * pg + 3]);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] = mfma32(vreg[pg][dt], pb, o[dt]);
    }
    if (more) {  // the value registers are free again
      int ofs = vofs;
      asm volatile("" : "+v"(ofs) : "v"(o[3][15]));
      load_v(step + 1, ofs);
    }
  };
  for (int step = 0; step < nsteps; step += 2) {
    body(step, kreg0);
    if (step + 1 < nsteps) body(step + 1, kreg1);
  }

  // ---- write this lane's column: 4 runs of 4 dims per accumulator
  const float lt = l_run + __shfl_xor(l_run, 32, 64);
  if (qn >= nq) return;
  int64_t out_off, part_row;
  dest_of(qn, out_off, part_row);
  const float inv = 1.f / lt;
  if (out_off >= 0) {
    uint16_t* orow = out + out_off;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        uint2 w;
        w.x = pa::pack_bf16x2(o[dt][4 * jg] * inv, o[dt][4 * jg + 1] * inv);
        w.y = pa::pack_bf16x2(o[dt][4 * jg + 2] * inv, o[dt][4 * jg + 3] * inv);
        *reinterpret_cast<uint2*>(orow + dt * 32 + 8 * jg + 4 * hh) = w;
      }
  } else if (part_row >= 0) {
    float* prow = ws.o + part_row * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg)
        *reinterpret_cast<float4*>(prow + dt * 32 + 8 * jg + 4 * hh) =
            make_float4(o[dt][4 * jg] * inv, o[dt][4 * jg + 1] * inv, o[dt][4 * jg + 2] * inv,
                        o[dt][4 * jg + 3] * inv);
    if (hh == 0) {
      ws.ml[2 * part_row] = m_run;
      ws.ml[2 * part_row + 1] = lt;
    }
  }
}

// The same attention for up to 16 query rows on v_mfma_f32_16x16x32_bf16: 16
// columns instead of 32 halve the query operand, the scores, the output
// accumulators and the matrix work (the grouped-query groups have 4 or 8
// rows, so 32 columns computed copies).  KB steps of keys and VB steps of
// values stay in flight per wave.
//
// Layout of a 32-token step (two pages).  Lane l = (qn = l % 16, q4 = l / 16).
//  * Scores, two 16 x 16 tiles S_i = K_i Q^T (4 instructions each, 32 dims
//    per instruction).  Row r of tile i is token (r & 7) + 8 i of page r / 8,
//    so each key load is whole 128-byte lines (8 tokens of a 16-byte chunk),
//    and lane (qn, q4) gets the scores of tokens a .. a+3 (tile 0) and
//    a+8 .. a+11 (tile 1), a = 4 q4 + 8 (q4 / 2), of column qn.
//  * Weights: lanes q4 and q4 ^ 1 trade one half, so lane (qn, q4) holds
//    tokens 8 q4 .. 8 q4 + 7 -- the k-slots of the P^T operand, and 16
//    contiguous bytes of one value row of the d-major page.
//  * O^T (128 dims x 16 columns) += V^T P^T: 8 instructions, tile dt's lane
//    (m, q4) holding dims 16 dt + m of tokens 8 q4 .. 8 q4 + 7.
// Softmax is the lazy scheme of the 32-wide body, with a column's 4 lanes
// exchanging maxima (xor 16, xor 32) only when a score passes the column's
// reference by more than 2^8.
__device__ __forceinline__ pa::f32x4_t mfma16(uint4 a, uint4 b, pa::f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

template <bool NT, int KB, int VB, typename QRow, typename Dest>
__device__ __forceinline__ void mfma16_decode_range(
    uint16_t* __restrict__ out, Partials ws, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ bt_row, int32_t num_kv_heads,
    int g, int part_start, int part_end, float scale_log2, int nq, QRow qrow_of, Dest dest_of) {
  static_assert(KB >= 2 && VB >= 1, "at least two key buffers and one value buffer");
  constexpr int U = (KB % VB == 0) ? KB : (VB % KB == 0 ? VB : KB * VB);  // buffers cycle
  const int lane = threadIdx.x & 63;
  const int qn = lane & 15;  // this lane's column
  const int q4 = lane >> 4;
  const int nsteps = (part_end - part_start + kStep - 1) / kStep;
  const int npages = (part_end - part_start + kBS - 1) / kBS;
  const int lb0 = part_start / kBS;

  // Q^T operand: dims 32 kk + 8 q4 .. +7 of this lane's column's query
  uint4 qreg[4];
  {
    const uint16_t* qrow = qrow_of(min(qn, nq - 1)) + 8 * q4;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qreg[kk] = *reinterpret_cast<const uint4*>(qrow + 32 * kk);
  }
  int ids = bt_row[lb0 + min(lane, npages - 1)];  // block ids of the first 64 pages
  auto page = [&](int pi) -> int {                // block id of page pi of the range
    return pi < 64 ? __builtin_amdgcn_readlane(ids, pi) : bt_row[lb0 + pi];
  };

  const int64_t blk_stride = static_cast<int64_t>(num_kv_heads) * kPageElems;
  const int64_t head_off = static_cast<int64_t>(g) * kPageElems;
  const int m = lane & 15;
  // key lane offset: chunk q4 (+ 4 kk) of token (m & 7) (+ 8 i) of page m / 8
  const int kofs = (q4 * kBS + (m & 7)) * 8;
  // value lane offset: dim m (+ 16 dt), tokens 8 (q4 & 1) .. +7 of page q4 / 2
  const int vofs = m * kBS + 8 * (q4 & 1);

  uint4 kbuf[KB][8], vbuf[VB][8];
#pragma unroll
  for (int b = 0; b < KB; ++b)
#pragma unroll
    for (int i = 0; i < 8; ++i) kbuf[b][i] = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int b = 0; b < VB; ++b)
#pragma unroll
    for (int i = 0; i < 8; ++i) vbuf[b][i] = make_uint4(0, 0, 0, 0);

  // Pages past the end are not loaded: their scores are masked and their
  // weights are 0 against values zeroed before use.
  // the step's two block ids (wave-uniform), then this lane's
  auto step_page = [&](int step, bool second) -> int {
    const int phys0 = page(2 * step);
    const int phys1 = 2 * step + 1 < npages ? page(2 * step + 1) : phys0;
    return second ? phys1 : phys0;
  };
  auto load_k = [&](int step, int ofs, uint4 (&kreg)[8]) {
    const int phys = step_page(step, m >> 3);
    if (2 * step + (m >> 3) < npages) {
      const uint16_t* base = kc + phys * blk_stride + head_off + ofs;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)  // chunk 4 kk + q4, token (m & 7) + 8 i
          kreg[4 * i + kk] = pa::ld16_kv<NT>(base + kk * 4 * kBS * 8 + i * 8 * 8);
    }
  };
  auto load_v = [&](int step, int ofs, uint4 (&vreg)[8]) {
    const int phys = step_page(step, q4 >> 1);
    if (2 * step + (q4 >> 1) < npages) {
      const uint16_t* base = vc + phys * blk_stride + head_off + ofs;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) vreg[dt] = pa::ld16_kv<NT>(base + dt * 16 * kBS);
    }
  };

  pa::f32x4_t o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = pa::f32x4_t{};
  float m_run = -INFINITY, l_run = 0.f, neg_m = 0.f;
  const int a0 = 4 * q4 + 8 * (q4 >> 1);  // first token of this lane's tile-0 scores

#pragma unroll
  for (int b = 0; b < KB; ++b)
    if (b < nsteps) load_k(b, kofs, kbuf[b]);
#pragma unroll
  for (int b = 0; b < VB; ++b)
    if (b < nsteps) load_v(b, vofs, vbuf[b]);

  auto body = [&](int step, uint4 (&kreg)[8], uint4 (&vreg)[8]) {
    const int t0 = part_start + step * kStep;
    // ---- S_i = K_i Q^T
    pa::f32x4_t s0 = pa::f32x4_t{}, s1 = pa::f32x4_t{};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      s0 = mfma16(kreg[kk], qreg[kk], s0);
      s1 = mfma16(kreg[4 + kk], qreg[kk], s1);
    }
    if (step + KB < nsteps) {  // this key buffer is free again
      int ofs = kofs;
      asm volatile("" : "+v"(ofs) : "v"(s1[3]));
      load_k(step + KB, ofs, kreg);
    }
    // ---- softmax of this lane's 8 scores: tokens a0 .. a0+3 and a0+8 .. a0+11
    float x[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] = s0[j];
      x[4 + j] = s1[j];
    }
    const bool tail = t0 + kStep > part_end;
    if (tail) {
      const int lim = part_end - 1 - t0 - a0;  // last valid token, relative to a0
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (j > lim) x[j] = -INFINITY;
        if (8 + j > lim) x[4 + j] = -INFINITY;
      }
    }
    float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                     fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    if (__any(mx * scale_log2 > m_run + kLazyRescale)) {
      float cm = fmaxf(mx, __shfl_xor(mx, 16, 64));
      cm = fmaxf(cm, __shfl_xor(cm, 32, 64));
      const float m_new = fmaxf(m_run, cm * scale_log2);
      const float alpha = pa::fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
      m_run = m_new;
      neg_m = m_new == -INFINITY ? 0.f : -m_new;
    }
    uint32_t pw[4];  // tokens a0 .. a0+3, then a0+8 .. a0+11
    float ls = 0.f;
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      const float p0 = pa::fast_exp2(fmaf(x[j], scale_log2, neg_m));
      const float p1 = pa::fast_exp2(fmaf(x[j + 1], scale_log2, neg_m));
      ls += p0 + p1;
      pw[j >> 1] = pa::pack_bf16x2(p0, p1);
    }
    l_run += ls;
    // lanes q4 and q4 ^ 1 trade halves: even q4 keeps its first half and takes
    // the partner's, odd q4 takes the partner's second half before its own
    const bool odd = q4 & 1;
    const uint32_t s_lo = odd ? pw[0] : pw[2], s_hi = odd ? pw[1] : pw[3];
    const uint32_t r_lo = __shfl_xor(s_lo, 16, 64), r_hi = __shfl_xor(s_hi, 16, 64);
    const uint4 pb = odd ? make_uint4(r_lo, r_hi, pw[2], pw[3]) : make_uint4(pw[0], pw[1], r_lo, r_hi);
    // values of tokens past the end may be anything (0 * NaN): zero them
    if (tail) {
      const int keep = part_end - (t0 + 8 * q4);
      if (keep < 8) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) vreg[dt] = mask_chunk<uint16_t>(vreg[dt], keep);
      }
    }
    // ---- O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] = mfma16(vreg[dt], pb, o[dt]);
    if (step + VB < nsteps) {  // this value buffer is free again
      int ofs = vofs;
      asm volatile("" : "+v"(ofs) : "v"(o[7][3]));
      load_v(step + VB, ofs, vreg);
    }
  };
  for (int step = 0; step < nsteps; step += U) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (step + u < nsteps) body(step + u, kbuf[u % KB], vbuf[u % VB]);
  }

  // ---- write this lane's column: dims 16 dt + 4 q4 .. +3
  float lt = l_run + __shfl_xor(l_run, 16, 64);
  lt += __shfl_xor(lt, 32, 64);
  if (qn >= nq) return;
  int64_t out_off, part_row;
  dest_of(qn, out_off, part_row);
  const float inv = 1.f / lt;
  if (out_off >= 0) {
    uint16_t* orow = out + out_off + 4 * q4;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      uint2 w;
      w.x = pa::pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv);
      w.y = pa::pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv);
      *reinterpret_cast<uint2*>(orow + 16 * dt) = w;
    }
  } else if (part_row >= 0) {
    float* prow = ws.o + part_row * kD + 4 * q4;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      *reinterpret_cast<float4*>(prow + 16 * dt) =
          make_float4(o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv);
    if (q4 == 0) {
      ws.ml[2 * part_row] = m_run;
      ws.ml[2 * part_row + 1] = lt;
    }
  }
}

// Steps of keys and of values a grouped-query wave keeps in flight.  Two and
// one (214 registers); two and two (245) and three and one (243) measured no
// faster on the 256-sequence, 64-over-8-head workload (399-401 us against
// 399 us), and deeper than that spills at two waves per SIMD.
constexpr int kGqaKeySteps = 2;
constexpr int kGqaValueSteps = 1;

// Grouped-query decode on the matrix cores: item li (partition, sequence, kv
// head) in decode_kernel's order, its G query heads as columns, run by the
// calling wave.
template <bool NT>
__device__ __forceinline__ void mfma_decode_item(
    uint32_t li, uint16_t* __restrict__ out, Partials ws, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ context_lens, int32_t num_seqs, int32_t num_heads,
    int32_t num_kv_heads, int32_t num_parts, int32_t partition, float scale_log2,
    RangeSplit rs) {
  const int g = static_cast<int>(li % static_cast<uint32_t>(num_kv_heads));
  const uint32_t ps = li / static_cast<uint32_t>(num_kv_heads);
  const int s = static_cast<int>(ps % static_cast<uint32_t>(num_seqs));
  const int part = static_cast<int>(ps / static_cast<uint32_t>(num_seqs));
  if (part >= num_parts) return;
  const int G = num_heads / num_kv_heads;
  // a length above the table row (a broken precondition) is cut to it
  const int L = min(context_lens[s], max_blocks * kBS);
  const int64_t row0 = static_cast<int64_t>(s) * num_heads + static_cast<int64_t>(g) * G;
  if (L <= 0) {
    if (part == 0)
      for (int i = threadIdx.x & 63; i < G * kD; i += 64) out[row0 * kD + i] = 0;
    return;
  }
  const int begin = rs.starts ? split_begin(rs.starts[s], L) : 0;
  const int part_start = begin + part * partition;
  if (part_start >= L) return;
  const int nparts_s = rs.starts ? split_parts(begin, L, partition, rs.pre_partition)
                                 : (L + partition - 1) / partition;
  if (nparts_s > 1 && ws.o == nullptr) return;
  const bool whole = nparts_s == 1;
  mfma16_decode_range<NT, kGqaKeySteps, kGqaValueSteps>(
      out, ws, kc, vc, block_tables + static_cast<int64_t>(s) * max_blocks, num_kv_heads, g,
      part_start, min(part_start + partition, L), scale_log2, G,
      [&](int i) { return q + (row0 + i) * kD; },
      [&](int i, int64_t& out_off, int64_t& part_row) {
        out_off = whole ? (row0 + i) * kD : -1;
        part_row = whole ? -1 : (row0 + i) * num_parts + rs.part_base + part;
      });
}

// One wave (one 64-thread workgroup) per item.
template <bool NT>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void decode_mfma_kernel(
    uint16_t* __restrict__ out, Partials ws, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ context_lens, int32_t num_seqs, int32_t num_heads,
    int32_t num_kv_heads, int32_t num_parts, int32_t partition, float scale_log2,
    RangeSplit rs) {
  mfma_decode_item<NT>(blockIdx.x, out, ws, q, kc, vc, block_tables, max_blocks, context_lens,
                   num_seqs, num_heads, num_kv_heads, num_parts, partition, scale_log2, rs);
}

}  // namespace
