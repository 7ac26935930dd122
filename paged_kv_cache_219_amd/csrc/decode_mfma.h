// Decode of several query rows against one kv head's paged K/V on the matrix
// cores, one wave, no LDS (gfx950; bf16, head_dim 128, 16-token blocks).
//
// Page "vLLM PagedAttention chuyên sâu: Phân mảnh bộ nhớ KV Cache, Prefill
// theo khối & Prefix Caching" (locionic.com), section "Cơ chế PagedAttention":
// look up the physical blocks in the block table, gather K and V, attend.
//
// With n (up to 32) query rows on one kv head -- the query heads of a
// grouped-query group, or the samples of a prompt over their shared prefix --
// a 32-token step is a small dense contraction, computed in the same
// transposed form as the chunked-prefill kernel:
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
  mfma_decode_range<NT>(
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
