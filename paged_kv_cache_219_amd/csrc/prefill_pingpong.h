// Chunked prefill over a paged KV cache on gfx950 matrix cores, 256 query
// rows per workgroup with a ping-pong schedule between the two waves that
// share each SIMD.
//
// Page "vLLM PagedAttention chuyên sâu: Phân mảnh bộ nhớ KV Cache, Prefill
// theo khối & Prefix Caching" (locionic.com), sections "Chunked Prefill" and
// "Cơ chế của Chunked Prefill": a long prompt is processed in chunks, in
// order, each chunk's K/V accumulating in paged blocks; prefill is the
// compute-heavy phase.  Query i of an n_q-row chunk sits at position
// L - n_q + i and attends to positions 0 .. L - n_q + i.
//
// Why ping-pong.  Per 32-token step a wave does 16 matrix products (512
// cycles of one SIMD's matrix core) and about 60 vector instructions of
// online softmax.  On gfx950 a SIMD runs one wave's MFMAs and another wave's
// vector instructions at the same time without slowing the MFMAs, but a wave
// alternating between the two leaves the matrix core idle during its own
// softmax.  So the 8 waves of a workgroup (two per SIMD: waves w and w + 4)
// form two groups that take turns: while waves 0-3 run their matrix phase,
// waves 4-7 run their softmax phase, and a workgroup barrier swaps the roles.
// A single wave issues about one instruction every 4-6 cycles whatever its
// kind, so the two phases are balanced by instruction count, not by unit: the
// matrix phase, which issues only 16 MFMAs in its 512 cycles, also issues the
// LDS reads of the next phase's operands (into the registers the products
// before them have read); the softmax phase issues this wave's share of a
// ring copy and runs the softmax.  Addresses are per-lane constants plus a
// scalar per step, block ids come from scalar loads a phase ahead, and the
// row sums come from v_dot2 on the bf16 weights.
//
// Per wave, step j of the keys/values (32 tokens = two 16-token pages):
//   matrix phase j:  O^T += V_{j-1}^T P_{j-1}^T   (8 x v_mfma_f32_32x32x16_bf16)
//                    S^T  = K_j Q^T               (8 more)
//                    with the LDS reads of V_j and K_{j+1} (operands of matrix
//                    phase j + 1) between them;
//   softmax phase j: this wave's share of the copy of step j + kRingPP - 1
//                    into the LDS ring, then the online softmax of S_j -> P_j
//                    (bf16, in registers).
// The transposed form and the token order of the K operand's rows are those of
// the 128-row kernel (prefill_core.h): each lane owns one query column, so the
// softmax of a query stays in two lanes and P^T is built from the lane's own
// scores.
//
// Rows.  Wave w owns the rows w, w + 8, w + 16, ... of the workgroup's 256, so
// every wave reaches the causal diagonal in the same step and no wave idles
// through the last steps of the tile.
//
// The LDS ring.  Step j's K and V pages (16 KB) are copied once per workgroup
// with direct-to-LDS loads, two 1 KB loads per wave, kRingPP - 1 steps ahead.
// Step m is read in the matrix phases m - 1 (K_m) and m (V_m) of both groups.
// At the end of its matrix phase j every wave waits for its own copy of step
// j + 2, so the barrier after group 1's matrix phase j publishes step j + 2
// before group 0's matrix phase j + 1 reads it.  The copy of step j + kRingPP
// - 1, issued in softmax phase j, overwrites step j - 1, whose last reader was
// group 1's matrix phase j - 1 (before the barrier that started the phase).
#pragma once

#include "prefill_core.h"

namespace {

constexpr int kWavesPP = 8;
constexpr int kRowsPP = 32 * kWavesPP;  // query rows per workgroup
#ifndef PA_PP_RING
#define PA_PP_RING 8
#endif
constexpr int kRingPP = PA_PP_RING;     // 16 KB per step of LDS: one workgroup per CU
static_assert(kRingPP >= 4 && kRingPP <= 9, "ring of 4 to 9 steps");

// Phase boundary: a workgroup barrier that the compiler may not move any
// instruction across (a plain barrier lets the scheduler pull the next phase's
// matrix products or the previous phase's softmax through it).
__device__ __forceinline__ void pp_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Wait until at most N of this wave's vector-memory loads are outstanding.
template <int N>
__device__ __forceinline__ void pp_wait_loads() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// The same for a count known only at run time (n even: whole steps of two
// copies each; up to 2 (kRingPP - 3)): a chain of compares and branches, so
// the loop's steady state uses pp_wait_loads instead.
__device__ __forceinline__ void pp_wait_copies(int n) {
  if (n >= 12) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
  else if (n >= 10) asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
  else if (n >= 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else if (n >= 6) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
  else if (n >= 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else if (n >= 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// The workgroup `bid` of a grid of ceil(num_heads * num_seqs / 8) * 8 *
// num_qtiles workgroups of 512 threads (num_qtiles = ceil(max chunk / 256)).
__device__ __forceinline__ void prefill_tile_pp(
    uint32_t bid, StepBuf (&ring)[kRingPP], uint16_t* __restrict__ out,
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ qsl, const int32_t* __restrict__ context_lens, int32_t num_seqs,
    int32_t num_heads, int32_t num_kv_heads, int32_t num_qtiles, float scale_log2) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;

  // Order of work, as in prefill_tile: a unit is one (sequence, head); units
  // run longest first and unit u on XCD u % 8, its q-tiles consecutive there.
  const uint32_t xcd = bid % kXcds, k = bid / kXcds;
  const uint32_t u = (k / num_qtiles) * kXcds + xcd;
  const int qt = num_qtiles - 1 - static_cast<int>(k % num_qtiles);
  if (u >= static_cast<uint32_t>(num_seqs) * num_heads) return;  // grid padding
  const int h = static_cast<int>(u % static_cast<uint32_t>(num_heads));
  const int rank = static_cast<int>(u / static_cast<uint32_t>(num_heads));
  int s = rank;
  if (num_seqs <= 64) {
    int work = -1;
    if (lane < num_seqs) {
      const int Li = context_lens[lane], nqi = qsl[lane + 1] - qsl[lane];
      work = 0;
      for (int t = 0; t < num_qtiles && t * kRowsPP < nqi; ++t)
        work += (Li - nqi + min((t + 1) * kRowsPP, nqi) - 1) / kStep + 1;
    }
    int my_rank = 0;
    for (int j = 0; j < num_seqs; ++j) {
      const int wj = __builtin_amdgcn_readlane(work, j);
      my_rank += (wj > work) || (wj == work && j < lane);
    }
    s = __builtin_ctzll(__ballot(lane < num_seqs && my_rank == rank));
  }

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;  // 0: matrix phase first; 1: softmax phase first
  const int g = h / (num_heads / num_kv_heads);
  const int q0 = qsl[s];
  const int n_q = qsl[s + 1] - q0;
  // a length above the table row (a broken precondition) is cut to it
  const int L = min(context_lens[s], max_blocks * kBS);
  const int wg_row0 = qt * kRowsPP;
  if (wg_row0 >= n_q) return;  // whole workgroup idle (uniform: no barrier is skipped)
  const int first_pos = L - n_q;  // position of chunk row 0
  const int wg_last = first_pos + min(wg_row0 + kRowsPP, n_q) - 1;
  const int nsteps = wg_last / kStep + 1;  // steps covering tokens 0 .. wg_last

  const int qn = lane & 31;  // this lane's query column
  const int hh = lane >> 5;  // which half of the accumulator rows
  const int my_row = min(wg_row0 + wave + 8 * qn, n_q - 1);
  const int my_pos = first_pos + my_row;
  const int wave_first = first_pos + wg_row0 + wave;  // lowest position among the wave's rows
  const int j_edge = (wave_first + 1) / kStep;        // first step with 32 j + 31 > wave_first

  // Q^T operand: lane (qn, hh) holds dims 16 kk + 8 hh .. + 7 of its row.
  uint4 qreg[8];
  {
    const uint16_t* qrow =
        q + (static_cast<int64_t>(q0 + my_row) * num_heads + h) * kD + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qreg[kk] = *reinterpret_cast<const uint4*>(qrow + 16 * kk);
  }

  // The block id of this wave's page of a step: a scalar load issued at the
  // start of the softmax phase before the one whose copy needs it, and taken
  // after that phase's operand wait (a wait for it at its use would also wait
  // for the operand reads of the matrix phase in between).  Pages past the
  // last needed token name logical block 0 (always valid): their scores are
  // masked and their values weighted by 0.
  const int32_t* bt_row = block_tables + static_cast<int64_t>(s) * max_blocks;
  const int pw = pa::ring::page_of<kWavesPP>(wave);
  auto block_of = [&](int st) {
    const int lb = st * kPages + pw;
    return bt_row[lb * kBS <= wg_last ? lb : 0];
  };
  // Consume the query registers before the copies are issued: the compiler
  // does not count the copies (inline asm), so a wait for these loads placed
  // at their first use would drain every copy in flight.
#pragma unroll
  for (int kk = 0; kk < 8; ++kk)
    asm volatile("" : "+v"(qreg[kk].x), "+v"(qreg[kk].y), "+v"(qreg[kk].z), "+v"(qreg[kk].w));

  const RingLane<kWavesPP> rl(wave, lane);
  // a block's bytes fit 32 bits (the entry point bounds num_kv_heads), so a
  // copy's source offset is one 32 x 32 -> 64-bit product
  const uint32_t page_bytes = static_cast<uint32_t>(kPageElems) * 2;
  const uint32_t blk_bytes = static_cast<uint32_t>(num_kv_heads) * page_bytes;
  const int64_t head_bytes = static_cast<int64_t>(g) * page_bytes;
  const uint32_t u0 = 64u * static_cast<uint32_t>(wave);  // this wave's run of the step
  const uint32_t ring_lds = pa::ring::lds_addr(&ring[0]);
  const char* lds = reinterpret_cast<const char*>(&ring[0]);
  const char* kc_b = reinterpret_cast<const char*>(kc) + head_bytes;
  const char* vc_b = reinterpret_cast<const char*>(vc) + head_bytes;
  auto issue = [&](int st, int phys) {
    const uint64_t src = static_cast<uint64_t>(static_cast<uint32_t>(phys)) * blk_bytes;
    const uint32_t dst = ring_lds + static_cast<uint32_t>(st % kRingPP) * kStepBytes + u0 * 16;
    dma16_sbase(kc_b + src, rl.k_src[0], dst);
    dma16_sbase(vc_b + src, rl.v_src[0], dst + kVBytes);
  };

  uint4 kop[8], vop[kPages][4];
  // After an explicit wait for the operand reads: tell the compiler they are
  // complete, so it places no waits of its own before the products.
  auto operands_ready = [&]() {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      asm volatile("" : "+v"(kop[kk].x), "+v"(kop[kk].y), "+v"(kop[kk].z), "+v"(kop[kk].w));
#pragma unroll
    for (int pg = 0; pg < kPages; ++pg)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        asm volatile("" : "+v"(vop[pg][dt].x), "+v"(vop[pg][dt].y), "+v"(vop[pg][dt].z),
                     "+v"(vop[pg][dt].w));
  };
  auto read_k = [&](int st) {
    const char* b = lds + static_cast<uint32_t>(st % kRingPP) * kStepBytes;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) kop[kk] = rl.k_op(b, kk);
  };

  pa::f32x16_t o[4], sa;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pa::f32x16_t{};
  sa = pa::f32x16_t{};
  uint4 pb[kPages];
  OnlineSoftmax sm;

  // ---- matrix phase j: PV of step j - 1 and the scores of step j, with the
  // LDS reads that refill the operand registers (V_j and K_{j+1}, for matrix
  // phase j + 1) one MFMA pair behind the products that read them: a read
  // into registers an MFMA in flight is still reading waits for that MFMA.
  auto matrix_phase = [&](int j, bool do_pv, bool do_s, bool ld_v, bool ld_k) {
    __builtin_amdgcn_s_setprio(1);
    const char* bk = lds + static_cast<uint32_t>((j + 1) % kRingPP) * kStepBytes;
    const char* bv = lds + static_cast<uint32_t>(j % kRingPP) * kStepBytes;
    auto refill = [&](int i) {
      if (ld_k) {
        kop[i] = rl.k_op(bk, i);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      if (ld_v) {
        vop[i >> 2][i & 3] = rl.v_op(bv, i >> 2, i & 3);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    };
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (do_s) {
        sa = mfma32(kop[i], qreg[i], i == 0 ? pa::f32x16_t{} : sa);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      if (do_pv) {
        o[i & 3] = mfma32(vop[i >> 2][i & 3], pb[i >> 2], o[i & 3]);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      if (i > 0) refill(i - 1);
    }
    refill(7);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    // this wave's copy of step j + 2 has landed (later steps may stay in
    // flight; the softmax phases issue the copies)
    if (j + kRingPP - 2 <= nsteps - 1) pp_wait_loads<2 * (kRingPP - 4)>();
    else pp_wait_copies(2 * max(0, nsteps - 1 - (j + 2)));
  };

  // ---- softmax phase of step j: the copy of step j + kRingPP - 1 (it
  // overwrites step j - 1, last read by group 1's matrix phase j - 1, before
  // the barrier that started this phase), then the softmax.  Lane (qn, hh)
  // element i is token t0 + 16 (i / 8) + 8 hh + i % 8 of its query row.
  int next_phys = 0;  // block id for the next softmax phase's copy
  auto softmax_phase = [&](int j) {
    const int t0 = j * kStep;
    if (j + kRingPP - 1 < nsteps) issue(j + kRingPP - 1, next_phys);
    if (j + kRingPP < nsteps) next_phys = block_of(j + kRingPP);
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = sa[i];
    // a diagonal or tail step: 32 j + 31 > wave_first (a tail step, 32 j + 32
    // > L > wave_first, is one), i.e. j >= j_edge -- one scalar compare
    const bool edge = j >= j_edge;
    if (edge) {
      const int lim = min(my_pos, L - 1) - t0 - 8 * hh;  // keep offsets <= lim
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (16 * (i >> 3) + (i & 7) > lim) x[i] = -INFINITY;
    }
    uint32_t pw[8];
    sm.step(x, scale_log2, pw, o);
#pragma unroll
    for (int pg = 0; pg < kPages; ++pg)
      pb[pg] = make_uint4(pw[4 * pg], pw[4 * pg + 1], pw[4 * pg + 2], pw[4 * pg + 3]);
    // Consume the weights and the row sum here: their only users are in the
    // next matrix phase, and the compiler would otherwise sink the
    // exponentials into it.
#pragma unroll
    for (int pg = 0; pg < kPages; ++pg)
      asm volatile("" : "+v"(pb[pg].x), "+v"(pb[pg].y), "+v"(pb[pg].z), "+v"(pb[pg].w));
    asm volatile("" : "+v"(sm.l_run));
    // the operands read in matrix phase j have landed
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    operands_ready();
    // the block id has landed too: taken here, the next softmax phase's copy
    // needs no wait (which would also drain the matrix phase's operand reads)
    asm volatile("" : "+s"(next_phys));
    if (edge && t0 + kStep > L) {  // values of tokens at or past L may be anything: 0 * NaN
#pragma unroll
      for (int pg = 0; pg < kPages; ++pg) {
        const int keep = L - (t0 + 16 * pg + 8 * hh);
        if (keep < 8) {
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) vop[pg][dt] = keep_tokens(vop[pg][dt], keep);
        }
      }
    }
  };

  // ---- prologue: copies of the first steps; steps 0 and 1 published
  for (int st = 0; st < kRingPP - 1 && st < nsteps; ++st) issue(st, block_of(st));
  if (kRingPP - 1 < nsteps) next_phys = block_of(kRingPP - 1);
  pp_wait_copies(2 * max(0, min(nsteps - 1, kRingPP - 2) - 1));
  pp_barrier();
  read_k(0);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  operands_ready();

  // ---- the two groups, one phase apart; both pass 2 nsteps + 3 barriers
  if (grp == 1) pp_barrier();
  if (nsteps > 1) {
    matrix_phase(0, false, true, true, true);
    pp_barrier();
    for (int j = 1; j + 1 < nsteps; ++j) {
      softmax_phase(j - 1);
      pp_barrier();
      matrix_phase(j, true, true, true, true);
      pp_barrier();
    }
    softmax_phase(nsteps - 2);
    pp_barrier();
    matrix_phase(nsteps - 1, true, true, true, false);
  } else {
    matrix_phase(0, false, true, true, false);
  }
  pp_barrier();
  softmax_phase(nsteps - 1);
  pp_barrier();
  matrix_phase(nsteps, true, false, false, false);
  if (grp == 0) pp_barrier();

  // ---- write this lane's column: O / l, 4 runs of 4 dims per accumulator
  const float lt = sm.l_run + __shfl_xor(sm.l_run, 32, 64);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const int row = wg_row0 + wave + 8 * qn;
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
