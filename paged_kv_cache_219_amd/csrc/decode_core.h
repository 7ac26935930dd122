// One-wave decode attention over a paged KV cache (gfx950, wave64, no matrix
// cores): the per-item body shared by the decode kernels.
//
// Page "vLLM PagedAttention chuyên sâu: Phân mảnh bộ nhớ KV Cache, Prefill
// theo khối & Prefix Caching" (locionic.com), section "Cơ chế PagedAttention":
// per query token the kernel (1) looks up the sequence's physical blocks in
// its block table, (2) gathers K and V from those scattered blocks and (3) runs
// ordinary attention on them.  Section "Chunked Prefill" states decode is
// bound by memory bandwidth: the design goal is to stream every K/V page once
// at HBM speed.
//
// Work decomposition.  One wave per item (partition, kv head, sequence): a
// 64-thread workgroup in decode_kernel, one wave of a 4-wave workgroup in the
// mixed-batch kernel.  A partition is a run of `partition` tokens (a multiple
// of 64); a sequence spanning several partitions is processed by independent
// waves that each emit (m, l, o) -- running max (log2 units), sum of
// exponentials and normalised partial output -- and a second kernel merges
// them with weights l_p * 2^(m_p - max m).  The wave walks its partition in
// tiles of 64 tokens = 64 / BS pages of BS tokens (BS = 8, 16, 32 or 64),
// prefetching the next tile's block ids, keys and values while it computes on
// the current one.
//
// Within a tile:
//  * QK, one token per lane: lane BS j + t owns token t of page j and loads
//    that token's whole key row -- with the x-packed key layout the BS lanes
//    of a page read 16 BS contiguous bytes per load.  The G query heads sharing the
//    kv head are wave-uniform and read with scalar loads into SGPRs, which
//    feed the dot products directly; bf16 products use v_dot2_f32_bf16 (exact
//    products, fp32 accumulation), so no cross-lane reduction is needed for
//    the dot products.
//  * online softmax per head: wave max -> rescale factor 2^(m_old - m_new),
//    per-lane partial sums of 2^(s - m) (reduced once at the end).
//  * PV, one value d-row per lane group: with the d-major value page a 16-byte
//    load holds X consecutive tokens of one dimension, so bf16 weights pair up
//    with values for v_dot2_f32_bf16 (G >= 4) or are widened to fp32 (G < 4).
//    The weights go through LDS (64 tokens x G heads).
// Tokens past the context are masked by selecting -inf scores and zeroing
// their value elements (the cache may hold anything there).

#pragma once

#include "page_ring.h"

#include <type_traits>

namespace {

using pa::ring::kBS;
constexpr int kTile = 64;

// Orders this wave's LDS accesses: wait for its outstanding LDS operations.
// Enough to exchange data between lanes of a single-wave workgroup (a
// workgroup barrier would also wait for every global load in flight).
__device__ __forceinline__ void lds_wave_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

// Shapes of the one-wave decode for element type T, head_dim D and block size
// BS (8, 16, 32 or 64 tokens; a 64-token tile is NP pages).
template <typename T, int D, int BS = kBS>
struct Geo {
  static_assert(BS == 8 || BS == 16 || BS == 32 || BS == 64, "block size 8, 16, 32 or 64");
  static constexpr int E = sizeof(T);
  static constexpr int X = 16 / E;          // elements per 16-byte chunk
  static constexpr int NKC = D / X;         // key chunks per token row
  static constexpr int NP = 64 / BS;        // pages per 64-token tile
  static constexpr int LPR = BS / X;        // lanes per value d-row (one row = BS tokens), <= 16
  static constexpr int DPI = 64 / LPR;      // value d-rows covered by one wave load
  static constexpr int NVI = D / DPI;       // wave loads per value page
  static constexpr int PAGE = D * BS;       // elements per (block, kv head) page
};

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

template <typename T>
__device__ __forceinline__ void store_out(T* p, float v);
template <>
__device__ __forceinline__ void store_out<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t* p, float v) {
  *p = static_cast<uint16_t>(pa::f32_to_bf16_bits(v));
}

// Zero the elements of a 16-byte value chunk whose token index (0..X-1 within
// the chunk) is >= keep.
template <typename T>
__device__ __forceinline__ uint4 mask_chunk(uint4 v, int keep) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
  if (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t m = (2 * i < keep ? 0x0000ffffu : 0u) | (2 * i + 1 < keep ? 0xffff0000u : 0u);
      w[i] &= m;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = i < keep ? w[i] : 0u;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Scratch layout (device workspace): per (seq, head, partition) the
// normalised partial output [D], then per (seq, head, partition) the pair
// (m, l).
struct Partials {
  float* o;
  float* ml;
};

// A sequence's tokens can be split between two passes at a page boundary:
// [0, begin) -- a shared prefix, attended once for every sequence that shares
// its blocks -- and [begin, L), with begin = starts[s] (no split when starts
// is null).  The prefix is cut into partitions of pre_partition tokens, the
// rest into partitions of `partition` tokens.  The prefix's partials occupy
// partial slots [0, prefix parts) of each (sequence, head) row and the rest's
// slots [part_base, part_base + rest parts); a sequence whose two ranges make
// only one partition in all has its output written directly.
struct RangeSplit {
  const int32_t* starts;
  int32_t part_base;
  int32_t pre_partition;
};

__device__ __forceinline__ int split_begin(int prefix, int L) {
  return max(0, min(prefix, L)) & ~(kBS - 1);
}
__device__ __forceinline__ int split_parts(int begin, int L, int partition, int pre_partition) {
  return (begin + pre_partition - 1) / pre_partition + (L - begin + partition - 1) / partition;
}

// The decode weights' LDS element type: bf16 pairs with values in
// v_dot2_f32_bf16 (PVB), or fp32.
template <bool PVB>
using weight_t = typename std::conditional<PVB, uint16_t, float>::type;

// One item (partition, sequence, kv head) of the one-wave decode, run by one
// wave of the calling workgroup; p_lds is that wave's own G * 64 weights.
template <typename T, int D, int G, bool PVB, int BS = kBS, bool NT = false>
__device__ __forceinline__ void decode_item(
    uint32_t li, weight_t<PVB>* __restrict__ p_lds, T* __restrict__ out, Partials ws,
    const T* __restrict__ q, const T* __restrict__ kc, const T* __restrict__ vc,
    const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ context_lens, int32_t num_seqs, int32_t num_heads,
    int32_t num_kv_heads, int32_t num_parts, int32_t partition, float scale_log2,
    RangeSplit rs) {
  using Gm = Geo<T, D, BS>;
  constexpr int X = Gm::X, NKC = Gm::NKC, LPR = Gm::LPR, DPI = Gm::DPI, NVI = Gm::NVI;
  constexpr int NP = Gm::NP;
  typedef weight_t<PVB> p_t;

  // Logical order (partition, sequence, kv head), kv head fastest, in plain
  // dispatch order.  Workgroups go to the 8 XCDs round-robin, so XCD x gets
  // the kv heads congruent to x (equal work per XCD); every kv head is in
  // flight at once (their pages sit at different offsets inside a block, which
  // spreads the reads over all HBM channels); the heavy low partitions run
  // first and the mostly-empty high ones last; and sequences adjacent in the
  // batch -- e.g. samples sharing a prompt's blocks -- read the same page on
  // the same XCD a few workgroups apart, through its L2.
  const int g = static_cast<int>(li % static_cast<uint32_t>(num_kv_heads));
  const uint32_t ps = li / static_cast<uint32_t>(num_kv_heads);
  const int s = static_cast<int>(ps % static_cast<uint32_t>(num_seqs));
  const int part = static_cast<int>(ps / static_cast<uint32_t>(num_seqs));
  if (part >= num_parts) return;

  const int lane = threadIdx.x & 63;
  const int h0 = g * G;
  // A length above the table row (a broken precondition) is cut to it, so no
  // read leaves the row.
  const int L = min(context_lens[s], max_blocks * BS);
  const int64_t out_row = (static_cast<int64_t>(s) * num_heads + h0) * D;

  if (L <= 0) {
    if (part == 0)
      for (int i = lane; i < G * D; i += 64) store_out<T>(out + out_row + i, 0.f);
    return;
  }
  // Tokens [begin, L) of the sequence; [0, begin) is another pass's share.
  const int begin = rs.starts ? split_begin(rs.starts[s], L) : 0;
  const int part_start = begin + part * partition;
  if (part_start >= L) return;
  const int part_end = min(part_start + partition, L);
  const int nparts_s = rs.starts ? split_parts(begin, L, partition, rs.pre_partition)
                                 : (L + partition - 1) / partition;
  if (nparts_s > 1 && ws.o == nullptr) return;  // no room for partials: context above the bound
  const int part_base = rs.part_base;

  // The G query rows (contiguous) are read-only and wave-uniform: reading them
  // through the constant address space turns them into scalar loads whose
  // SGPRs feed the dot products directly.
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  typedef const __attribute__((address_space(4))) u32x4* q_ptr_t;
  q_ptr_t q_const = (q_ptr_t)(q + out_row);
  // More than 64 dwords of queries do not fit the scalar register file: the
  // rows are then re-read (scalar cache hits) in every tile instead of being
  // kept live across the loop.
  constexpr bool kQReload = G * D * sizeof(T) > 256;

  const int32_t* bt_row = block_tables + static_cast<int64_t>(s) * max_blocks;
  const int64_t head_off = static_cast<int64_t>(g) * Gm::PAGE;
  const int64_t blk_stride = static_cast<int64_t>(num_kv_heads) * Gm::PAGE;
  const int j_me = lane / BS;   // page of this lane's token (QK layout)
  const int t_me = lane % BS;   // token within that page
  const int vrow = lane / LPR;  // value d-row within a wave load
  const int vtok = X * (lane % LPR);  // first token of this lane's value chunk

  uint4 kreg[NKC];
  uint4 vreg[NP][NVI];
#pragma unroll
  for (int c = 0; c < NKC; ++c) kreg[c] = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int j = 0; j < NP; ++j)
#pragma unroll
    for (int k = 0; k < NVI; ++k) vreg[j][k] = make_uint4(0, 0, 0, 0);
  float m[G], l[G], acc[G][NVI];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int k = 0; k < NVI; ++k) acc[h][k] = 0.f;
  }

  const int ntiles = (part_end - part_start + kTile - 1) / kTile;
  const int lb_part = part_start / BS;

  // Block id of this lane's own page (QK layout) for a tile; -1 past the end.
  auto page_id = [&](int tile, int j) -> int {
    const int lb = lb_part + tile * NP + j;
    return lb * BS < part_end ? bt_row[lb] : -1;
  };
  // Pages past the end of the partition are not loaded: their registers keep
  // stale contents, which no result uses (their scores are replaced by -inf
  // and their value pages are skipped).
  auto load_k = [&](int phys, int kofs) {
    if (phys >= 0) {
      const T* base = kc + phys * blk_stride + head_off + kofs;
#pragma unroll
      for (int c = 0; c < NKC; ++c) kreg[c] = pa::ld16_kv<NT>(base + c * (BS * X));
    }
  };
  auto load_v = [&](const int (&ids)[NP], int vofs) {
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      if (ids[j] >= 0) {
        const T* base = vc + ids[j] * blk_stride + head_off + vofs;
#pragma unroll
        for (int k = 0; k < NVI; ++k) vreg[j][k] = pa::ld16_kv<NT>(base + k * 64 * X);
      }
    }
  };
  auto page_ids = [&](int my, int (&ids)[NP]) {
#pragma unroll
    for (int j = 0; j < NP; ++j) ids[j] = __builtin_amdgcn_readlane(my, BS * j);
  };

  // Software pipeline inside the wave: block ids are fetched two tiles ahead;
  // the keys of tile t+1 are issued into the key registers as soon as the
  // scores of tile t are done, and the values of tile t+1 into the value
  // registers as soon as tile t's weighted sum is done, so about one and a
  // half tiles stay in flight per wave with a single set of load registers.
  // Small groups issue a tile's values together with its keys; large groups
  // (32+ accumulators) issue them right after the scores.  Each prefetch's
  // address takes an empty asm dependency on the value computed just before
  // it, which keeps the scheduler from hoisting the loads into extra
  // registers.
  // Large groups are VALU-heavy and register-bound: for them the next tile's
  // keys are loaded at the top of its own iteration instead (no prefetch).
  constexpr bool kEarlyV = G <= 2;
  constexpr bool kPipe = G <= 2;
  int id_cur = page_id(0, j_me);
  int id_next = ntiles > 1 ? page_id(1, j_me) : -1;
  int ids[NP];
  page_ids(id_cur, ids);
  load_k(id_cur, t_me * X);
  if (kEarlyV) load_v(ids, lane * X);

  for (int tile = 0; tile < ntiles; ++tile) {
    const int tile_start = part_start + tile * kTile;
    const bool more = tile + 1 < ntiles;
    const int id_next2 = tile + 2 < ntiles ? page_id(tile + 2, j_me) : -1;
    if (!kPipe && tile > 0) load_k(id_cur, t_me * X);

    // ---- scores, one token per lane
    float sc[G];
    auto dot_chunk = [&](float a, u32x4 qw, uint4 kv) -> float {
      if (sizeof(T) == 2) {
        a = pa::dot2_bf16(qw.x, kv.x, a);
        a = pa::dot2_bf16(qw.y, kv.y, a);
        a = pa::dot2_bf16(qw.z, kv.z, a);
        a = pa::dot2_bf16(qw.w, kv.w, a);
      } else {
        a = fmaf(__uint_as_float(qw.x), __uint_as_float(kv.x), a);
        a = fmaf(__uint_as_float(qw.y), __uint_as_float(kv.y), a);
        a = fmaf(__uint_as_float(qw.z), __uint_as_float(kv.z), a);
        a = fmaf(__uint_as_float(qw.w), __uint_as_float(kv.w), a);
      }
      return a;
    };
    if (kQReload) {
      // One head at a time; the next head's query row is loaded once this
      // head's scores are done (the address takes an empty asm dependency on
      // them), so only one row occupies scalar registers.
#pragma unroll
      for (int h = 0; h < G; ++h) {
        uint64_t qa = reinterpret_cast<uint64_t>(q_const + h * NKC);
        if (h > 0)
          asm volatile("" : "+s"(qa) : "v"(sc[h - 1]));
        else
          asm volatile("" : "+s"(qa));
        const q_ptr_t qh = reinterpret_cast<q_ptr_t>(qa);
        float a = 0.f;
#pragma unroll
        for (int c = 0; c < NKC; ++c) a = dot_chunk(a, qh[c], kreg[c]);
        sc[h] = a;
      }
    } else {
#pragma unroll
      for (int h = 0; h < G; ++h) sc[h] = 0.f;
#pragma unroll
      for (int c = 0; c < NKC; ++c) {
#pragma unroll
        for (int h = 0; h < G; ++h) sc[h] = dot_chunk(sc[h], q_const[h * NKC + c], kreg[c]);
      }
    }
    int ids_next[NP];
    page_ids(id_next, ids_next);
    {
      int vofs = lane * X, kofs = t_me * X;
      asm volatile("" : "+v"(vofs), "+v"(kofs) : "v"(sc[G - 1]));
      if (!kEarlyV) load_v(ids, vofs);
      if (kPipe && more) load_k(id_next, kofs);
    }

    const bool tok_ok = tile_start + lane < part_end;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float sv = tok_ok ? sc[h] * scale_log2 : -INFINITY;
      const float m_new = fmaxf(m[h], pa::wave_max_u(sv));
      const float alpha = pa::fast_exp2(m[h] - m_new);
      const float p = pa::fast_exp2(sv - m_new);
      l[h] = l[h] * alpha + p;
#pragma unroll
      for (int k = 0; k < NVI; ++k) acc[h][k] *= alpha;
      m[h] = m_new;
      if (PVB)
        p_lds[h * kTile + lane] = static_cast<p_t>(pa::f32_to_bf16_bits(p));
      else
        p_lds[h * kTile + lane] = static_cast<p_t>(p);
    }
    // The weights are exchanged between lanes of this (single-wave)
    // workgroup; its LDS operations complete in order, so waiting for the
    // writes suffices -- and unlike a workgroup barrier this does not wait
    // for the prefetches in flight.
    lds_wave_sync();

    // ---- weighted values
    if (tile_start + kTile > part_end) {
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        const int keep = part_end - (tile_start + BS * j + vtok);
        if (keep < X) {
#pragma unroll
          for (int k = 0; k < NVI; ++k) vreg[j][k] = mask_chunk<T>(vreg[j][k], keep);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      if (ids[j] < 0) continue;
      int pofs = BS * j + vtok;
      if (G > 2) asm volatile("" : "+v"(pofs));  // weights of one page at a time
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const p_t* pp = p_lds + h * kTile + pofs;
        if (PVB) {
          const uint4 pw = ld16(pp);
#pragma unroll
          for (int k = 0; k < NVI; ++k) {
            float a = acc[h][k];
            a = pa::dot2_bf16(pw.x, vreg[j][k].x, a);
            a = pa::dot2_bf16(pw.y, vreg[j][k].y, a);
            a = pa::dot2_bf16(pw.z, vreg[j][k].z, a);
            a = pa::dot2_bf16(pw.w, vreg[j][k].w, a);
            acc[h][k] = a;
          }
        } else if (sizeof(T) == 2) {
          const uint4 p0 = ld16(pp);
          const uint4 p1 = ld16(pp + 4);
          const float pf[8] = {__uint_as_float(p0.x), __uint_as_float(p0.y),
                               __uint_as_float(p0.z), __uint_as_float(p0.w),
                               __uint_as_float(p1.x), __uint_as_float(p1.y),
                               __uint_as_float(p1.z), __uint_as_float(p1.w)};
#pragma unroll
          for (int k = 0; k < NVI; ++k) {
            const uint32_t w[4] = {vreg[j][k].x, vreg[j][k].y, vreg[j][k].z, vreg[j][k].w};
            float a = acc[h][k];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              a = fmaf(pf[2 * i], pa::bf16_lo(w[i]), a);
              a = fmaf(pf[2 * i + 1], pa::bf16_hi(w[i]), a);
            }
            acc[h][k] = a;
          }
        } else {
          const uint4 p0 = ld16(pp);
#pragma unroll
          for (int k = 0; k < NVI; ++k) {
            float a = acc[h][k];
            a = fmaf(__uint_as_float(p0.x), __uint_as_float(vreg[j][k].x), a);
            a = fmaf(__uint_as_float(p0.y), __uint_as_float(vreg[j][k].y), a);
            a = fmaf(__uint_as_float(p0.z), __uint_as_float(vreg[j][k].z), a);
            a = fmaf(__uint_as_float(p0.w), __uint_as_float(vreg[j][k].w), a);
            acc[h][k] = a;
          }
        }
      }
    }
    lds_wave_sync();  // p_lds is rewritten by the next tile
    if (kEarlyV && more) {
      int vofs = lane * X;
      asm volatile("" : "+v"(vofs) : "v"(acc[G - 1][NVI - 1]));
      load_v(ids_next, vofs);
    }
#pragma unroll
    for (int j = 0; j < NP; ++j) ids[j] = ids_next[j];
    id_cur = id_next;
    id_next = id_next2;
  }

  // ---- combine lanes; write the output, or this partition's partial
  float lt[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    lt[h] = pa::wave_sum_u(l[h]);
    const float inv = 1.f / lt[h];
#pragma unroll
    for (int k = 0; k < NVI; ++k) {
      float a = acc[h][k];
      // sum over the LPR lanes sharing a value row
      if (LPR >= 2) a += pa::dpp<pa::kDppXor1>(a);
      if (LPR >= 4) a += pa::dpp<pa::kDppXor2>(a);
      if (LPR >= 8) a += pa::dpp<pa::kDppHalfMirror>(a);
      if (LPR >= 16) a += pa::dpp<pa::kDppMirror>(a);
      const int d = k * DPI + vrow;
      if (lane % LPR == 0) {
        if (nparts_s == 1) {
          store_out<T>(out + out_row + h * D + d, a * inv);
        } else {
          const int64_t row =
              (static_cast<int64_t>(s) * num_heads + h0 + h) * num_parts + part_base + part;
          ws.o[row * D + d] = a * inv;
        }
      }
    }
  }
  if (nparts_s > 1 && lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const int64_t row =
          (static_cast<int64_t>(s) * num_heads + h0 + h) * num_parts + part_base + part;
      ws.ml[2 * row] = m[h];
      ws.ml[2 * row + 1] = lt[h];
    }
  }
}

// Second pass, one wave per (sequence, query head) with more than one
// partition: out = sum_p w_p o_p / sum_p w_p with w_p = l_p * 2^(m_p - M),
// M = max_p m_p.  Lane p computes partition p's weight (64 partitions at a
// time); the partial outputs are then accumulated in partition order, each
// lane owning D/64 consecutive dimensions, so the result is deterministic.
// With a split sequence the partitions are the prefix's, slots [0, n_pre),
// then the rest's, slots [part_base, part_base + n_rest).
// (Merging inside the first pass would need an agent-scope release per
// partition -- an L2 write-back on this chip, far costlier than this launch.)
template <typename T, int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(
    T* __restrict__ out, Partials ws, const int32_t* __restrict__ context_lens, int32_t num_heads,
    int32_t num_parts, int32_t partition, RangeSplit rs, int32_t max_tokens) {
  constexpr int PER = D / 64;
  typedef float vec_t __attribute__((ext_vector_type(PER)));
  const int lane = threadIdx.x;
  const int64_t row = blockIdx.x;  // seq * num_heads + head
  const int s = static_cast<int>(row / num_heads);
  const int L = min(context_lens[s], max_tokens);  // as the first pass cut it
  if (L <= 0) return;
  const int begin = rs.starts ? split_begin(rs.starts[s], L) : 0;
  const int part_base = rs.part_base;
  // A length above the call's max_context_len (a broken precondition) would
  // name partitions past the row's slots: read only the slots that exist.
  const int n_pre = min(rs.starts ? (begin + rs.pre_partition - 1) / rs.pre_partition : 0,
                        part_base);
  const int n_rest = min((L - begin + partition - 1) / partition, num_parts - part_base);
  if (n_pre + n_rest <= 1) return;
  const int64_t row0 = row * num_parts;
  const float2* ml = reinterpret_cast<const float2*>(ws.ml) + row0;
  float M = -INFINITY;
  for (int p = lane; p < n_pre; p += 64) M = fmaxf(M, ml[p].x);
  for (int p = lane; p < n_rest; p += 64) M = fmaxf(M, ml[part_base + p].x);
  M = pa::wave_max_u(M);
  const vec_t* po = reinterpret_cast<const vec_t*>(ws.o + row0 * D) + lane;
  vec_t acc = {};
  float wsum = 0.f;
  // partials [first, first + n) of the row, in order
  auto run = [&](int first, int n) {
    for (int p0 = 0; p0 < n; p0 += 64) {
      float w = 0.f;
      if (p0 + lane < n) {
        const float2 v = ml[first + p0 + lane];
        w = v.y * pa::fast_exp2(v.x - M);
      }
      wsum += w;
      const int cnt = min(64, n - p0);
      const vec_t* pj = po + (first + p0) * 64;
      int j = 0;
      for (; j + 4 <= cnt; j += 4) {  // four partitions' loads in flight
        const vec_t o0 = pj[j * 64], o1 = pj[(j + 1) * 64], o2 = pj[(j + 2) * 64],
                    o3 = pj[(j + 3) * 64];
        acc += pa::readlane_f(w, j) * o0;
        acc += pa::readlane_f(w, j + 1) * o1;
        acc += pa::readlane_f(w, j + 2) * o2;
        acc += pa::readlane_f(w, j + 3) * o3;
      }
      for (; j < cnt; ++j) acc += pa::readlane_f(w, j) * pj[j * 64];
    }
  };
  run(0, n_pre);
  run(part_base, n_rest);
  const float inv = 1.f / pa::wave_sum_u(wsum);
  T* dst = out + row * D + lane * PER;
#pragma unroll
  for (int i = 0; i < PER; ++i) store_out<T>(dst + i, acc[i] * inv);
}

// ---- host side: the partials workspace

constexpr size_t kAlign = 256;

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// partial outputs | (m, l) pairs, each region 256-byte aligned
inline size_t ws_bytes(int64_t B, int64_t H, int64_t D, int64_t parts) {
  if (parts <= 1) return 0;
  return align_up(static_cast<size_t>(B * H * parts * D) * sizeof(float)) +
         static_cast<size_t>(B * H * parts * 2) * sizeof(float);
}

inline Partials carve(void* ws, int64_t B, int64_t H, int64_t D, int64_t slots) {
  Partials p{nullptr, nullptr};
  if (slots > 1) {
    uint8_t* base = static_cast<uint8_t*>(ws);
    p.o = reinterpret_cast<float*>(base);
    base += align_up(static_cast<size_t>(B * H * slots * D) * sizeof(float));
    p.ml = reinterpret_cast<float*>(base);
  }
  return p;
}

// partitions of `partition` tokens covering max_context_len (1 when unsplit)
inline int64_t parts_for(int32_t max_context_len, int32_t partition) {
  if (partition <= 0) return 1;
  return max_context_len <= 0 ? 1
                              : (static_cast<int64_t>(max_context_len) + partition - 1) / partition;
}

}  // namespace
