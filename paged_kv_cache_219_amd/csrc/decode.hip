// Decode attention over a paged KV cache (gfx950, wave64, no matrix cores).
//
// Page "vLLM PagedAttention chuyên sâu: Phân mảnh bộ nhớ KV Cache, Prefill
// theo khối & Prefix Caching" (locionic.com), section "Cơ chế PagedAttention":
// per query token the kernel (1) looks up the sequence's physical blocks in
// its block table, (2) gathers K and V from those scattered blocks and (3) runs
// ordinary attention on them.  Section "Chunked Prefill" states decode is
// bound by memory bandwidth: the design goal is to stream every K/V page once
// at HBM speed.
//
// Work decomposition.  One wave (one 64-thread workgroup) per (partition,
// kv head, sequence).  A partition is a run of `partition` tokens (a multiple
// of 64); a sequence spanning several partitions is processed by independent
// waves that each emit (m, l, o) -- running max (log2 units), sum of
// exponentials and normalised partial output -- and a second kernel merges
// them with weights l_p * 2^(m_p - max m).  The wave walks its partition in
// tiles of 64 tokens = 4 pages of 16 tokens, prefetching the next tile's
// block ids, keys and values while it computes on the current one.
//
// Within a tile:
//  * QK, one token per lane: lane 16j+t owns token t of page j and loads that
//    token's whole key row -- with the x-packed key layout the 16 lanes of a
//    page read 256 contiguous bytes per load.  The G query heads sharing the
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

#include "page_ring.h"

#include <type_traits>

namespace {

constexpr int kBS = 16;
constexpr int kTile = 64;

// Orders this wave's LDS accesses: wait for its outstanding LDS operations.
// Enough to exchange data between lanes of a single-wave workgroup (a
// workgroup barrier would also wait for every global load in flight).
__device__ __forceinline__ void lds_wave_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

template <typename T, int D>
struct Geo {
  static constexpr int E = sizeof(T);
  static constexpr int X = 16 / E;          // elements per 16-byte chunk
  static constexpr int NKC = D / X;         // key chunks per token row
  static constexpr int LPR = kBS / X;       // lanes per value d-row (one row = 16 tokens)
  static constexpr int DPI = 64 / LPR;      // value d-rows covered by one wave load
  static constexpr int NVI = D / DPI;       // wave loads per value page
  static constexpr int PAGE = D * kBS;      // elements per (block, kv head) page
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

template <typename T, int D, int G, bool PVB>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void decode_kernel(
    T* __restrict__ out, Partials ws, const T* __restrict__ q, const T* __restrict__ kc,
    const T* __restrict__ vc, const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ context_lens, int32_t num_seqs, int32_t num_heads,
    int32_t num_kv_heads, int32_t num_parts, int32_t partition, float scale_log2,
    RangeSplit rs) {
  using Gm = Geo<T, D>;
  constexpr int X = Gm::X, NKC = Gm::NKC, LPR = Gm::LPR, DPI = Gm::DPI, NVI = Gm::NVI;
  typedef typename std::conditional<PVB, uint16_t, float>::type p_t;

  __shared__ __attribute__((aligned(16))) p_t p_lds[G * kTile];

  // Logical order (partition, sequence, kv head), kv head fastest, in plain
  // dispatch order.  Workgroups go to the 8 XCDs round-robin, so XCD x gets
  // the kv heads congruent to x (equal work per XCD); every kv head is in
  // flight at once (their pages sit at different offsets inside a block, which
  // spreads the reads over all HBM channels); the heavy low partitions run
  // first and the mostly-empty high ones last; and sequences adjacent in the
  // batch -- e.g. samples sharing a prompt's blocks -- read the same page on
  // the same XCD a few workgroups apart, through its L2.
  const uint32_t li = blockIdx.x;
  const int g = static_cast<int>(li % static_cast<uint32_t>(num_kv_heads));
  const uint32_t ps = li / static_cast<uint32_t>(num_kv_heads);
  const int s = static_cast<int>(ps % static_cast<uint32_t>(num_seqs));
  const int part = static_cast<int>(ps / static_cast<uint32_t>(num_seqs));
  if (part >= num_parts) return;

  const int lane = threadIdx.x;
  const int h0 = g * G;
  const int L = context_lens[s];
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
  const int j_me = lane >> 4;   // page of this lane's token (QK layout)
  const int t_me = lane & 15;   // token within that page
  const int vrow = lane / LPR;  // value d-row within a wave load
  const int vtok = X * (lane % LPR);  // first token of this lane's value chunk

  uint4 kreg[NKC];
  uint4 vreg[4][NVI];
#pragma unroll
  for (int c = 0; c < NKC; ++c) kreg[c] = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int j = 0; j < 4; ++j)
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
  const int lb_part = part_start / kBS;

  // Block id of this lane's own page (QK layout) for a tile; -1 past the end.
  auto page_id = [&](int tile, int j) -> int {
    const int lb = lb_part + tile * 4 + j;
    return lb * kBS < part_end ? bt_row[lb] : -1;
  };
  // Pages past the end of the partition are not loaded: their registers keep
  // stale contents, which no result uses (their scores are replaced by -inf
  // and their value pages are skipped).
  auto load_k = [&](int phys, int kofs) {
    if (phys >= 0) {
      const T* base = kc + phys * blk_stride + head_off + kofs;
#pragma unroll
      for (int c = 0; c < NKC; ++c) kreg[c] = ld16(base + c * (kBS * X));
    }
  };
  auto load_v = [&](const int (&ids)[4], int vofs) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (ids[j] >= 0) {
        const T* base = vc + ids[j] * blk_stride + head_off + vofs;
#pragma unroll
        for (int k = 0; k < NVI; ++k) vreg[j][k] = ld16(base + k * 64 * X);
      }
    }
  };
  auto page_ids = [&](int my, int (&ids)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) ids[j] = __builtin_amdgcn_readlane(my, 16 * j);
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
  int ids[4];
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
    int ids_next[4];
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
      for (int j = 0; j < 4; ++j) {
        const int keep = part_end - (tile_start + 16 * j + vtok);
        if (keep < X) {
#pragma unroll
          for (int k = 0; k < NVI; ++k) vreg[j][k] = mask_chunk<T>(vreg[j][k], keep);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (ids[j] < 0) continue;
      int pofs = 16 * j + vtok;
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
    for (int j = 0; j < 4; ++j) ids[j] = ids_next[j];
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
      a += pa::dpp<pa::kDppXor1>(a);  // lanes sharing a value row: xor 1 (and 2)
      if (LPR == 4) a += pa::dpp<pa::kDppXor2>(a);
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

// Grouped-query decode (4 or 8 query heads per kv head; bf16, head_dim 128).
//
// One 4-wave workgroup per (partition, sequence, kv head).  The partition's
// pages stream through LDS in 32-token steps (page_ring.h: direct-to-LDS
// copies three steps ahead, so up to 48 KB per workgroup is in flight while
// the waves compute), and every wave reads the staged K/V for its own GW
// query heads -- each page leaves HBM once for all G heads, and no K/V bytes
// pass through registers before they are used.
//
// Per step and wave:
//  * QK: lane = (token, half): token (lane / 2) of the step, dims
//    64 * (lane % 2) .. +63 (8 chunks), so the 64 lanes cover 32 tokens x
//    128 dims; the two halves are summed with one DPP exchange.  The lane's
//    half of each query row sits in registers for the whole partition.
//  * softmax with a lazily moved reference: the weights of a step are
//    2^(s - m) for the wave-uniform reference m, and m (with the running sums
//    and accumulators) only moves when some score exceeds it by more than
//    2^8 -- rare after the first step, and the final o / l is unchanged.
//  * PV: lane = (token group, dim): token group (lane / 16) = 8 tokens of
//    one page, dims (lane % 16) + 16 k for k = 0..7; the group's 8 bf16
//    weights per head come from this wave's LDS row and pair with the d-major
//    value chunk in v_dot2_f32_bf16.  The four token groups are summed once,
//    at the end.
// Tokens past the partition's end are masked (-inf scores, zeroed value
// chunks); pages wholly past it re-read the step's first page (served from
// L2) so every wave issues the same number of copies per step.  Block ids of
// the first 64 pages of the partition are read once, into one register.
// Attention of W * GW query rows over tokens [part_start, part_end) of one
// block-table row, for kv head g: the pages stream through the LDS ring and
// wave w serves local queries w*GW .. w*GW+GW-1.  qrow_of(i) gives local query
// i's row; dest_of(i, out_off, part_row) where its result goes: the output
// row at element offset out_off (>= 0), or partial row part_row (>= 0) of the
// workspace, or nowhere (both -1).
template <int GW, int R, int W, typename QRow, typename Dest>
__device__ __forceinline__ void group_range(
    pa::ring::StepBuf (&buf)[R], uint4 (&p_lds)[W][GW][4], uint16_t* __restrict__ out,
    Partials ws, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ bt_row, int32_t num_kv_heads, int g, int part_start, int part_end,
    float scale_log2, QRow qrow_of, Dest dest_of) {
  using namespace pa::ring;
  constexpr float kLazy = 8.f;  // log2 units
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nsteps = (part_end - part_start + kStep - 1) / kStep;
  const int npages = (part_end - part_start + kBS - 1) / kBS;
  const int lb_part = part_start / kBS;
  const int half = lane & 1;        // QK: which 64 dims
  const int tok = lane >> 1;        // QK: token of the step
  const int tg = lane >> 4;         // PV: token group (page tg / 2, tokens 8 * (tg % 2) ..)
  const int dl = lane & 15;         // PV: dims dl + 16 k
  int ids = bt_row[lb_part + min(lane, npages - 1)];  // block ids of pages 0..63
  uint4 qreg[GW][8];
#pragma unroll
  for (int h = 0; h < GW; ++h) {
    const uint16_t* qrow = qrow_of(wave * GW + h) + 64 * half;
#pragma unroll
    for (int c = 0; c < 8; ++c) qreg[h][c] = *reinterpret_cast<const uint4*>(qrow + 8 * c);
  }
  // consume these loads before the copies start (loads retire in order: a
  // wait for them inside the loop would also drain the copies in flight)
  asm volatile("" : "+v"(ids));
#pragma unroll
  for (int h = 0; h < GW; ++h)
#pragma unroll
    for (int c = 0; c < 8; ++c)
      asm volatile("" : "+v"(qreg[h][c].x), "+v"(qreg[h][c].y), "+v"(qreg[h][c].z),
                   "+v"(qreg[h][c].w));

  const int64_t blk_stride = static_cast<int64_t>(num_kv_heads) * kPageElems;
  const int64_t head_off = static_cast<int64_t>(g) * kPageElems;
  auto issue = [&](int step) {
    int pi = step * kPages + page_of<W>(wave);  // page of the partition
    if (pi >= npages) pi = step * kPages;  // past the end: the step's first page
    const int phys = pi < 64 ? __builtin_amdgcn_readlane(ids, pi) : bt_row[lb_part + pi];
    issue_step<W>(buf[step % R], kc, vc, phys, blk_stride, head_off, wave, lane);
  };

  float m[GW], lsum[GW], acc[GW][8];
#pragma unroll
  for (int h = 0; h < GW; ++h) {
    m[h] = -INFINITY;
    lsum[h] = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[h][k] = 0.f;
  }

  for (int st = 0; st < R - 1 && st < nsteps; ++st) issue(st);

  const int kofs = ((tok >> 4) * 16 + 8 * half) * 16;  // page and chunk base of the key reads
  // One step; TAIL marks the last one, the only step that can hold tokens at
  // or past the partition's end.
  auto do_step = [&](int step, auto tail_tag) {
    constexpr bool TAIL = decltype(tail_tag)::value;
    const StepBuf& B = buf[step % R];
    wait_step<R, W>(min(R - 2, nsteps - 1 - step));
    // the buffer written next was last read in the previous step, which every
    // wave has finished (barrier above)
    if (!TAIL && step + R - 1 < nsteps) issue(step + R - 1);
    const int t0 = part_start + step * kStep;

    // ---- scores
    float sc[GW];
#pragma unroll
    for (int h = 0; h < GW; ++h) sc[h] = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint4 kv = B.k[kofs + c * 16 + kslot(8 * half + c, tok & 15)];
#pragma unroll
      for (int h = 0; h < GW; ++h) {
        float a = sc[h];
        a = pa::dot2_bf16(qreg[h][c].x, kv.x, a);
        a = pa::dot2_bf16(qreg[h][c].y, kv.y, a);
        a = pa::dot2_bf16(qreg[h][c].z, kv.z, a);
        a = pa::dot2_bf16(qreg[h][c].w, kv.w, a);
        sc[h] = a;
      }
    }
#pragma unroll
    for (int h = 0; h < GW; ++h) {
      const float full = sc[h] + pa::dpp<pa::kDppXor1>(sc[h]);  // same bits in both lanes
      float sv = full * scale_log2;
      if (TAIL && t0 + tok >= part_end) sv = -INFINITY;
      float m_new = m[h];
      if (__any(sv > m[h] + kLazy)) m_new = fmaxf(m[h], pa::wave_max_u(sv));  // wave-uniform
      // rescale unconditionally (by exactly 1 when the reference stays): a
      // branch here would make the compiler copy every accumulator
      const float alpha = m_new == m[h] ? 1.f : pa::fast_exp2(m[h] - m_new);
      lsum[h] *= alpha;
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[h][k] *= alpha;
      m[h] = m_new;
      const float p = pa::fast_exp2(sv - m[h]);
      lsum[h] += p;  // every token counted twice (both halves)
      reinterpret_cast<uint16_t*>(&p_lds[wave][h][0])[tok] =
          static_cast<uint16_t>(pa::f32_to_bf16_bits(p));
    }
    lds_wave_sync();

    // ---- weighted values
    const int keep = part_end - (t0 + 8 * tg);  // valid tokens of this lane's group
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int d = dl + 16 * k;
      uint4 vv = B.v[(tg >> 1) * 256 + d * 2 + vhalf(d, tg & 1)];
      if (TAIL) vv = mask_chunk<uint16_t>(vv, keep);
#pragma unroll
      for (int h = 0; h < GW; ++h) {
        const uint4 pw = p_lds[wave][h][tg];
        float a = acc[h][k];
        a = pa::dot2_bf16(pw.x, vv.x, a);
        a = pa::dot2_bf16(pw.y, vv.y, a);
        a = pa::dot2_bf16(pw.z, vv.z, a);
        a = pa::dot2_bf16(pw.w, vv.w, a);
        acc[h][k] = a;
      }
    }
    lds_wave_sync();  // p_lds is rewritten by the next step
  };
  for (int step = 0; step < nsteps - 1; ++step) do_step(step, std::false_type{});
  do_step(nsteps - 1, std::true_type{});

  // ---- sum the four token groups; write the output or a partial
#pragma unroll
  for (int h = 0; h < GW; ++h) {
    const float lt = 0.5f * pa::wave_sum_u(lsum[h]);
    const float inv = 1.f / lt;
    int64_t out_off, part_row;
    dest_of(wave * GW + h, out_off, part_row);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float a = acc[h][k];
      a += __shfl_xor(a, 16, 64);
      a += __shfl_xor(a, 32, 64);
      const int d = dl + 16 * k;
      if (tg == 0) {
        if (out_off >= 0)
          out[out_off + d] = static_cast<uint16_t>(pa::f32_to_bf16_bits(a * inv));
        else if (part_row >= 0)
          ws.o[part_row * kD + d] = a * inv;
      }
    }
    if (part_row >= 0 && lane == 0) {
      ws.ml[2 * part_row] = m[h];
      ws.ml[2 * part_row + 1] = lt;
    }
  }
}

template <int GW, int R, int W>
__device__ __forceinline__ void group_item(
    uint32_t li, pa::ring::StepBuf (&buf)[R], uint4 (&p_lds)[W][GW][4],
    uint16_t* __restrict__ out, Partials ws, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ context_lens, int32_t num_seqs, int32_t num_heads,
    int32_t num_kv_heads, int32_t num_parts, int32_t partition, float scale_log2,
    RangeSplit rs) {
  constexpr int G = W * GW;
  // same logical order as decode_kernel: kv head fastest, then sequence, then
  // partition
  const int g = static_cast<int>(li % static_cast<uint32_t>(num_kv_heads));
  const uint32_t ps = li / static_cast<uint32_t>(num_kv_heads);
  const int s = static_cast<int>(ps % static_cast<uint32_t>(num_seqs));
  const int part = static_cast<int>(ps / static_cast<uint32_t>(num_seqs));
  if (part >= num_parts) return;

  const int h0 = g * G;
  const int L = context_lens[s];
  const int64_t row0 = static_cast<int64_t>(s) * num_heads + h0;  // (seq, head) row of query 0
  if (L <= 0) {
    if (part == 0)
      for (int i = threadIdx.x; i < G * pa::ring::kD; i += W * 64) out[row0 * pa::ring::kD + i] = 0;
    return;
  }
  const int begin = rs.starts ? split_begin(rs.starts[s], L) : 0;
  const int part_start = begin + part * partition;
  if (part_start >= L) return;
  const bool whole = (rs.starts ? split_parts(begin, L, partition, rs.pre_partition)
                                : (L + partition - 1) / partition) == 1;
  const int part_base = rs.part_base;
  group_range<GW, R, W>(
      buf, p_lds, out, ws, kc, vc, block_tables + static_cast<int64_t>(s) * max_blocks,
      num_kv_heads, g, part_start, min(part_start + partition, L), scale_log2,
      [&](int i) { return q + (row0 + i) * pa::ring::kD; },
      [&](int i, int64_t& out_off, int64_t& part_row) {
        out_off = whole ? (row0 + i) * pa::ring::kD : -1;
        part_row = whole ? -1 : (row0 + i) * num_parts + part_base + part;
      });
}

// One workgroup per item (partition, sequence, kv head), in the one-wave
// kernel's order.
#ifndef PA_GROUP_RING
#define PA_GROUP_RING 3
#endif
constexpr int kGroupRing = PA_GROUP_RING;  // 3 x 16 KB: three workgroups per CU

template <int GW, int W>
__global__ __launch_bounds__(W * 64) void decode_group_kernel(
    uint16_t* __restrict__ out, Partials ws, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ context_lens, int32_t num_seqs, int32_t num_heads,
    int32_t num_kv_heads, int32_t num_parts, int32_t partition, float scale_log2,
    RangeSplit rs) {
  __shared__ pa::ring::StepBuf buf[kGroupRing];
  __shared__ uint4 p_lds[W][GW][4];  // per wave and head: 32 bf16 weights
  group_item<GW, kGroupRing, W>(blockIdx.x, buf, p_lds, out, ws, q, kc, vc, block_tables,
                                max_blocks, context_lens, num_seqs, num_heads, num_kv_heads,
                                num_parts, partition, scale_log2, rs);
}

// Shared-prefix pass (bf16, head_dim 128).  Prefix group i is `count`
// consecutive sequences starting at `first` whose block tables hold the same
// physical blocks for the first `prefix` tokens (a multiple of the block
// size) -- the samples of one prompt after a fork, or requests whose prompts
// matched the same cached blocks.  Those tokens' K/V pages are read once, from
// the first member's table, for the queries of every member: one workgroup
// per (partition of the prefix, group, chunk of 8 queries, kv head), kv head
// fastest, the queries of a kv head ordered (member, head within the kv
// head's group).  Each query's partial result goes to partial slot `part` of
// its (sequence, head) row, or straight to the output when the prefix is the
// sequence's whole context and fits one partition.
constexpr int kPrefixMembers = PA_PREFIX_MAX_MEMBERS;

template <int GW, int W>
__global__ __launch_bounds__(W * 64) void decode_prefix_kernel(
    uint16_t* __restrict__ out, Partials ws, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ groups,
    int32_t num_groups, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
    int32_t num_parts, int32_t prefix_parts, int32_t partition, float scale_log2) {
  constexpr int Q = W * GW;  // queries per workgroup
  __shared__ pa::ring::StepBuf buf[kGroupRing];
  __shared__ uint4 p_lds[W][GW][4];
  const int gq_heads = num_heads / num_kv_heads;
  const int nchunks = (kPrefixMembers * gq_heads + Q - 1) / Q;
  uint32_t li = blockIdx.x;
  const int g = static_cast<int>(li % static_cast<uint32_t>(num_kv_heads));
  li /= static_cast<uint32_t>(num_kv_heads);
  const int chunk = static_cast<int>(li % static_cast<uint32_t>(nchunks));
  li /= static_cast<uint32_t>(nchunks);
  const int gi = static_cast<int>(li % static_cast<uint32_t>(num_groups));
  const int part = static_cast<int>(li / static_cast<uint32_t>(num_groups));
  if (part >= prefix_parts) return;

  const int first = groups[3 * gi];
  const int count = min(min(groups[3 * gi + 1], kPrefixMembers), num_seqs - first);
  if (first < 0 || count <= 0) return;
  const int P = split_begin(groups[3 * gi + 2], context_lens[first]);
  const int part_start = part * partition;
  const int nq = count * gq_heads;
  const int q0 = chunk * Q;
  if (part_start >= P || q0 >= nq) return;
  const int n_pre = (P + partition - 1) / partition;
  // (sequence, head) row of the chunk's local query i
  auto row_of = [&](int i) -> int64_t {
    const int gq = min(q0 + i, nq - 1);
    const int s = first + gq / gq_heads;
    return static_cast<int64_t>(s) * num_heads + g * gq_heads + gq % gq_heads;
  };
  group_range<GW, kGroupRing, W>(
      buf, p_lds, out, ws, kc, vc, block_tables + static_cast<int64_t>(first) * max_blocks,
      num_kv_heads, g, part_start, min(part_start + partition, P), scale_log2,
      [&](int i) { return q + row_of(i) * pa::ring::kD; },
      [&](int i, int64_t& out_off, int64_t& part_row) {
        out_off = -1;
        part_row = -1;
        if (q0 + i >= nq) return;
        const int64_t row = row_of(i);
        const int s = first + (q0 + i) / gq_heads;
        if (n_pre == 1 && context_lens[s] <= P)
          out_off = row * pa::ring::kD;
        else
          part_row = row * num_parts + part;
      });
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
    int32_t num_parts, int32_t partition, RangeSplit rs) {
  constexpr int PER = D / 64;
  typedef float vec_t __attribute__((ext_vector_type(PER)));
  const int lane = threadIdx.x;
  const int64_t row = blockIdx.x;  // seq * num_heads + head
  const int s = static_cast<int>(row / num_heads);
  const int L = context_lens[s];
  if (L <= 0) return;
  const int begin = rs.starts ? split_begin(rs.starts[s], L) : 0;
  const int n_pre = rs.starts ? (begin + rs.pre_partition - 1) / rs.pre_partition : 0;
  const int n_rest = (L - begin + partition - 1) / partition;
  const int part_base = rs.part_base;
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

constexpr size_t kAlign = 256;
#ifndef PA_GROUP_WAVES8
#define PA_GROUP_WAVES8 4
#endif
constexpr int kGroupWaves8 = PA_GROUP_WAVES8;  // waves per workgroup for 8-head groups

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// partial outputs | (m, l) pairs, each region 256-byte aligned
size_t ws_bytes(int64_t B, int64_t H, int64_t D, int64_t parts) {
  if (parts <= 1) return 0;
  return align_up(static_cast<size_t>(B * H * parts * D) * sizeof(float)) +
         static_cast<size_t>(B * H * parts * 2) * sizeof(float);
}

Partials carve(void* ws, int64_t B, int64_t H, int64_t D, int64_t slots) {
  Partials p{nullptr, nullptr};
  if (slots > 1) {
    uint8_t* base = static_cast<uint8_t*>(ws);
    p.o = reinterpret_cast<float*>(base);
    base += align_up(static_cast<size_t>(B * H * slots * D) * sizeof(float));
    p.ml = reinterpret_cast<float*>(base);
  }
  return p;
}

// Where a decode call's partitions go: `slots` partial slots per (sequence,
// head) row; the first pass covers tokens [starts[s], L) (from 0 when starts
// is null) in up to `parts` partitions written from slot part_base on.
struct Split {
  int32_t slots;
  int32_t parts;
  RangeSplit rs;
};

template <typename T, int D, int G, bool PVB>
int launch_decode(void* out, const void* q, const void* kc, const void* vc, const int32_t* bt,
                  int32_t max_blocks, const int32_t* lens, int32_t B, int32_t H, int32_t KVH,
                  Split sp, int32_t partition, float scale_log2, void* ws, hipStream_t st) {
  const Partials p = carve(ws, B, H, D, sp.slots);
  const int64_t grid = static_cast<int64_t>(sp.parts) * KVH * B;
  if constexpr (sizeof(T) == 2 && D == 128 && (G == 4 || G == 8)) {
    constexpr int W = G == 8 ? kGroupWaves8 : 4;
    hipLaunchKernelGGL((decode_group_kernel<G / W, W>), dim3(static_cast<uint32_t>(grid)),
                       dim3(W * 64), 0, st, static_cast<uint16_t*>(out), p,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kc),
                       static_cast<const uint16_t*>(vc), bt, max_blocks, lens, B, H, KVH, sp.slots,
                       partition, scale_log2, sp.rs);
  } else {
    hipLaunchKernelGGL((decode_kernel<T, D, G, PVB>), dim3(static_cast<uint32_t>(grid)), dim3(64),
                       0, st, static_cast<T*>(out), p, static_cast<const T*>(q),
                       static_cast<const T*>(kc), static_cast<const T*>(vc), bt, max_blocks, lens,
                       B, H, KVH, sp.slots, partition, scale_log2, sp.rs);
  }
  if (sp.slots > 1)
    hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3(static_cast<uint32_t>(B) * H), dim3(64),
                       0, st, static_cast<T*>(out), p, lens, H, sp.slots, partition, sp.rs);
  return pa_launch_status();
}

template <typename T, int D>
int dispatch_group(int G, void* out, const void* q, const void* kc, const void* vc,
                   const int32_t* bt, int32_t mb, const int32_t* lens, int32_t B, int32_t H,
                   int32_t KVH, Split sp, int32_t partition, float sl2, void* ws,
                   hipStream_t st) {
  constexpr bool kBf = sizeof(T) == 2;
  switch (G) {
    case 1: return launch_decode<T, D, 1, false>(out, q, kc, vc, bt, mb, lens, B, H, KVH, sp, partition, sl2, ws, st);
    case 2: return launch_decode<T, D, 2, false>(out, q, kc, vc, bt, mb, lens, B, H, KVH, sp, partition, sl2, ws, st);
    case 4: return launch_decode<T, D, 4, kBf>(out, q, kc, vc, bt, mb, lens, B, H, KVH, sp, partition, sl2, ws, st);
    case 8: return launch_decode<T, D, 8, kBf>(out, q, kc, vc, bt, mb, lens, B, H, KVH, sp, partition, sl2, ws, st);
    default: return PA_ERR_UNSUPPORTED;
  }
}

int64_t parts_for(int32_t max_context_len, int32_t partition) {
  if (partition <= 0) return 1;
  return max_context_len <= 0 ? 1 : (static_cast<int64_t>(max_context_len) + partition - 1) / partition;
}

}  // namespace

extern "C" size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                            int32_t max_context_len, int32_t partition) {
  if (num_seqs <= 0 || num_heads <= 0 || head_dim <= 0) return 0;
  return ws_bytes(num_seqs, num_heads, head_dim, parts_for(max_context_len, partition));
}

extern "C" int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         int32_t num_blocks, float scale, int32_t partition,
                         int32_t max_context_len, void* workspace, size_t workspace_bytes,
                         int32_t dtype, void* stream) {
  if (dtype != PA_F32 && dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0 ||
      num_blocks <= 0 || partition < 0 || max_context_len < 0)
    return PA_ERR_INVALID_ARG;
  if (num_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (block_size != kBS || (head_dim != 64 && head_dim != 128)) return PA_ERR_UNSUPPORTED;
  if (partition % kTile != 0) return PA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * kBS)
    return PA_ERR_INVALID_ARG;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return PA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_cache) |
       reinterpret_cast<uintptr_t>(v_cache)) & 15)
    return PA_ERR_INVALID_ARG;
  // One pass when unpartitioned: a single "partition" covering the longest
  // context, rounded up to whole tiles.
  int32_t part = partition;
  if (part == 0) part = static_cast<int32_t>(((std::max(max_context_len, 1) + kTile - 1) / kTile) * kTile);
  const int64_t parts = parts_for(max_context_len, part);
  if (parts > 0x7fffffff) return PA_ERR_INVALID_ARG;
  const size_t need = ws_bytes(num_seqs, num_heads, head_dim, parts);
  if (static_cast<int64_t>(parts) * num_kv_heads * num_seqs > 0x7fffffffLL)
    return PA_ERR_INVALID_ARG;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return PA_ERR_WORKSPACE;
  const int G = num_heads / num_kv_heads;
  const float sl2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const Split sp{static_cast<int32_t>(parts), static_cast<int32_t>(parts), {nullptr, 0, part}};
  if (dtype == PA_BF16) {
    if (head_dim == 128)
      return dispatch_group<uint16_t, 128>(G, out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs, num_heads, num_kv_heads, sp, part, sl2, workspace, st);
    return dispatch_group<uint16_t, 64>(G, out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs, num_heads, num_kv_heads, sp, part, sl2, workspace, st);
  }
  if (head_dim == 128)
    return dispatch_group<float, 128>(G, out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs, num_heads, num_kv_heads, sp, part, sl2, workspace, st);
  return dispatch_group<float, 64>(G, out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs, num_heads, num_kv_heads, sp, part, sl2, workspace, st);
}

namespace {

// The prefix pass works in partitions twice as long as the rest's: its
// workgroups then keep their copy pipeline full for longer (measured 4%
// faster on 8-sample groups with a 1024-token prefix than equal partitions;
// four times as long gained nothing more).
constexpr int kPrefixPartMult = 2;

// Partition of a shared prefix, in tokens, for the rest's partition `part`.
int32_t prefix_partition(int32_t part) {
  return static_cast<int32_t>(
      std::min<int64_t>(static_cast<int64_t>(part) * kPrefixPartMult, 0x40000000));
}

// Partial slots of a shared-prefix call: the prefix's partitions, then the
// rest's.
void shared_slots(int32_t max_context_len, int32_t max_prefix_len, int32_t part, int64_t& pre,
                  int64_t& rest) {
  pre = max_prefix_len > 0 ? parts_for(max_prefix_len, prefix_partition(part)) : 0;
  rest = parts_for(max_context_len, part);
}

int32_t unsplit_partition(int32_t partition, int32_t max_context_len) {
  if (partition != 0) return partition;
  return static_cast<int32_t>(((std::max(max_context_len, 1) + kTile - 1) / kTile) * kTile);
}

}  // namespace

extern "C" size_t pa_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_heads,
                                                          int32_t head_dim,
                                                          int32_t max_context_len,
                                                          int32_t max_prefix_len,
                                                          int32_t partition) {
  if (num_seqs <= 0 || num_heads <= 0 || head_dim <= 0 || partition < 0) return 0;
  int64_t pre, rest;
  shared_slots(max_context_len, max_prefix_len, unsplit_partition(partition, max_context_len), pre,
               rest);
  return ws_bytes(num_seqs, num_heads, head_dim, pre + rest);
}

extern "C" int pa_decode_shared_prefix(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t num_blocks, float scale, int32_t partition,
    int32_t max_context_len, const int32_t* prefix_groups, int32_t num_groups,
    const int32_t* seq_prefix_lens, int32_t max_prefix_len, void* workspace,
    size_t workspace_bytes, int32_t dtype, void* stream) {
  if (dtype != PA_F32 && dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0 ||
      num_blocks <= 0 || partition < 0 || max_context_len < 0 || num_groups < 0 ||
      max_prefix_len < 0)
    return PA_ERR_INVALID_ARG;
  if (num_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (dtype != PA_BF16 || block_size != kBS || head_dim != 128) return PA_ERR_UNSUPPORTED;
  const int G = num_heads / num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return PA_ERR_UNSUPPORTED;
  if (partition % kTile != 0 || max_prefix_len % kBS != 0 || max_prefix_len > max_context_len)
    return PA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * kBS)
    return PA_ERR_INVALID_ARG;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return PA_ERR_INVALID_ARG;
  const bool split = num_groups > 0 && max_prefix_len > 0;
  if (split && (!prefix_groups || !seq_prefix_lens)) return PA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_cache) |
       reinterpret_cast<uintptr_t>(v_cache)) & 15)
    return PA_ERR_INVALID_ARG;
  const int32_t part = unsplit_partition(partition, max_context_len);
  int64_t pre, rest;
  shared_slots(max_context_len, split ? max_prefix_len : 0, part, pre, rest);
  const int64_t slots = pre + rest;
  const int64_t nchunks = (static_cast<int64_t>(kPrefixMembers) * G + 7) / 8;
  if (slots > 0x7fffffff || rest * num_kv_heads * num_seqs > 0x7fffffffLL ||
      pre * num_groups * nchunks * num_kv_heads > 0x7fffffffLL)
    return PA_ERR_INVALID_ARG;
  const size_t need = ws_bytes(num_seqs, num_heads, head_dim, slots);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return PA_ERR_WORKSPACE;
  const float sl2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (split) {
    const Partials p = carve(workspace, num_seqs, num_heads, 128, slots);
    const int64_t grid = pre * num_groups * nchunks * num_kv_heads;
    hipLaunchKernelGGL((decode_prefix_kernel<2, 4>), dim3(static_cast<uint32_t>(grid)), dim3(256),
                       0, st, static_cast<uint16_t*>(out), p, static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(k_cache),
                       static_cast<const uint16_t*>(v_cache), block_tables, max_blocks_per_seq,
                       context_lens, prefix_groups, num_groups, num_seqs, num_heads, num_kv_heads,
                       static_cast<int32_t>(slots), static_cast<int32_t>(pre),
                       prefix_partition(part), sl2);
    const int rc = pa_launch_status();
    if (rc != PA_OK) return rc;
  }
  const Split sp{static_cast<int32_t>(slots), static_cast<int32_t>(rest),
                 {split ? seq_prefix_lens : nullptr, static_cast<int32_t>(pre),
                  prefix_partition(part)}};
  return dispatch_group<uint16_t, 128>(G, out, q, k_cache, v_cache, block_tables,
                                       max_blocks_per_seq, context_lens, num_seqs, num_heads,
                                       num_kv_heads, sp, part, sl2, workspace, st);
}
