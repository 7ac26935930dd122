// Decode attention over a paged KV cache (gfx950): the kernels and the
// pa_decode / pa_decode_shared_prefix entry points.  The one-wave item body is
// in decode_core.h.

#include "decode_core.h"

namespace {

// One wave (one 64-thread workgroup) per item.
template <typename T, int D, int G, bool PVB, int BS>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void decode_kernel(
    T* __restrict__ out, Partials ws, const T* __restrict__ q, const T* __restrict__ kc,
    const T* __restrict__ vc, const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ context_lens, int32_t num_seqs, int32_t num_heads,
    int32_t num_kv_heads, int32_t num_parts, int32_t partition, float scale_log2,
    RangeSplit rs) {
  __shared__ __attribute__((aligned(16))) weight_t<PVB> p_lds[G * kTile];
  decode_item<T, D, G, PVB, BS>(blockIdx.x, p_lds, out, ws, q, kc, vc, block_tables,
                                max_blocks, context_lens, num_seqs, num_heads, num_kv_heads,
                                num_parts, partition, scale_log2, rs);
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

#ifndef PA_GROUP_WAVES8
#define PA_GROUP_WAVES8 4
#endif
constexpr int kGroupWaves8 = PA_GROUP_WAVES8;  // waves per workgroup for 8-head groups

// Where a decode call's partitions go: `slots` partial slots per (sequence,
// head) row; the first pass covers tokens [starts[s], L) (from 0 when starts
// is null) in up to `parts` partitions written from slot part_base on.
struct Split {
  int32_t slots;
  int32_t parts;
  RangeSplit rs;
};

template <typename T, int D, int G, bool PVB, int BS>
int launch_decode(void* out, const void* q, const void* kc, const void* vc, const int32_t* bt,
                  int32_t max_blocks, const int32_t* lens, int32_t B, int32_t H, int32_t KVH,
                  Split sp, int32_t partition, float scale_log2, void* ws, hipStream_t st) {
  const Partials p = carve(ws, B, H, D, sp.slots);
  const int64_t grid = static_cast<int64_t>(sp.parts) * KVH * B;
  if constexpr (BS == kBS && sizeof(T) == 2 && D == 128 && (G == 4 || G == 8)) {
    constexpr int W = G == 8 ? kGroupWaves8 : 4;
    hipLaunchKernelGGL((decode_group_kernel<G / W, W>), dim3(static_cast<uint32_t>(grid)),
                       dim3(W * 64), 0, st, static_cast<uint16_t*>(out), p,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kc),
                       static_cast<const uint16_t*>(vc), bt, max_blocks, lens, B, H, KVH, sp.slots,
                       partition, scale_log2, sp.rs);
  } else {
    hipLaunchKernelGGL((decode_kernel<T, D, G, PVB, BS>), dim3(static_cast<uint32_t>(grid)), dim3(64),
                       0, st, static_cast<T*>(out), p, static_cast<const T*>(q),
                       static_cast<const T*>(kc), static_cast<const T*>(vc), bt, max_blocks, lens,
                       B, H, KVH, sp.slots, partition, scale_log2, sp.rs);
  }
  if (sp.slots > 1)
    hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3(static_cast<uint32_t>(B) * H), dim3(64),
                       0, st, static_cast<T*>(out), p, lens, H, sp.slots, partition, sp.rs);
  return pa_launch_status();
}

template <typename T, int D, int BS = kBS>
int dispatch_group(int G, void* out, const void* q, const void* kc, const void* vc,
                   const int32_t* bt, int32_t mb, const int32_t* lens, int32_t B, int32_t H,
                   int32_t KVH, Split sp, int32_t partition, float sl2, void* ws,
                   hipStream_t st) {
  constexpr bool kBf = sizeof(T) == 2;
  switch (G) {
    case 1: return launch_decode<T, D, 1, false, BS>(out, q, kc, vc, bt, mb, lens, B, H, KVH, sp, partition, sl2, ws, st);
    case 2: return launch_decode<T, D, 2, false, BS>(out, q, kc, vc, bt, mb, lens, B, H, KVH, sp, partition, sl2, ws, st);
    case 4: return launch_decode<T, D, 4, kBf, BS>(out, q, kc, vc, bt, mb, lens, B, H, KVH, sp, partition, sl2, ws, st);
    case 8: return launch_decode<T, D, 8, kBf, BS>(out, q, kc, vc, bt, mb, lens, B, H, KVH, sp, partition, sl2, ws, st);
    default: return PA_ERR_UNSUPPORTED;
  }
}

// dtype and head_dim dispatch for one block size
template <int BS>
int dispatch_block(int32_t dtype, int32_t head_dim, int G, void* out, const void* q,
                   const void* kc, const void* vc, const int32_t* bt, int32_t mb,
                   const int32_t* lens, int32_t B, int32_t H, int32_t KVH, Split sp,
                   int32_t partition, float sl2, void* ws, hipStream_t st) {
  if (dtype == PA_BF16) {
    if (head_dim == 128)
      return dispatch_group<uint16_t, 128, BS>(G, out, q, kc, vc, bt, mb, lens, B, H, KVH, sp, partition, sl2, ws, st);
    return dispatch_group<uint16_t, 64, BS>(G, out, q, kc, vc, bt, mb, lens, B, H, KVH, sp, partition, sl2, ws, st);
  }
  if (head_dim == 128)
    return dispatch_group<float, 128, BS>(G, out, q, kc, vc, bt, mb, lens, B, H, KVH, sp, partition, sl2, ws, st);
  return dispatch_group<float, 64, BS>(G, out, q, kc, vc, bt, mb, lens, B, H, KVH, sp, partition, sl2, ws, st);
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
  if ((block_size != 8 && block_size != 16 && block_size != 32 && block_size != 64) ||
      (head_dim != 64 && head_dim != 128))
    return PA_ERR_UNSUPPORTED;
  if (partition % kTile != 0) return PA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * block_size)
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
#define PA_DECODE_BS(BSZ)                                                                      \
  dispatch_block<BSZ>(dtype, head_dim, G, out, q, k_cache, v_cache, block_tables,              \
                      max_blocks_per_seq, context_lens, num_seqs, num_heads, num_kv_heads, sp, \
                      part, sl2, workspace, st)
  switch (block_size) {
    case 8: return PA_DECODE_BS(8);
    case 32: return PA_DECODE_BS(32);
    case 64: return PA_DECODE_BS(64);
    default: return PA_DECODE_BS(16);
  }
#undef PA_DECODE_BS
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
