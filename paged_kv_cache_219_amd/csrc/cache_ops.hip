// Cache writes of libpa: scatter new tokens' K/V into their slots, and copy
// whole blocks for copy-on-write.  Pure data movement (bit-exact).
//
// Page "vLLM PagedAttention chuyên sâu: Phân mảnh bộ nhớ KV Cache, Prefill
// theo khối & Prefix Caching" (locionic.com): section "Tương tự phân trang bộ
// nhớ ảo" (new tokens land in newly mapped physical blocks, nothing moves),
// section "Cơ chế của Chunked Prefill" step 3 (a chunk's KV accumulates in
// the blocks the block manager hands out), section "Cơ chế APC" item 3
// (copy-on-write of a shared block before a diverging write).
//
// Layout (see include/pa.h): k_cache[NB][KVH][D/X][BS][X] with X elements per
// 16-byte chunk, v_cache[NB][KVH][D][BS].

#include "pa_device.h"

namespace {

// One 256-thread workgroup per (group of X consecutive tokens, kv head),
// X = 16 / element size: the number of tokens in one 16-byte unit of the
// d-major value page.  Waves 0-1 write the keys, waves 2-3 the values, so the
// two halves' loads and stores are in flight together.  Each thread issues its
// data loads before it needs a slot (only the stores' addresses depend on the
// slots), so the slot and data loads wait out one memory latency together.
//  * keys: the X tokens' rows as 16-byte chunks, each to its x-packed place;
//  * values: each thread holds one dimension of the X tokens; when the group's
//    slots are X consecutive slots starting at a multiple of X (the common
//    case when a chunk of a sequence is written) it stores them as one 16-byte
//    unit of the page, otherwise (scattered tokens, e.g. one new token per
//    sequence) one element per token.
template <int ESIZE>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const uint8_t* __restrict__ key, const uint8_t* __restrict__ value, uint8_t* __restrict__ kc,
    uint8_t* __restrict__ vc, const int64_t* __restrict__ slots, int32_t num_tokens,
    int64_t kstride_bytes, int64_t vstride_bytes, int32_t kvh, int32_t head_dim,
    int32_t block_size) {
  typedef typename std::conditional<ESIZE == 2, uint16_t, uint32_t>::type elem_t;
  constexpr int X = 16 / ESIZE;
  const int lane = threadIdx.x & 63;
  const int64_t grp = blockIdx.x / kvh;
  const int head = static_cast<int>(blockIdx.x % kvh);
  const int64_t tok0 = grp * X;
  if (tok0 >= num_tokens) return;
  const int ntok = static_cast<int>(min(static_cast<int64_t>(X), num_tokens - tok0));
  const int nchunk = head_dim * ESIZE / 16;

  // this group's slots, one per lane (lanes >= ntok hold -1), in every wave
  const int64_t my_slot = lane < ntok ? slots[tok0 + lane] : -1;

  if (threadIdx.x < 128) {
    // ---- keys (X * nchunk <= 128 units: one per thread at most)
    const int u = threadIdx.x;
    const int j = u / nchunk, c = u - (u / nchunk) * nchunk;
    const bool have = u < X * nchunk && j < ntok;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (have)
      v = *reinterpret_cast<const uint4*>(key + (tok0 + j) * kstride_bytes +
                                          static_cast<int64_t>(head) * head_dim * ESIZE + c * 16);
    const int64_t slot = __shfl(my_slot, j < X ? j : 0, 64);
    if (have && slot >= 0) {
      const int64_t blk = slot / block_size;
      const int off = static_cast<int>(slot % block_size);
      *reinterpret_cast<uint4*>(kc + ((((blk * kvh + head) * nchunk + c) * block_size) + off) * 16) =
          v;
    }
    return;
  }

  // ---- values (head_dim <= 128: one dimension per thread at most)
  const int d = threadIdx.x - 128;
  elem_t e[X];
#pragma unroll
  for (int j = 0; j < X; ++j) {
    e[j] = 0;
    if (d < head_dim && j < ntok)
      e[j] = reinterpret_cast<const elem_t*>(value + (tok0 + j) * vstride_bytes)
          [static_cast<int64_t>(head) * head_dim + d];
  }
  const int64_t s0 = __shfl(my_slot, 0, 64);
  const bool run = ntok == X && s0 >= 0 && s0 % X == 0 &&
                   __all(lane >= X || my_slot == s0 + lane);
  if (d >= head_dim) return;
  if (run) {
    const int64_t blk = s0 / block_size;
    const int off = static_cast<int>(s0 % block_size);
    elem_t* vpage = reinterpret_cast<elem_t*>(vc) + (blk * kvh + head) * head_dim * block_size + off;
    *reinterpret_cast<uint4*>(vpage + static_cast<int64_t>(d) * block_size) =
        __builtin_bit_cast(uint4, e);
  } else {
#pragma unroll
    for (int j = 0; j < X; ++j) {
      const int64_t slot = __shfl(my_slot, j, 64);
      if (j < ntok && slot >= 0) {
        const int64_t blk = slot / block_size;
        const int off = static_cast<int>(slot % block_size);
        reinterpret_cast<elem_t*>(vc)[(blk * kvh + head) * head_dim * block_size +
                                      static_cast<int64_t>(d) * block_size + off] = e[j];
      }
    }
  }
}

// grid (num_pairs, ceil(units / 256)); each thread copies one 16-byte unit of
// the K block and one of the V block.
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint4* __restrict__ kc,
                                                          uint4* __restrict__ vc,
                                                          const int32_t* __restrict__ pairs,
                                                          int64_t units_per_block) {
  const int64_t u = static_cast<int64_t>(blockIdx.y) * blockDim.x + threadIdx.x;
  if (u >= units_per_block) return;
  const int64_t src = pairs[2 * blockIdx.x];
  const int64_t dst = pairs[2 * blockIdx.x + 1];
  kc[dst * units_per_block + u] = kc[src * units_per_block + u];
  vc[dst * units_per_block + u] = vc[src * units_per_block + u];
}

int esize_of(int32_t dtype) { return dtype == PA_BF16 ? 2 : (dtype == PA_F32 ? 4 : 0); }

}  // namespace

extern "C" int pa_reshape_and_cache(const void* key, const void* value, void* k_cache,
                                    void* v_cache, const int64_t* slot_mapping, int32_t num_tokens,
                                    int64_t key_stride, int64_t value_stride, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                    int32_t dtype, void* stream) {
  const int es = esize_of(dtype);
  if (es == 0) return PA_ERR_UNSUPPORTED;
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return PA_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (block_size != 8 && block_size != 16 && block_size != 32 && block_size != 64)
    return PA_ERR_UNSUPPORTED;
  const int64_t row = static_cast<int64_t>(num_kv_heads) * head_dim;
  if (key_stride < row || value_stride < row) return PA_ERR_INVALID_ARG;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping) return PA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(key) | reinterpret_cast<uintptr_t>(k_cache) |
       reinterpret_cast<uintptr_t>(v_cache)) & 15)
    return PA_ERR_INVALID_ARG;
  if (((key_stride * es) & 15) != 0) return PA_ERR_INVALID_ARG;
  const int64_t groups = (static_cast<int64_t>(num_tokens) + 16 / es - 1) / (16 / es);
  const int64_t blocks = groups * num_kv_heads;
  if (blocks > 0x7fffffff) return PA_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (es == 2)
    hipLaunchKernelGGL(reshape_and_cache_kernel<2>, dim3(static_cast<uint32_t>(blocks)), dim3(256),
                       0, s, static_cast<const uint8_t*>(key), static_cast<const uint8_t*>(value),
                       static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache),
                       slot_mapping, num_tokens, key_stride * es, value_stride * es, num_kv_heads,
                       head_dim, block_size);
  else
    hipLaunchKernelGGL(reshape_and_cache_kernel<4>, dim3(static_cast<uint32_t>(blocks)), dim3(256),
                       0, s, static_cast<const uint8_t*>(key), static_cast<const uint8_t*>(value),
                       static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache),
                       slot_mapping, num_tokens, key_stride * es, value_stride * es, num_kv_heads,
                       head_dim, block_size);
  return pa_launch_status();
}

extern "C" int pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs,
                              int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, int32_t num_blocks, int32_t dtype, void* stream) {
  const int es = esize_of(dtype);
  if (es == 0) return PA_ERR_UNSUPPORTED;
  if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return PA_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (block_size != 8 && block_size != 16 && block_size != 32 && block_size != 64)
    return PA_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !pairs) return PA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache)) & 15)
    return PA_ERR_INVALID_ARG;
  const int64_t units = static_cast<int64_t>(num_kv_heads) * head_dim * block_size * es / 16;
  const int64_t gy = (units + 255) / 256;
  if (gy > 65535) return PA_ERR_INVALID_ARG;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(num_pairs, static_cast<uint32_t>(gy)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<uint4*>(k_cache),
                     static_cast<uint4*>(v_cache), pairs, units);
  return pa_launch_status();
}
