// Device-side helpers shared by libpa's gfx950 kernels: bf16 bit handling,
// wave64 reductions, launch-error mapping.  CDNA4 only (wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pa.h"

namespace pa {

constexpr int kWave = 64;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// fp32 -> bf16 bits, round to nearest even (the hardware conversion,
// v_cvt_pk_bf16_f32 on gfx950; NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// Two fp32 -> packed bf16 pair (lo in bits 0..15), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// 16-byte global load of K/V page data.  NT: with the non-temporal hint, for
// pages that the call reads once (no page shared by several sequences): the
// decode kernels then stream 8-11% faster, but pages that several sequences
// share stop being served from the caches.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
template <bool NT>
__device__ __forceinline__ uint4 ld16_kv(const void* p) {
  if constexpr (NT)
    return __builtin_bit_cast(uint4,
                              __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
  else
    return *reinterpret_cast<const uint4*>(p);
}

// Low / high bf16 of a packed pair, widened exactly to fp32.
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __builtin_bit_cast(float, v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) {
  return __builtin_bit_cast(float, v & 0xffff0000u);
}

// acc + a.lo*b.lo + a.hi*b.hi on bf16 pairs with fp32 accumulation.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// DPP lane permutations within 16-lane rows (no LDS traffic).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <- 7-i within each 8
constexpr int kDppMirror = 0x140;      // lane i <- 15-i within each 16

__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Max / sum over the whole wave, returned wave-uniform.  Four DPP steps make
// every 16-lane row uniform (each step combines two equal-shaped partial
// results, so all lanes of a row get identical bits), then the four row
// values are combined in a fixed order.
__device__ __forceinline__ float wave_max_u(float v) {
  v = fmaxf(v, dpp<kDppXor1>(v));
  v = fmaxf(v, dpp<kDppXor2>(v));
  v = fmaxf(v, dpp<kDppHalfMirror>(v));
  v = fmaxf(v, dpp<kDppMirror>(v));
  return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)), fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}

__device__ __forceinline__ float wave_sum_u(float v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  v += dpp<kDppMirror>(v);
  return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace pa

// Map the state after a launch to a pa_status.
static inline int pa_launch_status() {
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_DEVICE;
}
