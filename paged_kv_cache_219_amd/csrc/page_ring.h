// LDS staging of paged K/V for the bf16, head_dim 128, 16-token-page cache.
//
// A "step" is two consecutive logical pages (32 tokens) of one (sequence,
// kv head): 8 KB of keys and 8 KB of values.  A workgroup of W waves (4
// or 8 waves) copies a step into one of the LDS buffers of a ring with
// direct-to-LDS loads (global_load_lds_dwordx4: lane i of a wave instruction
// lands at base + 16 i): 16 loads of 1 KB per step, shared evenly by the
// waves.  Loads run (ring size - 1) steps ahead of use; wait_step() waits for
// the oldest step's loads and the workgroup barrier then publishes it.
//
// LDS layout of one step, in 16-byte units:
//   k: [page][chunk 16][token slot 16]: the cache's own key page layout,
//      except that chunks 8..15 hold token t in slot t ^ 8 (kslot), so that 8
//      tokens' chunk c and the same tokens' chunk c + 8 fall in different banks
//   v: [page][dim 128][2 halves of 8 tokens], the halves of each dim row
//      swapped when (dim / 8) is odd (vhalf), so that 16 lanes reading one
//      half of 16 consecutive dims, or 32 dims x 8 bytes, hit distinct banks.
#pragma once

#include "pa_device.h"

namespace pa {
namespace ring {

constexpr int kBS = 16;
constexpr int kD = 128;
constexpr int kPages = 2;
constexpr int kStep = kPages * kBS;   // tokens per step
constexpr int kPageElems = kBS * kD;  // elements of one (block, kv head) page
constexpr int kRing = 3;  // 48 KB per workgroup: three workgroups share a CU's 160 KB

struct StepBuf {
  uint4 k[kPages * 256];
  uint4 v[kPages * 256];
};

// LDS half slot that holds global half `half` of dim row d (an involution).
__device__ __forceinline__ int vhalf(int d, int half) { return half ^ ((d >> 3) & 1); }

// LDS token slot of token t's key chunk c (an involution in t).
__device__ __forceinline__ int kslot(int c, int t) { return t ^ (c & 8); }

// 16-byte direct-to-LDS load: lane i's bytes land at LDS byte address
// lds_base + 16 i.  Issued through asm so the compiler does not pair every
// later LDS read with a wait for all outstanding copies; the kernels wait for
// them explicitly (wait_step) before the barrier that publishes a step.
__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds_base)
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p));
}

// Physical block of the page that wave `wave` of a W-wave workgroup copies
// for a step is page_of<W>(wave) of the step: each wave moves 8 / W runs of
// 64 units (1 KB) of keys and the same of values, all within one page.
template <int W>
__device__ __forceinline__ int page_of(int wave) {
  static_assert(W == 2 || W == 4 || W == 8, "2, 4 or 8 waves per workgroup");
  return wave / (W / 2);
}

// This wave's share of one step; `phys` is the physical block of its page.
template <int W = 4>
__device__ __forceinline__ void issue_step(StepBuf& B, const uint16_t* kc, const uint16_t* vc,
                                           int phys, int64_t blk_stride, int64_t head_off,
                                           int wave, int lane) {
  constexpr int kRuns = 8 / W;
  const uint16_t* kp = kc + phys * blk_stride + head_off;
  const uint16_t* vp = vc + phys * blk_stride + head_off;
#pragma unroll
  for (int i = 0; i < kRuns; ++i) {
    const int u0 = 64 * (kRuns * wave + i);  // wave-uniform base unit of the step
    const int pos = (u0 + lane) & 255;       // unit within the page
    const int d = pos >> 1;
    const int c = pos >> 4;
    lds_dma16(kp + (c * 16 + kslot(c, pos & 15)) * 8,
              __builtin_amdgcn_readfirstlane(lds_addr(&B.k[u0])));
    lds_dma16(vp + (d * 2 + vhalf(d, pos & 1)) * 8,
              __builtin_amdgcn_readfirstlane(lds_addr(&B.v[u0])));
  }
}

// Wait until this wave's loads of the current step have landed, leaving the
// `ahead` later steps (0..R-2) in flight, then barrier the workgroup.  R is
// the number of step buffers in the ring (loads run R - 1 steps ahead); each
// step is 16 / W loads per wave.
template <int R = kRing, int W = 4>
__device__ __forceinline__ void wait_step(int ahead) {
  static_assert(R >= 2 && R <= 4, "ring of 2 to 4 steps");
  constexpr int kPer = 16 / W;
  if (R == 4 && ahead >= 2) {
    if (kPer == 8) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else if (kPer == 4) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  } else if (ahead >= 1) {
    if (kPer == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else if (kPer == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace ring
}  // namespace pa
