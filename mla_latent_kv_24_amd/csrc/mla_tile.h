// Device helpers shared by the attention kernels (internal): the LDS tile
// geometry of 1152-B rows, the global -> LDS DMA, the LDS transpose read, and
// the lane-pair reductions of the 32x32 MFMA layouts.
#pragma once
#include "mla_common.h"

namespace mla {

constexpr float NEG_INF = -__builtin_huge_valf();
constexpr float RESCALE_TAU = 8.0f;

// 16-byte chunk swizzle of tile row t: chunk k of the row lives at k ^ swz(t).
__device__ __forceinline__ int swz(int t) {
  const int m = (t >> 1) & 7;
  return ((m & 1) << 2) | (m >> 1);
}
// byte offset of element e of tile row t
__device__ __forceinline__ int tile_off(int t, int e) {
  return t * ROWB + 16 * ((e >> 3) ^ swz(t)) + 2 * (e & 7);
}

// s_waitcnt vmcnt(N) (gfx9 encoding; expcnt and lgkmcnt left at their maxima)
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
// One 16-B-per-lane global -> LDS copy: lane L's bytes from rsrc + soff + voff land
// at LDS address m0 + 16 L.  Issued from asm so that the compiler does not fence
// every later LDS read on it; the waits are explicit (vm_wait) at tile boundaries.
__device__ __forceinline__ void dma16(uint32_t lds_addr, int voff, i32x4 rsrc, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory", "m0");
}

__device__ __forceinline__ i16x4 tr_read(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
}
__device__ __forceinline__ bf16x8 cat(i16x4 a, i16x4 b) {
  struct {
    i16x4 lo, hi;
  } v = {a, b};
  return __builtin_bit_cast(bf16x8, v);
}

// Reductions over the lanes that hold the same head (lane ^ 32, and lane ^ 16
// for 16 heads per wave).  v_permlane32_swap / v_permlane16_swap (issued with
// the same value in both operands) return the lane's value and its partner's,
// so op(r[0], r[1]) is the pair result.  The empty asm pins both results in
// their registers: without it this compiler folds r[1] into r[0].
template <bool SWAP16>
__device__ __forceinline__ void pair_vals(float v, float& a, float& b) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  unsigned x, y;
  if constexpr (SWAP16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = r[0];
    y = r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    x = r[0];
    y = r[1];
  }
  asm volatile("" : "+v"(x), "+v"(y));
  a = __builtin_bit_cast(float, x);
  b = __builtin_bit_cast(float, y);
}
__device__ __forceinline__ float pair_max32(float v) { float a, b; pair_vals<false>(v, a, b); return fmaxf(a, b); }
__device__ __forceinline__ float pair_max16(float v) { float a, b; pair_vals<true>(v, a, b); return fmaxf(a, b); }
__device__ __forceinline__ float pair_sum32(float v) { float a, b; pair_vals<false>(v, a, b); return a + b; }
__device__ __forceinline__ float pair_sum16(float v) { float a, b; pair_vals<true>(v, a, b); return a + b; }

}  // namespace mla
