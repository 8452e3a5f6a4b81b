// Device helpers shared by the attention kernels (internal): the LDS tile
// geometry of 1152-B rows, the global -> LDS DMA, the LDS transpose read, the
// lane-pair reductions of the 32x32 MFMA layouts, and cache-row addressing
// (contiguous or paged).
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

// Address of cache row r of sequence b.  Contiguous: slot b of `stride` rows.
// Paged: row r & (2^page_shift - 1) of pool page block_table[b][r >> page_shift];
// with pages of 32 rows or more, a run of rows that starts at a multiple of 16
// and ends inside the same 32-row tile stays in one page.  The table is
// read-only for the kernels, so an entry at a uniform index comes through a
// scalar load.  An entry outside [0, num_pages) sets ok = false and yields the
// pool base, which the caller must not read.
template <bool PAGED>
__device__ __forceinline__ uint64_t cache_row_addr(const void* cache, const int32_t* block_table, int64_t num_pages,
                                                   int32_t bt_stride, int32_t page_shift, int64_t stride, int b,
                                                   int64_t r, int64_t row_bytes, bool& ok) {
  const uint64_t base = reinterpret_cast<uint64_t>(cache);
  if constexpr (!PAGED) {
    ok = true;
    return base + static_cast<uint64_t>((static_cast<int64_t>(b) * stride + r) * row_bytes);
  } else {
    const auto* bt = (const __attribute__((address_space(4))) int32_t*)(block_table);
    const int32_t pg = bt[static_cast<int64_t>(b) * bt_stride + (r >> page_shift)];
    ok = pg >= 0 && pg < num_pages;
    const int64_t prow = (static_cast<int64_t>(ok ? pg : 0) << page_shift) + (r & ((int64_t{1} << page_shift) - 1));
    return base + static_cast<uint64_t>(prow * row_bytes);
  }
}

// Query n -> (sequence, attended length), the length clamped to [0, min(max_len, stride)].
__device__ __forceinline__ void query_range(const SplitArgs& a, int n, int& b, int64_t& len) {
  b = n / a.q_per_seq;
  int64_t L = a.prefill ? static_cast<int64_t>(a.lens[b]) + (n % a.q_per_seq) + 1
                        : static_cast<int64_t>(a.lens[b]);
  L = min(L, static_cast<int64_t>(a.max_len));
  L = min(L, a.stride);
  len = max(L, static_cast<int64_t>(0));
}

// Grids of more workgroups than this (one per compute unit of the MI355X's
// 256) take their decode units longest first.
constexpr unsigned LPT_MIN_GRID = 256;

// Exclusive prefix sum of v over a workgroup of 256 threads, in thread order;
// `total` gets the sum over the workgroup.  red: 4 ints of LDS.  Every thread
// of the workgroup must call it (it holds two barriers).
__device__ __forceinline__ int block_excl_scan256(int v, int* red, int& total) {
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (l >= o) x += y;
  }
  __syncthreads();  // red is free
  if (l == 63) red[w] = x;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = red[i];
    if (i < w) before += t;
    total += t;
  }
  return before + x - v;
}

// Longest-first order of the units of a decode launch.  Unit (query n, split s)
// covers min(max(len_n - s R, 0), R) rows, R = split_rows.  With more
// workgroups than the compute units hold at once, the hardware hands them out
// in order of their linear index as compute units free up, so with ragged
// lengths a long unit handed out late sets the end of the launch.  Workgroup
// k = x + X (y + Y z) of a grid (X, Y, G) takes the unit of rank k / G and head
// group k % G, the ranks running over
//   the full units (R rows), by query and then split;
//   the partial units (1 .. R-1 rows), longest first in 32 length classes
//     (class c holds the lengths with floor(32 rows / R) = 31 - c), by query
//     within a class;
//   the empty units, by query and then split.
// Each workgroup works the order out from the lengths (three scans), so the
// mapping adds no launch and no buffer; it is a permutation of the units.
// blockDim.x = 256; scratch: 48 ints of LDS, free again when it returns.
__device__ __forceinline__ void longest_first_unit(const SplitArgs& a, int* scratch, int& n_out, int& split_out,
                                                   int& g_out) {
  int* hist = scratch;       // [32] partial units per length class
  int* red = scratch + 32;   // [4] scan
  int* res = scratch + 40;   // [2] the unit found
  const int tid = threadIdx.x;
  const int G = gridDim.z;
  const int k = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  const int r = k / G;
  g_out = k - r * G;
  const int S = a.num_splits;
  const int64_t R = a.split_rows;
  const int c = (a.n_q + 255) / 256;  // queries per thread, contiguous
  const int n0 = min(tid * c, a.n_q), n1 = min(n0 + c, a.n_q);
  // full, partial and empty units of query n; the partial unit's length class
  auto counts = [&](int n, int& f, int& p, int& cls) {
    int b;
    int64_t L;
    query_range(a, n, b, L);
    f = static_cast<int>(min(L / R, static_cast<int64_t>(S)));
    const int64_t rem = L - f * R;  // < R when f < S
    p = (rem > 0 && f < S) ? 1 : 0;
    cls = p ? 31 - static_cast<int>(rem * 32 / R) : 0;
  };
  if (tid < 32) hist[tid] = 0;
  __syncthreads();
  int sF = 0, sE = 0;
  for (int n = n0; n < n1; ++n) {
    int f, p, cls;
    counts(n, f, p, cls);
    sF += f;
    sE += S - f - p;
    if (p) atomicAdd(&hist[cls], 1);
  }
  int F;
  const int exF = block_excl_scan256(sF, red, F);  // its barriers also publish hist
  if (r < F) {
    if (exF <= r && r < exF + sF) {
      int acc = exF;
      for (int n = n0; n < n1; ++n) {
        int f, p, cls;
        counts(n, f, p, cls);
        if (r < acc + f) {
          res[0] = n;
          res[1] = r - acc;
          break;
        }
        acc += f;
      }
    }
  } else {
    int P = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) P += hist[i];
    if (r < F + P) {
      const int j = r - F;
      int cb = 0, cum = 0;  // the class holding rank j, and the ranks before it
      while (j >= cum + hist[cb]) cum += hist[cb++];
      const int i = j - cum;
      int cnt = 0;
      for (int n = n0; n < n1; ++n) {
        int f, p, cls;
        counts(n, f, p, cls);
        cnt += (p && cls == cb) ? 1 : 0;
      }
      int tot;
      const int ex = block_excl_scan256(cnt, red, tot);
      if (ex <= i && i < ex + cnt) {
        int acc = ex;
        for (int n = n0; n < n1; ++n) {
          int f, p, cls;
          counts(n, f, p, cls);
          if (p && cls == cb) {
            if (acc == i) {
              res[0] = n;
              res[1] = f;
              break;
            }
            ++acc;
          }
        }
      }
    } else {
      const int j = r - F - P;
      int E;
      const int ex = block_excl_scan256(sE, red, E);
      if (ex <= j && j < ex + sE) {
        int acc = ex;
        for (int n = n0; n < n1; ++n) {
          int f, p, cls;
          counts(n, f, p, cls);
          const int e = S - f - p;
          if (j < acc + e) {
            res[0] = n;
            res[1] = f + p + (j - acc);
            break;
          }
          acc += e;
        }
      }
    }
  }
  __syncthreads();
  n_out = res[0];
  split_out = res[1];
  __syncthreads();  // scratch is free again
}

// Sum (or max) of v over the workgroup (blockDim.x a multiple of 64, up to 256).
__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max) {
  for (int o = 32; o > 0; o >>= 1) {
    const float u = __shfl_xor(v, o);
    v = is_max ? fmaxf(v, u) : v + u;
  }
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  v = red[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) v = is_max ? fmaxf(v, red[i]) : v + red[i];
  return v;
}

}  // namespace mla
