// A6 in the unabsorbed form -- causal prefill of MLA on gfx950.
//
// The attention of the absorbed path (jiphyeonjeon.kr DeepSeek-V2 review,
// sections 2-3), computed from per-head keys and values made explicit once
// for every cached row:
//   k^C_{j,i} = U^K_i c_j,  v^C_{j,i} = U^V_i c_j,  k_{j,i} = [k^C_{j,i}; k^R_j]
//   l_ij = [q^C_i; RoPE(q^R_i)] . k_{j,i} / sqrt(d_h + d_hR)
//   o_i  = sum_j softmax_j(l_ij) v^C_{j,i}
// A chunk of queries shares every key, so per (key, query, head) the score
// is a 192-deep product and the value a 128-wide one: 640 multiply-adds
// against the absorbed form's 1,088.  Two kernels:
//   expand_kv_kernel: per (sequence, 128-row block, 8 to 32 heads) an MFMA GEMM
//     [k^C; v^C] = [U^K_i; U^V_i] c^T with the rows' c staged in LDS; results
//     leave as hi/lo bf16 rows that keep the cache-row geometry (the layout
//     is in mla_common.h), with k^R copied in;
//   prefill_attn_kernel: per (sequence, head, 256 queries) a causal flash
//     attention over those rows, on the decode kernels' tile stream.
// Precision: a query that sees few keys has an output made of few terms, so
// one bf16 rounding of an operand shows in it at full size.  A workgroup
// whose first query sees fewer than precise_below keys takes hi + lo
// products for k^C, q^R, P and v^C (every operand to ~2^-16); the others
// take the hi parts alone.
#include "mla_common.h"
#include "mla_tile.h"

namespace mla {

// Attention MFMAs from asm, to fix the register files: the queries sit in
// AGPRs (B operand), the score and output accumulators in VGPRs, so that the
// rare rescale of the output is a plain multiply (with the accumulators in
// AGPRs the compiler copied all of them out and back on every tile).  The
// compiler does not see these as MFMAs, so each starts with the 2 wait states
// that an MFMA needs after a VALU write of one of its sources (P and the
// queries' copies are written by VALU just before), and a VALU read of a
// result waits for its write-back (pf_drain); consecutive products into one
// accumulator need no wait.
__device__ __forceinline__ void pf_mfma0(f32x16& acc, const bf16x8& a, const u32x4& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "a"(b));
}
__device__ __forceinline__ void pf_mfma_qa(f32x16& acc, const bf16x8& a, const u32x4& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "a"(b));
}
__device__ __forceinline__ void pf_mfma_vv(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void pf_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// s_waitcnt for the tile ring: `later` (0..K) tiles of L DMA chunks each may
// stay in flight (later is wave-uniform: scalar branches)
template <int L, int K>
__device__ __forceinline__ void vm_wait_tiles(int64_t later) {
  if constexpr (K == 0) {
    vm_wait<0>();
  } else {
    if (later >= K)
      vm_wait<K * L>();
    else
      vm_wait_tiles<L, K - 1>(later);
  }
}

constexpr int XB_ROWS = 128;  // rows per expansion workgroup
constexpr int XB_HEADS = 8;   // heads per head group (a workgroup takes 1, 2 or 4 groups)
constexpr int XB_WAVES = 8;   // expansion waves (two per SIMD)
constexpr int XPF = 4;        // expansion: W operand prefetch depth (k-steps)
constexpr int PF_WAVES = 8;   // attention waves per workgroup (two per SIMD)
constexpr int PF_QBW = 1;     // query blocks of 32 per attention wave
constexpr int PQ = 32 * PF_QBW * PF_WAVES;  // queries per attention workgroup (256)
static_assert(XB_ROWS == XROWS_ALIGN, "expanded rows come in whole expansion blocks");

// ------------------------------------------------------------------------
// Expansion.  A workgroup stages its 128 rows' c in LDS once and expands
// them for a range of 8, 16 or 32 heads.  Eight waves, two per SIMD: wave w
// computes output dims 64 (w & 3) .. +63 of [k^C | v^C] (256 dims) for all
// 128 rows of every other head of the range (parity w >> 2), so one SIMD
// runs two heads' products side by side: A = W rows (U^K or U^V, d_c
// contiguous, from global), B = c^T (rows from LDS), 2 x 4 blocks of 32 x 32
// accumulators.
// ------------------------------------------------------------------------
template <bool PAGED>
__global__ __launch_bounds__(64 * XB_WAVES, 1) void expand_kv_kernel(ExpandArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[XB_ROWS * D_C * 2];  // c rows, 1024 B each
  const int tid = threadIdx.x, l = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int w = wv & 3, hp = wv >> 2;
  const int g = l >> 5, l32 = l & 31;
  const int b = blockIdx.z;
  // Workgroups go to the 8 XCDs round robin by linear index.  The mapping
  // below gives the workgroups that an XCD runs together one head range, so
  // that they share its W^UK and W^UV rows in the XCD's L2 instead of several
  // ranges streaming from the memory-side cache: with the head ranges a
  // multiple of 8, XCD x takes ranges x, x + 8, ... over all row blocks; with
  // 8 / gy XCDs per range (gy ranges), each takes a share of the row blocks.
  const int gx = gridDim.x, gy = gridDim.y;
  const int nhw = a.n_h / gy;  // heads h0 .. h0 + nhw - 1 (8, 16 or 32)
  int rb = blockIdx.x, hg = blockIdx.y;
  if (gy % 8 == 0) {
    const int k = blockIdx.x + gx * blockIdx.y;
    const int x = k % 8, j = k / 8;
    hg = x + 8 * (j / gx);
    rb = j % gx;
  } else if (8 % gy == 0 && gx % (8 / gy) == 0) {
    // 8 / gy XCDs share a head range, each over its own share of the row blocks
    const int k = blockIdx.x + gx * blockIdx.y;
    const int x = k % 8, j = k / 8;
    hg = x % gy;
    rb = (x / gy) * (gx / (8 / gy)) + j;
  }
  const int h0 = hg * nhw;
  const int64_t row0 = static_cast<int64_t>(rb) * XB_ROWS;
  // the prefix clamped to [0, max_len - chunk] exactly as the attention kernel
  // clamps it, so that every row the attention reads is expanded
  int64_t prefix = a.prefix_lens[b];
  prefix = max(min(prefix, static_cast<int64_t>(a.max_len - a.chunk)), static_cast<int64_t>(0));
  int64_t L = prefix + a.chunk;
  L = min(L, a.stride);
  if (row0 >= L) return;  // uniform over the workgroup
  // lo_rows = precise_below + PQ (or INT_MAX when every workgroup is hi + lo).
  // A sequence whose first query already sees precise_below keys has no
  // hi + lo workgroup, so nothing reads its lo parts
  const bool any_precise = a.lo_rows == 0x7fffffff || prefix + 1 + PQ < a.lo_rows;
  const int64_t lo_rows = any_precise ? a.lo_rows : 0;
  const int nrows = static_cast<int>(min(static_cast<int64_t>(XB_ROWS), L - row0));
  auto row_at = [&](int64_t r, bool& ok) {
    return cache_row_addr<PAGED>(a.cache, a.block_table, a.num_pages, a.bt_stride, a.page_shift, a.stride, b, r,
                                 ROWB, ok);
  };

  // ---- c rows -> LDS.  LDS chunk f = 512 i + tid is row 8 i + wv, slot l, and
  // holds the row's global chunk l ^ (row & 15): the swizzle spreads the 16
  // rows that one pass of an operand read touches over distinct banks (with
  // row & 7, rows r and r + 8 met in the same banks).  The block's rows
  // come as four 32-row runs (one page each when paged), each through a buffer
  // resource that spans the run's valid rows, so rows past the sequence (and
  // the rows of a page outside the pool) arrive as zeros.  bad_runs marks the
  // runs of such pages; their expanded rows are written as NaN.
  uint32_t bad_runs = 0;  // uniform
  {
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
                              (__attribute__((address_space(3))) uint8_t*)smem)) +
                          1024u * static_cast<uint32_t>(wv);
#pragma unroll
    for (int k = 0; k < XB_ROWS / 32; ++k) {
      const int rows = max(min(nrows - 32 * k, 32), 0);
      bool ok = true;
      const uint64_t ga = rows > 0 ? row_at(row0 + 32 * k, ok) : reinterpret_cast<uint64_t>(a.cache);
      if (!ok) bad_runs |= 1u << k;
      const i32x4 rs = {__builtin_amdgcn_readfirstlane(static_cast<int>(ga & 0xffffffffu)),
                        __builtin_amdgcn_readfirstlane(static_cast<int>((ga >> 32) & 0xffffu)),
                        __builtin_amdgcn_readfirstlane(ok ? rows * ROWB : 0), 0x00020000};
#pragma unroll
      for (int i = 4 * k; i < 4 * k + 4; ++i) {
        const int r = 8 * i + wv;  // row of the block; 32 k <= r < 32 k + 32
        dma16(lds0 + 8192u * i, (r - 32 * k) * ROWB + 16 * (l ^ (r & 15)), rs, 0);
      }
    }
  }

  // ---- k^R (the last d_hR elements of the cache row) into each head's row
  uint16_t* xb = static_cast<uint16_t*>(a.x) + (static_cast<int64_t>(b) * a.n_h + h0) * a.rows_cap * ROWE;
  for (int idx = tid; idx < XB_ROWS * 8; idx += 64 * XB_WAVES) {
    const int r = idx >> 3, c = idx & 7;
    if (r < nrows) {
      bool ok;
      const uint64_t ga = row_at(row0 + r, ok);
      const u32x4 nan8 = {0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u};
      const u32x4 v = ok ? *reinterpret_cast<const u32x4*>(ga + 2 * D_C + 16 * c) : nan8;
      for (int hh = 0; hh < nhw; ++hh)
        *reinterpret_cast<u32x4*>(xb + (hh * a.rows_cap + row0 + r) * ROWE + D_C + 8 * c) = v;
    }
  }
  vm_wait<0>();
  __syncthreads();

  // B operand: row 32 rb + l32, elements 16 s + 8 g .. +7 (chunk 2 s + g)
  const int cx = l32 & 15;
  auto cread = [&](int rb, int s) -> u32x4 {
    return *reinterpret_cast<const u32x4*>(smem + (32 * rb + l32) * (D_C * 2) + 16 * ((2 * s + g) ^ cx));
  };
  // A operand rows: this wave's dims 64 w + 32 db + l32; U^K for dims < 128, U^V above
  const uint16_t* wsrc = static_cast<const uint16_t*>(w < 2 ? a.w_uk : a.w_uv);
  const int dloc = 64 * (w & 1) + l32;
  // head hh's W rows for this lane (db adds 32 rows)
  auto w_rows = [&](int hh) { return wsrc + (static_cast<int64_t>(h0 + hh) * D_H + dloc) * D_C + 8 * g; };
  // the first XPF k-steps of a head's W operands; the next head's go out
  // before this head's stores, so that their waits do not also wait for the
  // stores (loads and stores share one counter)
  u32x4 wa[XPF][2];
  auto w_first = [&](int hh) {
    const uint16_t* wr = w_rows(hh);
#pragma unroll
    for (int s = 0; s < XPF; ++s)
#pragma unroll
      for (int db = 0; db < 2; ++db) wa[s][db] = *reinterpret_cast<const u32x4*>(wr + 32 * db * D_C + 16 * s);
  };
  w_first(hp);
  for (int hh = hp; hh < nhw; hh += 2) {
    const int h = h0 + hh;
    const uint16_t* wr = w_rows(hh);
    f32x16 acc[2][4];
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][rb][r] = 0.f;
#pragma unroll
    for (int s = 0; s < D_C / 16; ++s) {
      const u32x4 a0 = wa[s % XPF][0], a1 = wa[s % XPF][1];
      if (s + XPF < D_C / 16) {
#pragma unroll
        for (int db = 0; db < 2; ++db)
          wa[s % XPF][db] = *reinterpret_cast<const u32x4*>(wr + 32 * db * D_C + 16 * (s + XPF));
      }
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const bf16x8 bv = __builtin_bit_cast(bf16x8, cread(rb, s));
        acc[0][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a0), bv, acc[0][rb], 0, 0, 0);
        acc[1][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a1), bv, acc[1][rb], 0, 0, 0);
      }
    }
    if (hh + 2 < nhw) w_first(hh + 2);
    // lane l holds dims 8 jq + 4 g + (0..3) of block (db) for row 32 rb + l32.
    // One v_permlane32_swap per pair of values (jq = 2q and 2q + 1) trades the
    // lane pair (l, l + 32)'s halves, after which lane g holds run q: the 8
    // consecutive dims 8 (2q + g) .. +7, stored as 16 B: hi at element d, lo
    // at element 256 + d of the expanded row.  Only the hi + lo attention
    // workgroups read lo, and their keys all lie below lo_rows; past it (and
    // in a sequence without such workgroups) the lo parts are left unwritten.
    uint16_t* xh = static_cast<uint16_t*>(a.x) + (static_cast<int64_t>(b) * a.n_h + h) * a.rows_cap * ROWE;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int r = 32 * rb + l32;
      uint16_t* xr = xh + (row0 + r) * ROWE;
      const bool pz = (bad_runs >> rb) & 1;  // row of a page outside the pool
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const f32x16& v = acc[db][rb];
        float run[2][8];
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[8 * q + e]),
                                                             __float_as_uint(v[8 * q + 4 + e]), false, false);
            run[q][e] = __uint_as_float(sw[0]);
            run[q][4 + e] = __uint_as_float(sw[1]);
          }
        if (r < nrows) {
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int d = 64 * w + 32 * db + 8 * (2 * q + g);
            uint32_t hw[4], lw[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float x0 = pz ? __builtin_nanf("") : run[q][2 * e];
              const float x1 = pz ? __builtin_nanf("") : run[q][2 * e + 1];
              hw[e] = pack_bf16x2(x0, x1);
              lw[e] = pack_bf16x2(x0 - __uint_as_float(hw[e] << 16), x1 - __uint_as_float(hw[e] & 0xffff0000u));
            }
            *reinterpret_cast<uint4*>(xr + d) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
            if (row0 + r < lo_rows)
              *reinterpret_cast<uint4*>(xr + 2 * D_H + d) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------------
// Causal flash attention over the expanded rows.  Wave w owns queries
// q0 + 32 w .. +31 (PF_QBW blocks of 32; the N side of every product):
//   score S^T = K . Q^T: A = tile rows (k^C hi [lo], k^R), B = [q^C; RoPE(q^R)
//   hi [lo]] held in AGPRs;
//   value O^T += V^T . P^T: A = v^C hi [lo] columns by transpose reads, B = P^T
//   hi [lo] straight from the score accumulator (the transpose read fetches
//   exactly the keys whose scores the lane holds).
// The tile stream (32-row tiles, a ring of 4 LDS buffers with 3 in flight,
// one barrier per tile) and the lazy-rescale online softmax are those of the
// decode kernels.  A wave stops computing once its last query's keys end;
// the workgroup streams up to its last query's keys.
// ------------------------------------------------------------------------
template <bool PRECISE>
__global__ __launch_bounds__(64 * PF_WAVES, 1) void prefill_attn_kernel(PrefillArgs a) {
  // ring of NBUF tiles, AHEAD = NBUF - 1 of them requested ahead of the one in
  // use (the hi-only layout's 20 KB tiles would leave room for eight, which
  // measured no faster than four)
  constexpr int NBUF = 4;
  constexpr int AHEAD = NBUF - 1;
  // LDS row: the expanded row as stored (1,152 B) for hi + lo, or its hi
  // parts and k^R alone (k^C hi, v^C hi, k^R: 640 B) for the hi-only instance
  constexpr int RB = PRECISE ? ROWB : 640;
  constexpr int NCH = RB / 16;                    // 16-B chunks per LDS row
  constexpr int TB = TILE * RB;                   // LDS bytes per tile
  constexpr int LOADS = TB / (16 * 256);          // DMA chunks per thread per tile: 9 or 5
  static_assert(TB == LOADS * 16 * 256, "a tile must split evenly over the 256 DMA threads");
  __shared__ __attribute__((aligned(16))) uint8_t smem[NBUF * TB];

  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g32 = l >> 5, l32 = l & 31, j16 = l & 15;
  const int nqb = (a.chunk + PQ - 1) / PQ;
  // Workgroups go to the 8 XCDs round robin by linear index.  With the heads
  // a multiple of 8, all query blocks of head h run on XCD h % 8, so its L2
  // holds the head's expanded rows for all of them.  Within a head the
  // latest (longest) query blocks come first.
  int qi = blockIdx.x, h = blockIdx.y;
  if (gridDim.y % 8 == 0) {
    const int k = blockIdx.x + gridDim.x * blockIdx.y;
    const int x = k % 8, j = k / 8;
    h = x + 8 * (j / gridDim.x);
    qi = j % gridDim.x;
  }
  const int qb = nqb - 1 - qi;
  const int b = blockIdx.z;
  int64_t prefix = a.prefix_lens[b];
  prefix = max(min(prefix, static_cast<int64_t>(a.max_len - a.chunk)), static_cast<int64_t>(0));
  const int prefix32 = static_cast<int>(prefix);
  const int q0 = qb * PQ;
  const int64_t kend = prefix + min(q0 + PQ, a.chunk);  // keys of the workgroup: [0, kend)
  const int64_t ntiles = (kend + TILE - 1) / TILE;
  const int qw = q0 + 32 * PF_QBW * w;                  // this wave's first query
  const int64_t my_tiles = (qw < a.chunk) ? (prefix + min(qw + 32 * PF_QBW, a.chunk) + TILE - 1) / TILE : 0;
  const bool dma_wave = w < 4;                          // waves 0..3 move the tiles
  // both instances are launched over the same grid; each workgroup runs in
  // the one that matches its first query's key count (uniform)
  if ((prefix + q0 + 1 < a.precise_below) != PRECISE) return;

  // ---- tile DMA (as in the decode kernels), into the LDS row layout above
  const uint8_t* xh = static_cast<const uint8_t*>(a.x) + (static_cast<int64_t>(b) * a.n_h + h) * a.rows_cap * ROWB;
  const uint64_t gaddr = reinterpret_cast<uint64_t>(xh);
  const uint32_t lds_w = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
                             (__attribute__((address_space(3))) uint8_t*)smem)) +
                         1024u * static_cast<uint32_t>(w);
  auto tile_rsrc = [&](int64_t it) {
    const uint64_t ga = gaddr + static_cast<uint64_t>(it) * TILE_BYTES;
    const int64_t rows = max(min(static_cast<int64_t>(TILE), kend - it * TILE), static_cast<int64_t>(0));
    const i32x4 rs = {__builtin_amdgcn_readfirstlane(static_cast<int>(ga & 0xffffffffu)),
                      __builtin_amdgcn_readfirstlane(static_cast<int>((ga >> 32) & 0xffffu)),
                      __builtin_amdgcn_readfirstlane(static_cast<int>(rows * ROWB)), 0x00020000};
    return rs;
  };
  // A thread's i-th chunk of a tile: LDS chunk f = tid + 256 i, row t = f / NCH,
  // slot p = f % NCH, holds the row's chunk p ^ swz(t); in the hi-only layout
  // slots 32..39 hold k^R, the expanded row's chunks 64..71 (its lo chunks
  // 32..63 are never fetched).  Both layouts keep a row stride of 32 mod 64
  // dwords, so the swizzle spreads the banks as in the decode kernels.
  auto issue_one = [&](const i32x4& rs, uint32_t dst, int i, uint32_t c) {
    dma16(dst + 4096u * i, static_cast<int>(c << 4), rs, 0);
  };
  auto tile_dst = [&](int64_t it) { return lds_w + static_cast<uint32_t>((it & (NBUF - 1)) * TB); };
  uint32_t ch[LOADS];  // kept in registers (the DMA waves have room for them)
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int f = tid + 256 * i;
    const int t = f / NCH, p = f - NCH * t;
    const int q = p ^ swz(t);
    ch[i] = static_cast<uint32_t>(72 * t + ((!PRECISE && q >= 32) ? q + 32 : q));
  }
  // the first three tiles now, the rest of the ring once the queries are in
  auto issue_tiles = [&](int64_t t0, int64_t t1) {
    if (!dma_wave) return;
    for (int64_t it = t0; it < min(ntiles, t1); ++it) {
      const i32x4 rs = tile_rsrc(it);
#pragma unroll
      for (int i = 0; i < LOADS; ++i) issue_one(rs, tile_dst(it), i, ch[i]);
    }
  };
  issue_tiles(0, 3);

  // ---- score B operands per query block k: q^C (8 k-steps), RoPE(q^R) hi and
  // lo (4 k-steps).  Lanes past the chunk take its last query (never stored).
  u32x4 qc[PF_QBW][8], qrh[PF_QBW][4], qrl[PF_QBW][PRECISE ? 4 : 1];
#pragma unroll
  for (int k = 0; k < PF_QBW; ++k) {
    const int q = min(qw + 32 * k + l32, a.chunk - 1);
    const int64_t nq = (static_cast<int64_t>(b) * a.chunk + q) * a.n_h + h;
    const uint16_t* qcp = static_cast<const uint16_t*>(a.q_c) + nq * D_H + 8 * g32;
#pragma unroll
    for (int s = 0; s < 8; ++s) qc[k][s] = *reinterpret_cast<const u32x4*>(qcp + 16 * s);
    const uint16_t* qrp = static_cast<const uint16_t*>(a.q_r) + nq * D_R + 8 * g32;
    const int64_t pos = prefix + q;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 raw = *reinterpret_cast<const u32x4*>(qrp + 16 * s);
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        // pair 8 s + 4 g32 + pp; both candidates are read uniformly, then selected
        const double th = g32 ? a.rope.theta[8 * s + 4 + pp] : a.rope.theta[8 * s + pp];
        float y0, y1;
        rope_pair(__uint_as_float(raw[pp] << 16), __uint_as_float(raw[pp] & 0xffff0000u), pos, th, y0, y1);
        const uint32_t hi = pack_bf16x2(y0, y1);
        qrh[k][s][pp] = hi;
        if constexpr (PRECISE)
          qrl[k][s][pp] = pack_bf16x2(y0 - __uint_as_float(hi << 16), y1 - __uint_as_float(hi & 0xffff0000u));
      }
      // one AGPR tuple each from here on (built a lane pair at a time, they
      // were otherwise regathered before every product)
      asm volatile("" : "+a"(qrh[k][s]));
      if constexpr (PRECISE) asm volatile("" : "+a"(qrl[k][s]));
    }
  }
  vm_wait<0>();  // queries and the first tiles resident: the loop carries no compiler waits
  issue_tiles(3, AHEAD);

  // ---- per-lane LDS operand offsets (as in the 32-head decode kernel)
  int sc_off[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) sc_off[m] = l32 * RB + 16 * ((2 * m + g32) ^ swz(l32));
  int tr_off[2][2];
  {
    const int hf = (l >> 4) & 1;
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int t = 4 * g32 + (j16 >> 2) + 8 * r, e = 32 * p + 16 * hf + 4 * (j16 & 3);
        tr_off[r][p] = t * RB + 16 * ((e >> 3) ^ swz(t)) + 2 * (e & 7);  // element e of LDS row t
      }
  }

  f32x16 oacc[PF_QBW][4];  // O^T of query block k, dims 32 db .. +31
#pragma unroll
  for (int k = 0; k < PF_QBW; ++k)
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[k][db][r] = 0.f;
  float m_run[PF_QBW], l_run[PF_QBW];
#pragma unroll
  for (int k = 0; k < PF_QBW; ++k) {
    m_run[k] = NEG_INF;
    l_run[k] = 0.f;
  }
  const float qscale = a.qscale;

  // One tile for this wave's two query blocks; PRECISE adds the lo products.
  // dma: this wave moves tile it+AHEAD (its LOADS chunks go out one after each
  // of the first score products)
  auto tile = [&](const uint8_t* buf, int64_t it, bool dma) {
    // k-step s reads elements 16 s .. +15 (128-B group s >> 2 of the stored
    // row); in the hi-only layout k^R's groups 8, 9 sit at 4, 5
    auto kread = [&](int s) -> bf16x8 {
      const int grp = (!PRECISE && s >= 32) ? (s >> 2) - 4 : (s >> 2);
      return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(buf + sc_off[s & 3] + 128 * grp));
    };
    // value A: 32 columns of the expanded row from column block cbg, keys of half u
    auto vread = [&](int cbg, int u) -> bf16x8 {
      const uint8_t* bu = buf + 128 * (cbg >> 1) + 16 * u * RB;
      return cat(tr_read(bu + tr_off[0][cbg & 1]), tr_read(bu + tr_off[1][cbg & 1]));
    };
    // ---- score: elements 0..127 (k^C hi: k-steps 0..7), 256..383 (k^C lo:
    // 16..23), 512..575 (k^R: 32..35).  The operands are read KPF k-steps
    // ahead of their products (the order: k^C hi, with each k^C lo right
    // after its hi part, then k^R).
    constexpr int NK = PRECISE ? 20 : 12;
    constexpr int KPF = 4;
    auto kstep = [](int i) {
      if (PRECISE) return i < 16 ? ((i & 1) ? 16 + (i >> 1) : (i >> 1)) : 32 + (i - 16);
      return i < 8 ? i : 32 + (i - 8);
    };
    f32x16 sacc[PF_QBW];
    i32x4 rs3 = {0, 0, 0, 0};
    if (dma) rs3 = tile_rsrc(it + AHEAD);
    {
      bf16x8 kb[KPF];
#pragma unroll
      for (int i = 0; i < KPF; ++i) kb[i] = kread(kstep(i));
#pragma unroll
      for (int i = 0; i < NK; ++i) {
        const bf16x8 kv = kb[i % KPF];
        if (i + KPF < NK) kb[i % KPF] = kread(kstep(i + KPF));
        const int ks = kstep(i);
#pragma unroll
        for (int k = 0; k < PF_QBW; ++k) {
          if (ks == 0)
            pf_mfma0(sacc[k], kv, qc[k][0]);
          else if (ks < 8)
            pf_mfma_qa(sacc[k], kv, qc[k][ks]);
          else if (ks < 32)
            pf_mfma_qa(sacc[k], kv, qc[k][ks - 16]);  // k^C lo against the same query part
          else {
            pf_mfma_qa(sacc[k], kv, qrh[k][ks - 32]);
            if constexpr (PRECISE) pf_mfma_qa(sacc[k], kv, qrl[k][ks - 32]);
          }
        }
        if (dma && i < LOADS) issue_one(rs3, tile_dst(it + AHEAD), i, ch[i]);
      }
    }
    // the value operands (v^C hi) do not depend on P: their transpose reads
    // are issued now and land while the softmax runs
    constexpr int NVA = PRECISE ? 1 : 8;
    bf16x8 va[NVA];
    if constexpr (!PRECISE) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int u = 0; u < 2; ++u) va[2 * db + u] = vread(4 + db, u);
    }
    pf_drain();
    // ---- causal mask, online softmax (log2, lazy rescale) and P^T
    bf16x8 ph[PF_QBW][2], pl[PF_QBW][PRECISE ? 2 : 1];
#pragma unroll
    for (int k = 0; k < PF_QBW; ++k) {
      f32x16& x = sacc[k];
      // positions fit in 32 bits (prefix + chunk <= max_len < 2^31)
      const int pos = prefix32 + min(qw + 32 * k + l32, a.chunk - 1);
      const int key0 = TILE * static_cast<int>(it);
      if (key0 + TILE - 1 > prefix32 + qw + 32 * k) {  // the tile reaches past the block's first query
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (key0 + 8 * (j >> 2) + 4 * g32 + (j & 3) > pos) x[j] = NEG_INF;
      }
      float mx = x[0];
#pragma unroll
      for (int j = 1; j < 16; ++j) mx = fmaxf(mx, x[j]);
      mx = pair_max32(mx);
      const float mt = mx * qscale;  // scale > 0 commutes with max
      const bool need = mt > m_run[k] + RESCALE_TAU;
      if (__ballot(need)) {
        const float m_new = need ? mt : m_run[k];
        const float alpha = __builtin_amdgcn_exp2f(m_run[k] - m_new);  // 0 when m_run = -inf
        l_run[k] *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db) oacc[k][db] *= alpha;
        m_run[k] = m_new;
      }
      const float neg_m = -m_run[k];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(x[8 * u + i], qscale, neg_m));
          l_run[k] += pv;
          ph[k][u][i] = static_cast<__bf16>(pv);
          if constexpr (PRECISE) pl[k][u][i] = static_cast<__bf16>(pv - static_cast<float>(ph[k][u][i]));
        }
    }
    // ---- value: v^C hi at elements 128..255 (column blocks 4..7), lo at
    // 384..511 (12..15)
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bf16x8 vh = PRECISE ? vread(4 + db, u) : va[(2 * db + u) % NVA];
#pragma unroll
        for (int k = 0; k < PF_QBW; ++k) {
          pf_mfma_vv(oacc[k][db], vh, ph[k][u]);
          if constexpr (PRECISE) pf_mfma_vv(oacc[k][db], vh, pl[k][u]);
        }
        if constexpr (PRECISE) {
          const bf16x8 vl = vread(12 + db, u);
#pragma unroll
          for (int k = 0; k < PF_QBW; ++k) pf_mfma_vv(oacc[k][db], vl, ph[k][u]);
        }
      }
  };

  for (int64_t it = 0; it < ntiles; ++it) {
    // tile `it` must have landed: the loads of the (up to AHEAD - 1) later
    // tiles may stay in flight
    vm_wait_tiles<LOADS, AHEAD - 1>(min(static_cast<int64_t>(AHEAD - 1), ntiles - 1 - it));
    __syncthreads();
    // every wave passed this barrier, so buffer (it+AHEAD) % NBUF == (it-1) % NBUF is free:
    // its refill goes out between this tile's score products (or at once
    // from a wave whose queries have no keys left)
    const bool dma = dma_wave && it + AHEAD < ntiles;
    const uint8_t* buf = smem + (it & (NBUF - 1)) * TB;
    if (it < my_tiles) {
      tile(buf, it, dma);
    } else if (dma) {
      const i32x4 rs = tile_rsrc(it + AHEAD);
#pragma unroll
      for (int i = 0; i < LOADS; ++i) issue_one(rs, tile_dst(it + AHEAD), i, ch[i]);
    }
  }

  pf_drain();  // the last output products have landed

  // ---- normalise and store: lane l holds dims 32 db + 8 jq + 4 g32 + (0..3)
  // of query qw + 32 k + l32
  if (qw < a.chunk) {
#pragma unroll
    for (int k = 0; k < PF_QBW; ++k) {
      const int q = qw + 32 * k + l32;
      const float lt = pair_sum32(l_run[k]);
      const float inv = (lt > 0.f) ? 1.f / lt : 0.f;
      if (q < a.chunk) {
        float* orow = a.out + ((static_cast<int64_t>(b) * a.chunk + q) * a.n_h + h) * D_H + 4 * g32;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int jq = 0; jq < 4; ++jq) {
            const f32x16& o = oacc[k][db];
            const f32x4 v = {o[4 * jq] * inv, o[4 * jq + 1] * inv, o[4 * jq + 2] * inv, o[4 * jq + 3] * inv};
            *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * jq) = v;
          }
      }
    }
  }
}

hipError_t launch_prefill_unabsorbed(const ExpandArgs& e_in, const PrefillArgs& p, hipStream_t st) {
  if (p.chunk <= 0 || p.batch <= 0) return hipSuccess;
  ExpandArgs e = e_in;
  // a hi + lo workgroup's first query sees < precise_below keys, so all its
  // keys lie below precise_below + PQ - 1 (every row when all workgroups are)
  const int64_t lo_rows = static_cast<int64_t>(p.precise_below) + PQ;
  e.lo_rows = static_cast<int32_t>(lo_rows < 0x7fffffff ? lo_rows : 0x7fffffff);
  // up to 4 head groups per workgroup (c rows loaded once for all of them)
  // while the grid still fills one round of the compute units
  const int nhg = e.n_h / XB_HEADS;
  const int64_t nrb = e.rows_cap / XB_ROWS;
  int hpw = 1;
  for (int c = 4; c >= 2; c /= 2)
    if (nhg % c == 0 && nrb * (nhg / c) * e.batch >= 256) { hpw = c; break; }
  const dim3 g1(static_cast<unsigned>(nrb), nhg / hpw, e.batch);
  if (e.block_table)
    expand_kv_kernel<true><<<g1, 64 * XB_WAVES, 0, st>>>(e);
  else
    expand_kv_kernel<false><<<g1, 64 * XB_WAVES, 0, st>>>(e);
  const hipError_t r = hipGetLastError();
  if (r != hipSuccess) return r;
  const dim3 g2((p.chunk + PQ - 1) / PQ, p.n_h, p.batch);
  prefill_attn_kernel<true><<<g2, 64 * PF_WAVES, 0, st>>>(p);
  const hipError_t r2 = hipGetLastError();
  if (r2 != hipSuccess) return r2;
  prefill_attn_kernel<false><<<g2, 64 * PF_WAVES, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace mla
