// A3 -- split-KV latent attention for gfx950 (MI355X).
//
// For one query token and all its heads, over the rows j of one split:
//   l_ij = (q~_i . c_j + q^R_i . k^R_j) * scale        (jiphyeonjeon.kr DeepSeek-V2
//                                                       review, section 3)
//   lse_i = log sum_j exp(l_ij),  Z_i = sum_j exp(l_ij - lse_i) c_j
// i.e. softmax_j restricted to the split; the combine (A4) re-associates the
// splits exactly.  Every head reads the same cache row (review section 2: the
// latent is shared, but a_ij differs per head), so one LDS tile of rows feeds
// all heads of the query and both contractions are dense:
//   S^T[t][i] = sum_e row[t][e] q_lat[i][e]    (e over d_c + d_hR = 576)
//   Z^T[c][i] += sum_t row[t][c] P^T[t][i]    (t over the tile's rows)
//
// MFMA fast paths (bf16, d_c=512, d_hR=64, n_h in {16,32,64,128}): n_h = 128
// and n_h = 16 have kernels of their own below; n_h = 32 and 64 run
// splitkv_mfma_kernel:
//   * 4 waves; a wave owns 32 heads and a slice of the 512 latent columns
//     (n_h = 32: 1 head group x 4 column quarters; 64: 2 x 2).
//   * Tiles of 32 rows (36,864 B) stream into a ring of 4 LDS buffers by
//     buffer_load ... lds (global -> LDS DMA, no staging registers), three tiles
//     in flight while one is computed.  Rows keep their natural 1152-B stride;
//     16-B chunks are XOR-swizzled by row (by choosing each lane's source
//     chunk) so the score reads and the transpose reads are conflict free.
//     The buffer resource spans exactly the split's rows, so rows past the
//     split end arrive as zeros: no masking code on the load side.
//   * Score: A = tile rows (ds_read_b128, e contiguous), B = the wave's
//     absorbed queries, held in VGPRs for the whole split.
//   * Value: A = tile columns via ds_read_b64_tr_b16 (the LDS transpose read
//     turns 4 rows x 16 columns into per-lane columns), B = P^T taken straight
//     from the score accumulators: each transpose read fetches exactly the
//     rows whose scores the lane holds, so no shuffle is needed.
//   * Online softmax in the log2 domain with a lazy rescale: the reference max
//     only moves when a tile max exceeds it by more than 8 (so p <= 2^8), and
//     the Z accumulators are rescaled only then.  Exact up to rounding.
#include "mla_common.h"
#include "mla_tile.h"

namespace mla {

#ifdef MLA_PHASE_STAMPS
// Measurement build only (build.py --probe): per-wave cycle sums of the
// 128-head kernel's tile loop, by phase, for the first 1,024 workgroups.
__device__ uint64_t g_phase_stamps[1024 * 4 * 8];
#endif

constexpr int NQ16 = (D_C + D_R) / 32;  // 16-head score k-steps of 32 elements

template <bool PAGED>
__device__ __forceinline__ uint64_t row_addr(const SplitArgs& a, int b, int64_t r, int64_t row_bytes, bool& ok) {
  return cache_row_addr<PAGED>(a.cache, a.block_table, a.num_pages, a.bt_stride, a.page_shift, a.stride, b, r,
                               row_bytes, ok);
}

// A split whose rows include one of a bad page reports lse = +inf and z = NaN:
// the combine then turns every output of the query into NaN.
constexpr float POS_INF = __builtin_huge_valf();

// ------------------------------------------------------------------------
// n_h = 16 (the V2-Lite shape), and the precise path of every head count.
// Per cache row the matrix work of 16 heads is an eighth of the 128-head
// case, so this body is a stream of the cache: what counts is bytes in
// flight and little LDS traffic.  Each wave owns every fourth 16-row tile of
// the split (tiles w, w+4, ...) with its own online softmax and its own Z for
// the group's 16 heads x 512 columns (128 accumulators), and two LDS buffers
// that its own DMAs fill (one tile scored while the next lands), so the loop
// has no workgroup barrier.  The four waves' (m, l, Z) merge through LDS at
// the end.
//   score: v_mfma_f32_16x16x32_bf16, A = tile rows, B = absorbed queries (hi,
//          then lo: the two products sum to the fp32 query to ~2^-16);
//   value: v_mfma_f32_16x16x32_bf16, A = tile columns by transpose reads
//          (each read twice along K), B = P^T straight from the score
//          accumulator (lane l holds rows 4(l/16)+i of head l%16 in both),
//          hi in the first half of K and lo in the second.
// Neither product rounds an operand that the result depends on beyond the
// stored values, so this body matches the exact softmax to ~1e-5 of the
// output rms at any length.  The wider kernels score with the bf16 query
// alone and pack the weights once to bf16 (a relative 2^-9 on each score and
// weight); over few rows, and under the long-context temperature, that shows
// at the 1e-2 level of max|err|/rms, so queries that attend fewer than
// `precise_below` rows run this body one 16-head group at a time instead.
// ------------------------------------------------------------------------
constexpr int T16 = 16;                          // rows per tile
constexpr int T16_BYTES = T16 * ROWB;            // 18,432 B
constexpr int T16_LOADS = T16_BYTES / (16 * 64);  // 18 DMA chunks per lane per tile
constexpr int ZPAD = D_C * 4 + 16;               // merge: bytes per staged head row

// Heads h0..h0+15 of query n over split `split` (sequence b, attended length
// len): the 16-head kernel's body, also the precise path of the wider kernels
// (every query row scored with hi + lo, every softmax weight carried as hi +
// lo).  smem: at least 8 * T16_BYTES of LDS; the caller separates two calls
// with a barrier.
template <bool PAGED>
__device__ __forceinline__ void h16_group(const SplitArgs& a, uint8_t* smem, int n, int split, int h0, int b,
                                          int64_t len) {
  static_assert(4 * 16 * ZPAD + 2 * 4 * 16 * 4 <= 8 * T16_BYTES, "merge staging must fit the buffers");
  static_assert(T16_BYTES == T16_LOADS * 16 * 64, "tile must split evenly over 64 lanes");

  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: DMA addresses go to SGPRs
  const int q4 = l >> 4, j16 = l & 15;
  const int64_t lo = static_cast<int64_t>(split) * a.split_rows;
  const int64_t hi = min(lo + a.split_rows, len);
  float* zo = a.z_part + ((static_cast<int64_t>(n) * a.num_splits + split) * a.n_h + h0) * D_C;
  float* lse_o = a.lse_part + (static_cast<int64_t>(n) * a.num_splits + split) * a.n_h + h0;

  if (lo >= hi) {  // empty split (uniform over the workgroup)
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    for (int idx = tid; idx < 16 * D_C / 4; idx += 256) reinterpret_cast<f32x4*>(zo)[idx] = zero;
    if (tid < 16) lse_o[tid] = NEG_INF;
    return;
  }
  const int64_t ntiles = (hi - lo + T16 - 1) / T16;
  const int my_tiles = static_cast<int>((ntiles > w) ? (ntiles - w + 3) / 4 : 0);  // wave-uniform

  // ---- absorbed queries (B operands): head h0 + j16, elements 32 s + 8 q4 .. +7
  // of the hi plane and of the lo plane (zeros without one)
  u32x4 qh[NQ16], ql[NQ16];
  {
    const int64_t qo = (static_cast<int64_t>(n) * a.n_h + h0 + j16) * ROWE + 8 * q4;
    const uint16_t* q = static_cast<const uint16_t*>(a.q_lat) + qo;
#pragma unroll
    for (int s = 0; s < NQ16; ++s) qh[s] = *reinterpret_cast<const u32x4*>(q + 32 * s);
    if (a.q_lat_lo) {
      const uint16_t* ql_src = static_cast<const uint16_t*>(a.q_lat_lo) + qo;
#pragma unroll
      for (int s = 0; s < NQ16; ++s) ql[s] = *reinterpret_cast<const u32x4*>(ql_src + 32 * s);
    } else {
#pragma unroll
      for (int s = 0; s < NQ16; ++s) ql[s] = u32x4{0u, 0u, 0u, 0u};
    }
  }

  // ---- this wave's tile DMAs: its k-th tile (split tile w + 4k) goes to
  // buffer 2w + (k & 1).  LDS chunk f = 64 i + l of a buffer receives global
  // chunk (t, p ^ swz(t)) with (t, p) = (f / 72, f % 72).  The buffer resource
  // spans the tile's rows inside the split, so rows past its end arrive as zeros.
  const uint8_t* gsplit =
      static_cast<const uint8_t*>(a.cache) + (static_cast<int64_t>(b) * a.stride + lo) * ROWB;
  const uint64_t gaddr = reinterpret_cast<uint64_t>(gsplit);
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) uint8_t*)smem));
  bool bad = false;  // one of this wave's tiles sits in a page outside the pool (wave-uniform)
  auto issue = [&](int k) {
    const int64_t it = w + 4 * static_cast<int64_t>(k);
    uint64_t ga = gaddr + static_cast<uint64_t>(it) * T16_BYTES;
    int64_t rows = min(static_cast<int64_t>(T16), hi - lo - it * T16);
    if constexpr (PAGED) {
      bool ok = true;
      if (rows > 0) ga = row_addr<true>(a, b, lo + it * T16, ROWB, ok);
      if (!ok) {
        rows = 0;
        bad = true;
      }
    }
    const i32x4 rs = {__builtin_amdgcn_readfirstlane(static_cast<int>(ga & 0xffffffffu)),
                      __builtin_amdgcn_readfirstlane(static_cast<int>((ga >> 32) & 0xffffu)),
                      __builtin_amdgcn_readfirstlane(static_cast<int>(rows * ROWB)), 0x00020000};
    const uint32_t dst = lds0 + static_cast<uint32_t>((2 * w + (k & 1)) * T16_BYTES);
    // the lane index passes through an empty asm so that the 18 source offsets
    // are formed here, not hoisted out of the loop into 18 live registers
    int lx = l;
    asm volatile("" : "+v"(lx));
#pragma unroll
    for (int i = 0; i < T16_LOADS; ++i) {
      const int f = 64 * i + lx;
      const int t = f / 72, p = f - 72 * t;
      dma16(dst + 1024u * i, 16 * (72 * t + (p ^ swz(t))), rs, 0);
    }
  };
  if (my_tiles > 0) issue(0);
  if (my_tiles > 1) issue(1);
  // queries and the first two tiles resident: after this the compiler has no
  // load of its own in flight, so the loop carries no waits but the explicit ones
  vm_wait<0>();

  // ---- per-lane LDS operand offsets
  // score A: row j16, elements 32 s + 8 q4 .. +7 -> chunk 4 s + q4
  int sc_off[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) sc_off[m] = j16 * ROWB + 16 * ((4 * m + q4) ^ swz(j16));
  // value A (transpose reads): rows 4 q4 + (j16 >> 2), columns 16 cb + 4 (j16 & 3)
  int tr_off[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) tr_off[p] = tile_off(4 * q4 + (j16 >> 2), 16 * p + 4 * (j16 & 3));

  f32x4 zacc[32];  // Z^T of c-block cb: columns 16 cb + 4 q4 + i of head j16
#pragma unroll
  for (int c = 0; c < 32; ++c) zacc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = NEG_INF, l_run = 0.f;
  const float qscale = a.qscale;

  for (int k = 0; k < my_tiles; ++k) {
    // this tile has landed (the next one's loads may stay in flight)
    if (k + 1 < my_tiles)
      vm_wait<T16_LOADS>();
    else
      vm_wait<0>();
    const uint8_t* buf = smem + (2 * w + (k & 1)) * T16_BYTES;
    const int64_t it = w + 4 * static_cast<int64_t>(k);
    const int valid = static_cast<int>(min(hi - lo - it * T16, static_cast<int64_t>(T16)));

    // -------------------------------------------------- score S^T = rows . q
    constexpr int PF = 4;
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
    {
      u32x4 kb[PF];
#pragma unroll
      for (int s = 0; s < PF; ++s) kb[s] = *reinterpret_cast<const u32x4*>(buf + sc_off[s & 1] + 128 * (s >> 1));
#pragma unroll
      for (int s = 0; s < NQ16; ++s) {
        const u32x4 kv = kb[s % PF];
        if (s + PF < NQ16)
          kb[s % PF] = *reinterpret_cast<const u32x4*>(buf + sc_off[(s + PF) & 1] + 128 * ((s + PF) >> 1));
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kv),
                                                       __builtin_bit_cast(bf16x8, qh[s]), sacc, 0, 0, 0);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kv),
                                                       __builtin_bit_cast(bf16x8, ql[s]), sacc, 0, 0, 0);
      }
    }
    // first value operands: independent of P, so their latency overlaps the softmax
    constexpr int VPF = 4;
    i16x4 vb[VPF];
#pragma unroll
    for (int c = 0; c < VPF; ++c) vb[c] = tr_read(buf + 128 * (c >> 2) + tr_off[c & 3]);

    // -------------------------------------------------- online softmax (log2)
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = (4 * q4 + i < valid) ? sacc[i] : NEG_INF;
    float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mx = pair_max32(mx);
    mx = pair_max16(mx);
    const float mt = mx * qscale;  // scale > 0 commutes with max
    const bool need = mt > m_run + RESCALE_TAU;
    if (__ballot(need)) {
      const float m_new = need ? mt : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 when m_run = -inf
      l_run *= alpha;
#pragma unroll
      for (int c = 0; c < 32; ++c) zacc[c] *= alpha;
      m_run = m_new;
    }
    const float neg_m = -m_run;
    i16x4 ph, pl;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pv = __builtin_amdgcn_exp2f(fmaf(x[i], qscale, neg_m));
      l_run += pv;
      const uint16_t h16 = f32_to_bf16(pv);
      ph[i] = static_cast<short>(h16);
      pl[i] = static_cast<short>(f32_to_bf16(pv - bf16_to_f32(h16)));
    }
    // one K = 32 product covers both parts: k < 4 pairs the tile rows with
    // P hi, k >= 4 pairs the same rows with P lo
    const bf16x8 pp = cat(ph, pl);

    // -------------------------------------------------- value Z^T += rows^T . P^T
#pragma unroll
    for (int c = 0; c < 32; ++c) {
      const i16x4 va = vb[c % VPF];
      if (c + VPF < 32) vb[c % VPF] = tr_read(buf + 128 * ((c + VPF) >> 2) + tr_off[(c + VPF) & 3]);
      zacc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cat(va, va), pp, zacc[c], 0, 0, 0);
    }

    // the buffer is free once this wave's reads of it returned: refill it
    if (k + 2 < my_tiles) {
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt at their maxima
      issue(k + 2);
    }
  }

  // ---- merge the four waves: M = max m_w, L = sum_w 2^(m_w - M) l_w,
  // z = sum_w 2^(m_w - M) Z_w / L.  A wave without tiles has m = -inf, l = 0.
  float lt = pair_sum32(l_run);
  lt = pair_sum16(lt);
  if (PAGED && bad) lt = __builtin_nanf("");  // carried into L by the merge
  __syncthreads();  // every wave is done with its buffers
  float* mst = reinterpret_cast<float*>(smem + 4 * 16 * ZPAD);
  float* lst = mst + 64;
  if (q4 == 0) {
    mst[16 * w + j16] = m_run;
    lst[16 * w + j16] = lt;
  }
  __syncthreads();
  float M = NEG_INF;
#pragma unroll
  for (int v = 0; v < 4; ++v) M = fmaxf(M, mst[16 * v + j16]);
  float L = 0.f;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const float mv = mst[16 * v + j16];
    if (mv != NEG_INF) L += lst[16 * v + j16] * __builtin_amdgcn_exp2f(mv - M);
  }
  float f = (m_run != NEG_INF && L > 0.f) ? __builtin_amdgcn_exp2f(m_run - M) / L : 0.f;
  float lse = (L > 0.f) ? (M + log2f(L)) * LN2 : NEG_INF;
  if (PAGED && L != L) {
    f = __builtin_nanf("");
    lse = POS_INF;
  }
  {
    uint8_t* row = smem + w * 16 * ZPAD + j16 * ZPAD + 16 * q4;
#pragma unroll
    for (int c = 0; c < 32; ++c) {
      const f32x4 v = {zacc[c][0] * f, zacc[c][1] * f, zacc[c][2] * f, zacc[c][3] * f};
      *reinterpret_cast<f32x4*>(row + 64 * c) = v;
    }
  }
  if (w == 0 && q4 == 0) lse_o[j16] = lse;
  __syncthreads();
  for (int idx = tid; idx < 16 * (D_C / 4); idx += 256) {
    const int h = idx >> 7, c4 = idx & 127;
    f32x4 acc = *reinterpret_cast<const f32x4*>(smem + h * ZPAD + 16 * c4);
#pragma unroll
    for (int v = 1; v < 4; ++v) acc += *reinterpret_cast<const f32x4*>(smem + v * 16 * ZPAD + h * ZPAD + 16 * c4);
    *reinterpret_cast<f32x4*>(zo + h * D_C + 4 * c4) = acc;
  }
}

template <int CG, bool PAGED>
__global__ __launch_bounds__(256, 1) void splitkv_mfma_kernel(
    SplitArgs a) {
  constexpr int HPW = 32;                        // heads per wave
  constexpr int NHG = 4 / CG;                    // head groups per workgroup
  constexpr int COLS = D_C / CG;                 // latent columns per wave
  constexpr int CB = COLS / HPW;                 // value c-blocks per wave
  constexpr int NQ = 36;                         // score k-steps (576 / 16)
  constexpr int NSC = 16;                        // scores held per lane per tile
  constexpr int LOADS = TILE_BYTES / (16 * 256);  // 9 chunk loads per thread per tile
  constexpr int PF = 4;                          // LDS operand prefetch depth (MFMA steps)
  static_assert(TILE_BYTES == LOADS * 16 * 256, "tile must split evenly over 256 threads");

  __shared__ __attribute__((aligned(16))) uint8_t smem[4 * TILE_BYTES + 9 * 256 * 4];  // tile ring + DMA offset table
  static_assert(4 * TILE_BYTES + 9 * 256 * 4 >= 8 * T16_BYTES, "the precise path's buffers must fit");

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int hg = w % NHG, cg = w / NHG;
  const int n = blockIdx.x, split = blockIdx.y;
  int b;
  int64_t len;
  query_range(a, n, b, len);
  const int64_t lo = static_cast<int64_t>(split) * a.split_rows;
  const int64_t hi = min(lo + a.split_rows, len);
  const int h0 = hg * HPW;
  float* zo = a.z_part + (static_cast<int64_t>(n) * a.num_splits + split) * a.n_h * D_C;
  float* lse_o = a.lse_part + (static_cast<int64_t>(n) * a.num_splits + split) * a.n_h;

  if (lo >= hi) {  // empty split (uniform over the workgroup)
    for (int idx = l; idx < HPW * COLS; idx += 64) {
      const int hh = idx / COLS, c = cg * COLS + idx % COLS;
      zo[static_cast<int64_t>(h0 + hh) * D_C + c] = 0.f;
    }
    if (cg == 0 && l < HPW) lse_o[h0 + l] = NEG_INF;
    return;
  }
  if (len < a.precise_below) {  // few rows: 16-head groups with hi + lo products (uniform)
    for (int g = 0; g < NHG * HPW / 16; ++g) {
      if (g) __syncthreads();
      h16_group<PAGED>(a, smem, n, split, 16 * g, b, len);
    }
    return;
  }

  const int g32 = l >> 5, j16 = l & 15;

  // ---- tile loads: LDS chunk f = tid + 256 i of the tile receives global
  // chunk (t, p ^ swz(t)) with (t, p) = (f / 72, f % 72).  Nothing the loop
  // reads may be spilled: a spilled value comes back through a VMEM reload that
  // the compiler would then fence every (asm) DMA on.
  constexpr int NBUF = 4;
  const uint8_t* gsplit =
      static_cast<const uint8_t*>(a.cache) + (static_cast<int64_t>(b) * a.stride + lo) * ROWB;
  // One buffer resource per tile, based at the tile's first row and sized to
  // the tile's rows inside the split: the range check (voffset only) returns
  // zeros for rows past the split end, so nothing past it is ever read.
  const uint64_t gaddr = reinterpret_cast<uint64_t>(gsplit);
  const int64_t ntiles = (hi - lo + TILE - 1) / TILE;
  const uint32_t lds_w = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
                             (__attribute__((address_space(3))) uint8_t*)smem)) +
                         1024u * static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(w));
  // source byte offset (inside the tile) of the chunk that lands in LDS slot tid + 256 i
  auto chunk_off = [&](int i, int z) {
    const int f = tid + 256 * i + z;
    const int t = f / 72, p = f - 72 * t;
    return 16 * (f - p + (p ^ swz(t)));
  };
  bool bad = false;  // a tile of this split sits in a page outside the pool (uniform)
  auto tile_rsrc = [&](int64_t it) {
    uint64_t ga = gaddr + static_cast<uint64_t>(it) * TILE_BYTES;
    int64_t rows = min(static_cast<int64_t>(TILE), hi - lo - it * TILE);
    if constexpr (PAGED) {
      bool ok = true;
      if (rows > 0) ga = row_addr<true>(a, b, lo + it * TILE, ROWB, ok);
      if (!ok) {
        rows = 0;
        bad = true;
      }
    }
    const i32x4 rs = {__builtin_amdgcn_readfirstlane(static_cast<int>(ga & 0xffffffffu)),
                      __builtin_amdgcn_readfirstlane(static_cast<int>((ga >> 32) & 0xffffu)),
                      __builtin_amdgcn_readfirstlane(static_cast<int>(rows * ROWB)), 0x00020000};
    return rs;
  };
  // prologue issues: offsets recomputed (registers are scarce while the queries load)
  auto issue_direct = [&](int64_t it) {
    const i32x4 rs = tile_rsrc(it);
    const uint32_t dst = lds_w + static_cast<uint32_t>((it & (NBUF - 1)) * TILE_BYTES);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) dma16(dst + 4096u * i, chunk_off(i, 0), rs, 0);
  };

  // the first tiles stream in while the queries load
  issue_direct(0);
  if (ntiles > 1) issue_direct(1);
  if (ntiles > 2) issue_direct(2);

  // ---- absorbed queries -> B-operand registers: the hi plane (the register
  // file has no room for lo at 32 heads per wave)
  u32x4 qreg[NQ];
  {
    const uint16_t* q = static_cast<const uint16_t*>(a.q_lat) + static_cast<int64_t>(n) * a.n_h * ROWE;
    const uint16_t* qh = q + (h0 + (l & 31)) * ROWE + 8 * g32;
#pragma unroll
    for (int s = 0; s < NQ; ++s) qreg[s] = *reinterpret_cast<const u32x4*>(qh + 16 * s);
  }
  vm_wait<0>();  // queries and the first tiles resident: the loop itself carries no compiler waits

  // loop issues: each thread's 9 source offsets live in a small LDS table (the
  // loop's register budget has no room for them, and a spilled copy would come
  // back through VMEM reloads)
  int* voff_tab = reinterpret_cast<int*>(smem + NBUF * TILE_BYTES);
#pragma unroll
  for (int i = 0; i < LOADS; ++i) voff_tab[i * 256 + tid] = chunk_off(i, 0);
  auto issue = [&](int64_t it) {
    const i32x4 rs = tile_rsrc(it);
    const uint32_t dst = lds_w + static_cast<uint32_t>((it & (NBUF - 1)) * TILE_BYTES);
    int vo[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) vo[i] = voff_tab[i * 256 + tid];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) dma16(dst + 4096u * i, vo[i], rs, 0);
  };

  // ---- per-lane LDS offsets of the MFMA operands
  // score A: row t = l%32, element 16 s + 8 g  -> chunk 2 s + g
  int sc_off[4];
  {
    const int t = l & 31;
#pragma unroll
    for (int m = 0; m < 4; ++m) sc_off[m] = t * ROWB + 16 * ((2 * m + g32) ^ swz(t));
  }
  // value A: rows 16u + 4g + (j16>>2) and +8, columns 32 cb + 16 hf + 4 (j16&3)
  int tr_off[2][2];  // [first/second transpose read][odd/even 32-column block]
  {
    const int hf = (l >> 4) & 1;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int tt = 4 * g32 + (j16 >> 2) + 8 * r;
#pragma unroll
      for (int p = 0; p < 2; ++p) tr_off[r][p] = tile_off(tt, 32 * p + 16 * hf + 4 * (j16 & 3));
    }
  }

  f32x16 zacc[CB];
#pragma unroll
  for (int c = 0; c < CB; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) zacc[c][r] = 0.f;
  float m_run = NEG_INF, l_run = 0.f;

  for (int64_t it = 0; it < ntiles; ++it) {
    // tile `it` must have landed: the loads of the (up to 2) later tiles may stay in flight
    if (it + 2 < ntiles)
      vm_wait<2 * LOADS>();
    else if (it + 1 < ntiles)
      vm_wait<LOADS>();
    else
      vm_wait<0>();
    __syncthreads();
    const uint8_t* buf = smem + (it & (NBUF - 1)) * TILE_BYTES;
    // rows of this tile inside the split (1..32); only a partial tile needs masking
    const int valid = static_cast<int>(min(hi - (lo + it * TILE), static_cast<int64_t>(TILE)));

    // -------------------------------------------------- score S^T = rows . q
    float x[NSC];
    {
      // operands are read PF steps ahead of their MFMA; each (read, MFMA) pair is
      // pinned in place so the LDS latency hides behind the previous MFMAs
      f32x16 sacc = {0};
      u32x4 kb[PF];
#pragma unroll
      for (int s = 0; s < PF; ++s) kb[s] = *reinterpret_cast<const u32x4*>(buf + sc_off[s & 3] + 128 * (s >> 2));
#pragma unroll
      for (int s = 0; s < NQ; ++s) {
        const u32x4 kv = kb[s % PF];
        if (s + PF < NQ)
          kb[s % PF] = *reinterpret_cast<const u32x4*>(buf + sc_off[(s + PF) & 3] + 128 * ((s + PF) >> 2));
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kv),
                                                       __builtin_bit_cast(bf16x8, qreg[s]), sacc, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) x[j] = sacc[j];
      if (valid < TILE) {
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (8 * (j >> 2) + 4 * g32 + (j & 3) >= valid) x[j] = NEG_INF;
      }
    }

    // first value operands: they do not depend on P, so their LDS latency
    // overlaps the softmax below
    constexpr int VSTEPS = 2 * CB;
    auto vread = [&](int st) -> bf16x8 {
      const int cbg = cg * CB + (st >> 1), u = st & 1;
      const uint8_t* bu = buf + 128 * (cbg >> 1) + 16 * u * ROWB;
      return cat(tr_read(bu + tr_off[0][cbg & 1]), tr_read(bu + tr_off[1][cbg & 1]));
    };
    bf16x8 vb[PF];
#pragma unroll
    for (int st = 0; st < PF; ++st) vb[st] = vread(st);

    // -------------------------------------------------- online softmax (log2)
    // raw scores x; the scale is folded into one FMA per element: p = 2^(x*c - m),
    // with c = scale*log2(e) > 0 so max(x*c) = c*max(x)
    float mx = x[0];
#pragma unroll
    for (int j = 1; j < NSC; ++j) mx = fmaxf(mx, x[j]);
    mx = pair_max32(mx);
    const float mt = mx * a.qscale;
    const bool need = mt > m_run + RESCALE_TAU;
    if (__ballot(need)) {
      const float m_new = need ? mt : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 when m_run = -inf
      l_run *= alpha;
#pragma unroll
      for (int c = 0; c < CB; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float e = zacc[c][r];
          float tmp;
          asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                       : "+a"(e), "=&v"(tmp) : "v"(alpha));
          zacc[c][r] = e;
        }
      m_run = m_new;
    }
    const float neg_m = -m_run;
    float p[NSC];
#pragma unroll
    for (int j = 0; j < NSC; ++j) {
      p[j] = __builtin_amdgcn_exp2f(fmaf(x[j], a.qscale, neg_m));
      l_run += p[j];
    }

    // -------------------------------------------------- value Z^T += rows^T . P^T
    bf16x8 pb[2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[u][i] = static_cast<__bf16>(p[8 * u + i]);
#pragma unroll
    for (int st = 0; st < VSTEPS; ++st) {
      const bf16x8 va = vb[st % PF];
      if (st + PF < VSTEPS) vb[st % PF] = vread(st + PF);
      zacc[st >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[st & 1], zacc[st >> 1], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }

    // every wave passed this iteration's barrier, so buffer (it+3)&3 == (it-1)&3 is free
    if (it + 3 < ntiles) issue(it + 3);
  }

  // ---- finalize: total over the lanes sharing a head, normalise, store.  The
  // normalised Z is staged row-major in the (now idle) LDS ring so that the
  // global stores are contiguous 16-byte runs along each head's row.
  const float lt = pair_sum32(l_run);
  float inv = (lt > 0.f) ? 1.f / lt : 0.f;
  float lse = (lt > 0.f) ? (m_run + log2f(lt)) * LN2 : NEG_INF;
  if (PAGED && bad) {
    inv = __builtin_nanf("");
    lse = POS_INF;
  }
  if (cg == 0 && l < HPW) lse_o[h0 + l] = lse;

  constexpr int WH = NHG * HPW;                                        // heads of the query (= n_h)
  constexpr int PCOLS = (WH * (D_C * 4 + 16) <= NBUF * TILE_BYTES) ? D_C : D_C / 2;
  constexpr int RS = PCOLS * 4 + 16;                                   // staged row stride (bytes)
  static_assert(WH * RS <= NBUF * TILE_BYTES, "staging must fit the LDS ring");
  float* zq = a.z_part + (static_cast<int64_t>(n) * a.num_splits + split) * a.n_h * D_C;
#pragma unroll
  for (int pass = 0; pass < D_C / PCOLS; ++pass) {
    const int cbase = pass * PCOLS;
    __syncthreads();  // every wave is done with the ring (tiles, or the previous pass)
    uint8_t* row = smem + (h0 + (l & 31)) * RS;
#pragma unroll
    for (int c = 0; c < CB; ++c) {
      const int cbg = cg * CB + c;
      if (32 * cbg < cbase || 32 * cbg >= cbase + PCOLS) continue;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const f32x4 v = {zacc[c][4 * jj] * inv, zacc[c][4 * jj + 1] * inv, zacc[c][4 * jj + 2] * inv,
                         zacc[c][4 * jj + 3] * inv};
        *reinterpret_cast<f32x4*>(row + 4 * (32 * cbg + 8 * jj + 4 * g32 - cbase)) = v;
      }
    }
    __syncthreads();
    constexpr int CH = PCOLS / 4;  // 16-byte chunks per staged row
    for (int idx = tid; idx < WH * CH; idx += 256) {
      const int r = idx / CH, k = idx % CH;
      *reinterpret_cast<f32x4*>(zq + static_cast<int64_t>(r) * D_C + cbase + 4 * k) =
          *reinterpret_cast<const f32x4*>(smem + r * RS + 16 * k);
    }
  }
}

// ------------------------------------------------------------------------
// n_h = 128 (the V2 shape): one workgroup streams its split once for all 128
// heads, and the work is cut two ways.
//   * score: wave w owns heads 32w..32w+31; their absorbed queries stay in
//     VGPRs as the B operand.
//   * value: wave w owns latent columns 128w..128w+127 of every head.  The
//     probabilities of all four head groups reach it through an 8 KB LDS slot,
//     so each wave transposes only its quarter of the tile's columns (a
//     quarter of the LDS reads of a head split).
//   * software pipeline: while the matrix cores score tile t+1, the same wave
//     runs the softmax of tile t (max, exp, sums), so that VALU work issues in
//     the shadow of the MFMAs; after a barrier the value MFMAs of tile t run.
// The score accumulator is kept in VGPRs by issuing those MFMAs from asm; the
// 256 AGPRs hold the Z accumulators (16 blocks of 32 columns x 32 heads).
// ------------------------------------------------------------------------
__device__ __forceinline__ void mfma_v0(f32x16& acc, const u32x4& a, const u32x4& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v(f32x16& acc, const u32x4& a, const u32x4& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
// A VALU read of an asm-issued MFMA result must wait for its write-back; 24
// idle cycles cover the 32x32x16 latency with margin.
__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

template <bool PAGED>
__global__ __launch_bounds__(256, 1) void splitkv_wide_kernel(SplitArgs a) {
  constexpr int NQ = 36;                           // score k-steps (576 / 16)
  constexpr int NBUF = 4;                          // LDS tile ring
  constexpr int LOADS = TILE_BYTES / (16 * 256);   // 9 DMA chunks per thread per tile
  constexpr int PF = 4;                            // score operand prefetch depth
  constexpr int P_OFF = NBUF * TILE_BYTES;         // P^T slots: [head group][row half][lane] x 16 B
  constexpr int A_OFF = P_OFF + 4 * 2 * 64 * 16;   // rescale factors: [head % 32][head group] floats
  constexpr int I_OFF = A_OFF + 128 * 4;           // 1 / l per head (128 floats)
  constexpr int T_OFF = I_OFF + 128 * 4;           // per-thread DMA source chunk indices, u16 [LOADS][256]
  __shared__ __attribute__((aligned(16))) uint8_t smem[T_OFF + LOADS * 256 * 2];
  static_assert(T_OFF + LOADS * 256 * 2 >= 8 * T16_BYTES, "the precise path's buffers must fit");

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int g32 = l >> 5, j16 = l & 15, l32 = l & 31;
  const int n = blockIdx.x, split = blockIdx.y;
  int b;
  int64_t len;
  query_range(a, n, b, len);
  const int64_t lo = static_cast<int64_t>(split) * a.split_rows;
  const int64_t hi = min(lo + a.split_rows, len);
  float* zo = a.z_part + (static_cast<int64_t>(n) * a.num_splits + split) * 128 * D_C;
  float* lse_o = a.lse_part + (static_cast<int64_t>(n) * a.num_splits + split) * 128;

  if (lo >= hi) {  // empty split (uniform over the workgroup)
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    for (int idx = tid; idx < 128 * D_C / 4; idx += 256) reinterpret_cast<f32x4*>(zo)[idx] = zero;
    if (tid < 128) lse_o[tid] = NEG_INF;
    return;
  }
  if (len < a.precise_below) {  // few rows: 16-head groups with hi + lo products (uniform)
    for (int g = 0; g < 8; ++g) {
      if (g) __syncthreads();
      h16_group<PAGED>(a, smem, n, split, 16 * g, b, len);
    }
    return;
  }

  // ---- tile DMA: LDS chunk f = tid + 256 i of a tile receives global chunk
  // (t, p ^ swz(t)) with (t, p) = (f / 72, f % 72).  Each thread keeps its nine
  // source chunk byte offsets in its own LDS slots (live in registers across the
  // loop they would be spilled, and a spill reload is a VMEM access that fences
  // the DMAs); only the thread itself reads them, so no barrier is needed.
  const uint8_t* gsplit =
      static_cast<const uint8_t*>(a.cache) + (static_cast<int64_t>(b) * a.stride + lo) * ROWB;
  const uint64_t gaddr = reinterpret_cast<uint64_t>(gsplit);
  const int64_t ntiles = (hi - lo + TILE - 1) / TILE;
  const uint32_t lds_w = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
                             (__attribute__((address_space(3))) uint8_t*)smem)) +
                         1024u * static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(w));
  uint16_t* otab = reinterpret_cast<uint16_t*>(smem + T_OFF);
  // A tile's buffer resource: based at the tile, sized to its rows inside the
  // split (0 past the last tile: such loads only zero-fill a free buffer, which
  // keeps the issue pattern and the vmcnt bookkeeping uniform).
  bool bad = false;  // a tile of this split sits in a page outside the pool (uniform)
  auto tile_rsrc = [&](int64_t it) {
    uint64_t ga = gaddr + static_cast<uint64_t>(it) * TILE_BYTES;
    int64_t rows = max(min(static_cast<int64_t>(TILE), hi - lo - it * TILE), static_cast<int64_t>(0));
    if constexpr (PAGED) {
      bool ok = true;
      if (rows > 0) ga = row_addr<true>(a, b, lo + it * TILE, ROWB, ok);
      if (!ok) {
        rows = 0;
        bad = true;
      }
    }
    const i32x4 rs = {__builtin_amdgcn_readfirstlane(static_cast<int>(ga & 0xffffffffu)),
                      __builtin_amdgcn_readfirstlane(static_cast<int>((ga >> 32) & 0xffffu)),
                      __builtin_amdgcn_readfirstlane(static_cast<int>(rows * ROWB)), 0x00020000};
    return rs;
  };
  // (a chunk's byte offset in the tile, chunk << 4 < 36,864, fits the u16 slot)
  auto dma = [&](int64_t it, const i32x4& rs, int i, uint32_t off) {
    dma16(lds_w + static_cast<uint32_t>((it & (NBUF - 1)) * TILE_BYTES) + 4096u * i, static_cast<int>(off), rs, 0);
  };
  {
    uint32_t ch[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int f = tid + 256 * i;
      const int t = f / 72, p = f - 72 * t;
      ch[i] = static_cast<uint32_t>(72 * t + (p ^ swz(t))) << 4;
      otab[i * 256 + tid] = static_cast<uint16_t>(ch[i]);
    }
#pragma unroll
    for (int it = 0; it < 3; ++it) {
      const i32x4 rs = tile_rsrc(it);
#pragma unroll
      for (int i = 0; i < LOADS; ++i) dma(it, rs, i, ch[i]);
    }
  }

  // ---- this wave's 32 absorbed queries: the hi plane gives the B operands
  u32x4 qreg[NQ];
  {
    const uint16_t* qh = static_cast<const uint16_t*>(a.q_lat) +
                         (static_cast<int64_t>(n) * 128 + 32 * w + l32) * ROWE + 8 * g32;
#pragma unroll
    for (int s = 0; s < NQ; ++s) qreg[s] = *reinterpret_cast<const u32x4*>(qh + 16 * s);
  }

  // ---- per-lane LDS operand offsets
  // score A: tile row l%32, elements 16 s + 8 g (chunk 2 s + g)
  int sc_off[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) sc_off[m] = l32 * ROWB + 16 * ((2 * m + g32) ^ swz(l32));
  // value A (transpose reads): rows 4g + (j16>>2) [+8], columns 16 hf + 4 (j16&3) of a 32-block
  int tr_off[2][2];
  {
    const int hf = (l >> 4) & 1;
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int p = 0; p < 2; ++p)
        tr_off[r][p] = tile_off(4 * g32 + (j16 >> 2) + 8 * r, 32 * p + 16 * hf + 4 * (j16 & 3));
  }
  auto vread = [&](const uint8_t* buf, int cbg, int u) -> bf16x8 {
    const uint8_t* bu = buf + 128 * (cbg >> 1) + 16 * u * ROWB;
    return cat(tr_read(bu + tr_off[0][cbg & 1]), tr_read(bu + tr_off[1][cbg & 1]));
  };
  auto kread = [&](const uint8_t* buf, int s) -> u32x4 {
    return *reinterpret_cast<const u32x4*>(buf + sc_off[s & 3] + 128 * (s >> 2));
  };

  vm_wait<0>();  // queries and the first tiles resident
  __syncthreads();

  // sA: scores in softmax; sB: scores being accumulated by the asm MFMAs.
  f32x16 sA, sB;
  {
    u32x4 kb[PF];
#pragma unroll
    for (int s = 0; s < PF; ++s) kb[s] = kread(smem, s);
#pragma unroll
    for (int s = 0; s < NQ; ++s) {
      const u32x4 kv = kb[s % PF];
      if (s + PF < NQ) kb[s % PF] = kread(smem, s + PF);
      if (s == 0)
        mfma_v0(sA, kv, qreg[0]);
      else
        mfma_v(sA, kv, qreg[s]);
      __builtin_amdgcn_sched_barrier(0);
    }
    mfma_drain();
  }

  f32x16 zacc[16];  // [c-block cb][head group hb] at 4 cb + hb
#pragma unroll
  for (int c = 0; c < 16; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) zacc[c][r] = 0.f;
  float m_run = NEG_INF, l_run = 0.f;
  const float qscale = a.qscale;

  // Rows of tile t inside the split: <= 0 past the last tile (every row masked).
  auto tile_valid = [&](int64_t t) {
    return static_cast<int>(max(min(hi - lo - t * TILE, static_cast<int64_t>(TILE)), static_cast<int64_t>(-1)));
  };
  // Reference update for a freshly scored tile (scores sc, masked in place):
  // the max over the head's 32 rows (lanes l and l^32), moved only when it
  // exceeds the reference by more than tau; returns the factor 2^(m_old - m_new)
  // (exactly 1 when unchanged, 0 from -inf) and rescales l_run.  A fully
  // masked tile leaves everything unchanged.  Spread over several calls with
  // `part` so that each piece fits between two MFMAs.
  float ma = 0.f, mb = 0.f, mc = 0.f, md = 0.f, me = 0.f, m_new = 0.f, alpha = 1.f;
  auto ref_update = [&](f32x16& sc, int part, int valid) {
    if (part == 0) {
      if (valid < TILE) {
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (8 * (j >> 2) + 4 * g32 + (j & 3) >= valid) sc[j] = NEG_INF;
      }
    } else if (part == 1) {
      ma = fmaxf(fmaxf(sc[0], sc[1]), sc[2]);
      mb = fmaxf(fmaxf(sc[3], sc[4]), sc[5]);
      mc = fmaxf(fmaxf(sc[6], sc[7]), sc[8]);
    } else if (part == 2) {
      md = fmaxf(fmaxf(sc[9], sc[10]), sc[11]);
      me = fmaxf(fmaxf(sc[12], sc[13]), sc[14]);
      ma = fmaxf(ma, sc[15]);
    } else if (part == 3) {
      ma = fmaxf(fmaxf(ma, mb), mc);
      md = fmaxf(md, me);
    } else if (part == 4) {
      ma = fmaxf(ma, md);
    } else if (part == 5) {
      pair_vals<false>(ma, mb, mc);
    } else if (part == 6) {
      ma = fmaxf(mb, mc) * qscale;  // scale > 0 commutes with max
    } else if (part == 7) {
      m_new = (ma > m_run + RESCALE_TAU) ? ma : m_run;
    } else if (part == 8) {
      alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    } else if (part == 9) {
      l_run *= alpha;
      m_run = m_new;
    }
  };
  // tile 0's reference (Z and l are still zero: no factor is needed)
#pragma unroll
  for (int part = 0; part < 10; ++part) ref_update(sA, part, tile_valid(0));

  // One tile step.  Entering step t: sx holds tile t's masked scores and
  // m_run / l_run already include tile t's reference update, whose factor
  // every head group published in LDS.
  //   phase 1: 36 score MFMAs of tile t+1 (into sn) with the exp pipeline of
  //            tile t and its P^T export woven in;
  //   phase 2: 32 value MFMAs of tile t with the reference update of tile t+1
  //            woven in (its factor is read by every wave in the next phase 1).
  // The DMA of tile t+3 is issued between score MFMAs (measured faster than
  // between value MFMAs).
#ifdef MLA_PHASE_STAMPS
  // cycle sums per phase: 0 wait + barrier, 1 phase 1, 2 barrier, 3 phase 2
  uint64_t ps_acc[4] = {0, 0, 0, 0};
  uint64_t ps_prev = __builtin_amdgcn_s_memtime();
  const uint64_t ps_t0 = ps_prev, ps_rt0 = __builtin_amdgcn_s_memrealtime();
  auto ps_tick = [&](int k) {
    const uint64_t now = __builtin_amdgcn_s_memtime();
    ps_acc[k] += now - ps_prev;
    ps_prev = now;
  };
#define MLA_TICK(k) ps_tick(k)
#else
#define MLA_TICK(k)
#endif
  // this lane's P^T slot reads: one base register, offsets 1024 i in the
  // instruction (the empty asm keeps the compiler from folding P_OFF, past the
  // 16-bit offset field, into each address)
  int pslot_off = P_OFF + 16 * l;
  asm volatile("" : "+v"(pslot_off));
  const uint8_t* pslot = smem + pslot_off;
  auto step = [&](int64_t t, f32x16& sx, f32x16& sn) {
    // tile t+1 must have landed (only the nine loads of tile t+2 may still be
    // in flight); every wave is done with tile t-1, whose buffer takes tile t+3
    vm_wait<LOADS>();
    __syncthreads();
    MLA_TICK(0);
    const i32x4 rs3 = tile_rsrc(t + 3);
    const uint8_t* nb = smem + ((t + 1) & (NBUF - 1)) * TILE_BYTES;
    const uint8_t* cbuf = smem + (t & (NBUF - 1)) * TILE_BYTES;
    uint32_t ch[LOADS];  // DMA source chunk index, read two MFMAs ahead of its issue

    // ---- phase 1
    bf16x8 va0, va1;
    f32x4 al4;
    {
      u32x4 kb[PF];
#pragma unroll
      for (int s = 0; s < PF; ++s) kb[s] = kread(nb, s);
      const float neg_m = -m_run;
      float y[16], p[16], ls0 = 0.f, ls1 = 0.f;
      uint32_t pw[8];  // P^T of the lane's 16 rows as packed bf16 pairs
#pragma unroll
      for (int s = 0; s < NQ; ++s) {
        const u32x4 kv = kb[s % PF];
        if (s + PF < NQ) kb[s % PF] = kread(nb, s + PF);
        if (s == 0)
          mfma_v0(sn, kv, qreg[0]);
        else
          mfma_v(sn, kv, qreg[s]);
        if (s == 0) al4 = *reinterpret_cast<const f32x4*>(smem + A_OFF + 16 * l32);  // tile t's factors
        // exp pipeline: fma in slot j, exp in slot j+1, sums and packing after
        if (s < 16) y[s] = fmaf(sx[s], qscale, neg_m);
        if (s >= 1 && s <= 16) p[s - 1] = __builtin_amdgcn_exp2f(y[s - 1]);
        if (s >= 3 && s <= 17 && (s & 1) == 1) {
          const int k = s - 3;  // p[k], p[k+1] ready
          ls0 += p[k];
          ls1 += p[k + 1];
          pw[k >> 1] = pack_bf16x2(p[k], p[k + 1]);
        }
        if (s == 18 || s == 19) {
          const int o = 4 * (s - 18);
          const u32x4 pb = {pw[o], pw[o + 1], pw[o + 2], pw[o + 3]};
          *reinterpret_cast<u32x4*>(smem + P_OFF + 2048 * w + 1024 * (s - 18) + 16 * l) = pb;
        }
        if (s == 20) l_run += ls0 + ls1;
        if (s == 33) va0 = vread(cbuf, 4 * w, 0);
        if (s == 34) va1 = vread(cbuf, 4 * w, 1);
        if (s >= 10 && s <= 10 + 2 * (LOADS - 1) && (s & 1) == 0) ch[(s - 10) >> 1] = otab[((s - 10) >> 1) * 256 + tid];
        if (s >= 12 && s <= 12 + 2 * (LOADS - 1) && (s & 1) == 0) dma(t + 3, rs3, (s - 12) >> 1, ch[(s - 12) >> 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    MLA_TICK(1);
    __syncthreads();  // P^T of every head group visible
    MLA_TICK(2);

    // ---- phase 2
    {
      // tile t's rescale (rare): a head group whose reference moved has a
      // factor != 1 in some lane; Z is still zero on the first tile
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) {
        if (t > 0 && __ballot(al4[hb] != 1.f)) {
          const float al = al4[hb];
#pragma unroll
          for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              float e = zacc[4 * cb + hb][r];
              float tmp;
              asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                           : "+a"(e), "=&v"(tmp) : "v"(al));
              zacc[4 * cb + hb][r] = e;
            }
        }
      }
      u32x4 pv[8];  // [hb][u] at 2 hb + u
#pragma unroll
      for (int i = 0; i < 8; ++i) pv[i] = *reinterpret_cast<const u32x4*>(pslot + 1024 * i);
      const int valid1 = tile_valid(t + 1);
      bf16x8 va[2][2];
      va[0][0] = va0;
      va[0][1] = va1;
#pragma unroll
      for (int v = 0; v < 32; ++v) {
        const int cb = v >> 3, hb = (v >> 1) & 3, u = v & 1;
        zacc[4 * cb + hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            va[cb & 1][u], __builtin_bit_cast(bf16x8, pv[2 * hb + u]), zacc[4 * cb + hb], 0, 0, 0);
        if (cb + 1 < 4 && (v & 7) == 1) va[(cb + 1) & 1][0] = vread(cbuf, 4 * w + cb + 1, 0);
        if (cb + 1 < 4 && (v & 7) == 2) va[(cb + 1) & 1][1] = vread(cbuf, 4 * w + cb + 1, 1);
        // tile t+1's reference update; sn's last MFMA is far behind by now
        if (v >= 8 && v < 18) ref_update(sn, v - 8, valid1);
        if (v == 18) *reinterpret_cast<float*>(smem + A_OFF + 16 * l32 + 4 * w) = alpha;
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // The scores of tile t+1 move into sA at the end of each step with asm
  // copies: their position stays after phase 2, far behind sB's last MFMA.
  for (int64_t t = 0; t < ntiles; ++t) {
    step(t, sA, sB);
    MLA_TICK(3);
    // (as eight 64-bit moves of register pairs)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      f32x2_t d;
      const f32x2_t v = {sB[2 * j], sB[2 * j + 1]};
      asm volatile("v_mov_b64 %0, %1" : "=v"(d) : "v"(v));
      sA[2 * j] = d[0];
      sA[2 * j + 1] = d[1];
    }
  }

  // ---- finalize: lse per head from its score wave; Z normalised by every
  // column wave with the head's 1/l taken from LDS.  The zero-fill loads
  // issued past the last tile are drained before the workgroup may exit.
  vm_wait<0>();
  const float lt = pair_sum32(l_run);
  float inv = (lt > 0.f) ? 1.f / lt : 0.f;
  float lse = (lt > 0.f) ? (m_run + log2f(lt)) * LN2 : NEG_INF;
  if (PAGED && bad) {
    inv = __builtin_nanf("");
    lse = POS_INF;
  }
  if (l < 32) lse_o[32 * w + l] = lse;
  *reinterpret_cast<float*>(smem + I_OFF + 4 * (32 * w + l32)) = inv;
  __syncthreads();
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    const float ih = *reinterpret_cast<const float*>(smem + I_OFF + 4 * (32 * hb + l32));
    float* zrow = zo + static_cast<int64_t>(32 * hb + l32) * D_C + 128 * w + 4 * g32;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const f32x16& zz = zacc[4 * cb + hb];
        const f32x4 v = {zz[4 * jj] * ih, zz[4 * jj + 1] * ih, zz[4 * jj + 2] * ih, zz[4 * jj + 3] * ih};
        *reinterpret_cast<f32x4*>(zrow + 32 * cb + 8 * jj) = v;
      }
  }
#ifdef MLA_PHASE_STAMPS
  {
    const uint64_t t1 = __builtin_amdgcn_s_memtime(), rt1 = __builtin_amdgcn_s_memrealtime();
    const int wg = blockIdx.x + gridDim.x * blockIdx.y;
    if (l == 0 && wg < 1024) {
      uint64_t* o = g_phase_stamps + (static_cast<int64_t>(wg) * 4 + w) * 8;
      for (int k = 0; k < 4; ++k) o[k] = ps_acc[k];
      o[4] = t1 - ps_t0;    // shader cycles from the loop's start to the end
      o[5] = rt1 - ps_rt0;  // the same span in 100 MHz ticks
      o[6] = static_cast<uint64_t>(ntiles);
    }
  }
#endif
#undef MLA_TICK
}

// n_h a multiple of 16: one workgroup per (query, split, group of 16 heads),
// one workgroup per compute unit.  A decode launch of more workgroups than
// compute units takes its units longest first.
template <bool PAGED>
__global__ __launch_bounds__(256, 1) void splitkv_h16_kernel(SplitArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[8 * T16_BYTES];
  int n = blockIdx.x, split = blockIdx.y, g = blockIdx.z;
  if (!a.prefill && gridDim.x * gridDim.y * gridDim.z > LPT_MIN_GRID)
    longest_first_unit(a, reinterpret_cast<int*>(smem), n, split, g);
  int b;
  int64_t len;
  query_range(a, n, b, len);
  h16_group<PAGED>(a, smem, n, split, 16 * g, b, len);
}

// ------------------------------------------------------------------------
// Generic fp32 VALU path (MLA_F32 storage, or bf16 with an n_h without an MFMA
// instance).  One workgroup per (query, split, head); 256 rows per step: one
// thread scores one row, then every thread accumulates two latent columns.
// ------------------------------------------------------------------------

template <typename T, bool PAGED>
__global__ __launch_bounds__(256) void splitkv_generic_kernel(SplitArgs a) {
  __shared__ float q[D_C + 2 * MAX_PAIRS];
  __shared__ float pr[256];
  __shared__ float red[4];
  const int n = blockIdx.x, split = blockIdx.y, h = blockIdx.z;
  const int tid = threadIdx.x;
  int b;
  int64_t len;
  query_range(a, n, b, len);
  const int64_t lo = static_cast<int64_t>(split) * a.split_rows;
  const int64_t hi = min(lo + a.split_rows, len);
  const int row_e = a.d_c + a.d_r;
  float* zo = a.z_part + ((static_cast<int64_t>(n) * a.num_splits + split) * a.n_h + h) * a.d_c;
  float* lse_o = a.lse_part + (static_cast<int64_t>(n) * a.num_splits + split) * a.n_h + h;
  if (lo >= hi) {
    for (int c = tid; c < a.d_c; c += 256) zo[c] = 0.f;
    if (tid == 0) *lse_o = NEG_INF;
    return;
  }
  for (int e = tid; e < row_e; e += 256) q[e] = load_q<T>(a.q_lat, a.q_lat_lo, static_cast<int64_t>(n) * a.n_h + h, row_e, e);
  __syncthreads();
  // a row of a bad page reads as zeros (as in the MFMA kernels) and poisons the split
  bool bad = false;
  auto row_ptr = [&](int64_t r, bool& ok) {
    return reinterpret_cast<const T*>(row_addr<PAGED>(a, b, r, static_cast<int64_t>(row_e) * sizeof(T), ok));
  };
  float m = NEG_INF, lsum = 0.f, z0 = 0.f, z1 = 0.f;
  for (int64_t base = lo; base < hi; base += 256) {
    const int cnt = static_cast<int>(min(static_cast<int64_t>(256), hi - base));
    float s = NEG_INF;
    if (tid < cnt) {
      bool ok;
      const T* r = row_ptr(base + tid, ok);
      float acc = 0.f;
      if (ok)
        for (int e = 0; e < row_e; ++e) acc = fmaf(q[e], load_as_f32(r, e), acc);
      else
        bad = true;
      s = acc * a.qscale;
    }
    const float mt = block_reduce(s, red, true);
    const float m_new = fmaxf(m, mt);
    const float alpha = (m == NEG_INF) ? 0.f : exp2f(m - m_new);
    const float p = (tid < cnt) ? exp2f(s - m_new) : 0.f;
    pr[tid] = p;
    const float ps = block_reduce(p, red, false);  // also orders the pr[] writes
    lsum = lsum * alpha + ps;
    z0 *= alpha;
    z1 *= alpha;
    m = m_new;
    for (int r = 0; r < cnt; ++r) {
      const float pv = pr[r];
      bool ok;
      const T* rr = row_ptr(base + r, ok);
      if (!ok) continue;
      if (tid < a.d_c) z0 = fmaf(pv, load_as_f32(rr, tid), z0);
      if (tid + 256 < a.d_c) z1 = fmaf(pv, load_as_f32(rr, tid + 256), z1);
    }
    __syncthreads();
  }
  float inv = 1.f / lsum;
  float lse = (m + log2f(lsum)) * LN2;
  if (PAGED && __syncthreads_or(bad)) {
    inv = __builtin_nanf("");
    lse = POS_INF;
  }
  if (tid < a.d_c) zo[tid] = z0 * inv;
  if (tid + 256 < a.d_c) zo[tid + 256] = z1 * inv;
  if (tid == 0) *lse_o = lse;
}

bool splitkv_has_fast_path(int n_h, int bf16, int d_c, int d_r) {
  return bf16 && d_c == D_C && d_r == D_R && (n_h == 16 || n_h == 32 || n_h == 64 || n_h == 128);
}

// Every query takes the precise path when no attended length reaches
// precise_below; the grouped 16-head kernel then runs it with one workgroup
// per (query, split, head group).
bool splitkv_all_precise(int n_h, int32_t max_len, int32_t precise_below) {
  return n_h % 16 == 0 && max_len < precise_below;
}

template <bool PAGED>
static void launch_splitkv_as(const SplitArgs& a, int bf16, hipStream_t st) {
  if (splitkv_has_fast_path(a.n_h, bf16, a.d_c, a.d_r)) {
    dim3 grid(a.n_q, a.num_splits);
    if (a.n_h == 16 || splitkv_all_precise(a.n_h, a.max_len, a.precise_below)) {
      grid.z = a.n_h / 16;
      splitkv_h16_kernel<PAGED><<<grid, 256, 0, st>>>(a);
      return;
    }
    switch (a.n_h) {
      case 32: splitkv_mfma_kernel<4, PAGED><<<grid, 256, 0, st>>>(a); break;
      case 64: splitkv_mfma_kernel<2, PAGED><<<grid, 256, 0, st>>>(a); break;
      default: splitkv_wide_kernel<PAGED><<<grid, 256, 0, st>>>(a); break;
    }
  } else {
    dim3 grid(a.n_q, a.num_splits, a.n_h);
    if (bf16)
      splitkv_generic_kernel<uint16_t, PAGED><<<grid, 256, 0, st>>>(a);
    else
      splitkv_generic_kernel<float, PAGED><<<grid, 256, 0, st>>>(a);
  }
}

hipError_t launch_splitkv(const SplitArgs& a, int bf16, hipStream_t st) {
  if (a.n_q <= 0) return hipSuccess;
  if (a.block_table)
    launch_splitkv_as<true>(a, bf16, st);
  else
    launch_splitkv_as<false>(a, bf16, st);
  return hipGetLastError();
}

}  // namespace mla

#ifdef MLA_PHASE_STAMPS
// Copies the phase stamps of the last 128-head decode launch to host memory
// (1,024 x 4 x 8 uint64); measurement build only.
extern "C" int mla_probe_phase_stamps(void* host) {
  return static_cast<int>(hipMemcpyFromSymbol(host, HIP_SYMBOL(mla::g_phase_stamps),
                                              sizeof(uint64_t) * 1024 * 4 * 8, 0, hipMemcpyDeviceToHost));
}
#endif
