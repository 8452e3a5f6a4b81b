// Quantised latent cache: c^KV as FP8 E4M3 codes with one fp32 scale per row,
// k^R in bf16 (the review's section 4 reports the served model's cache at
// about 6 bits per element but gives no format; this is the 8-bit form).
// A row of the cache is three arrays with the same row index:
//   codes [rows][d_c] uint8, rope [rows][d_hR] bf16, scale [rows] fp32,
// and stands for [E4M3(codes) * scale ; rope].  Scores and weighted sums are
// those of the bf16 path (jiphyeonjeon.kr DeepSeek-V2 review, sections 2-3)
// over the dequantised rows:
//   l_ij = (s_j (q~_i . E4M3(code_j)) + q^R_i . k^R_j) * scale
//   Z_i  = sum_j p_ij s_j E4M3(code_j)
// so the scale multiplies the latent part of a score once, and folds into the
// softmax weight before the value product; E4M3 -> bf16 is exact.
//   append_fp8_kernel: A1 into this cache (amax, scale and codes in fp32 with
//     correctly rounded divisions; the codes by the hardware's round-to-nearest-
//     even conversion);
//   splitkv_fp8_wide_kernel, splitkv_fp8_h16_kernel: A3 for 128 and 16
//     heads, the bf16 kernels' designs on the FP8 tile (see below);
//   splitkv_fp8_generic_kernel: A3 for any other head count (fp32 VALU).
#include "mla_common.h"
#include "mla_tile.h"

namespace mla {

constexpr float E4M3_MAX = 448.f;

// ------------------------------------------------------------------------
// A1 into the FP8 cache: one 64-thread workgroup per token, lane l holding
// latent elements 8l .. 8l+7.
// ------------------------------------------------------------------------
__global__ __launch_bounds__(64) void append_fp8_kernel(AppendArgs a) {
  const int t = blockIdx.x, l = threadIdx.x;
  const int64_t dst = a.row[t];
  const u32x4 raw = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.c_kv) +
                                                    static_cast<int64_t>(t) * D_C + 8 * l);
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_to_f32(static_cast<uint16_t>(raw[i] & 0xffffu));
    v[2 * i + 1] = bf16_to_f32(static_cast<uint16_t>(raw[i] >> 16));
  }
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  const float s = (m > 0.f) ? m / E4M3_MAX : 1.f;
  uint32_t w[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t x = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * h] / s, v[4 * h + 1] / s, 0, false);
    w[h] = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * h + 2] / s, v[4 * h + 3] / s, x, true);
  }
  *reinterpret_cast<uint2*>(static_cast<uint8_t*>(a.cache) + dst * D_C + 8 * l) = make_uint2(w[0], w[1]);
  if (l < D_R / 2) {
    const uint16_t* kr = static_cast<const uint16_t*>(a.k_r) + static_cast<int64_t>(t) * D_R;
    float y0, y1;
    rope_pair(bf16_to_f32(kr[2 * l]), bf16_to_f32(kr[2 * l + 1]), a.pos[t], a.rope.theta[l], y0, y1);
    reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.fp8_rope) + dst * D_R)[l] = pack_bf16x2(y0, y1);
  }
  if (l == 0) a.fp8_scale[dst] = s;
}

hipError_t launch_append_fp8(const AppendArgs& a, hipStream_t st) {
  if (a.n_tok <= 0) return hipSuccess;
  append_fp8_kernel<<<a.n_tok, 64, 0, st>>>(a);
  return hipGetLastError();
}

// 8 E4M3 codes (two dwords) -> 8 bf16 (exact), in element order
__device__ __forceinline__ u32x4 fp8x8_to_bf16(uint32_t x0, uint32_t x1) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x0, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x0, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x1, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x1, 1.0f, true);
  return u32x4{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, c),
               __builtin_bit_cast(uint32_t, d)};
}

__device__ __forceinline__ float fp8_value(uint8_t code) {
  return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(code), 0);
}

// ------------------------------------------------------------------------
// Generic A3 over the FP8 cache (any head count): one workgroup per (query,
// split, head), 256 rows per step, fp32 arithmetic on the dequantised rows.
// ------------------------------------------------------------------------
__global__ __launch_bounds__(256) void splitkv_fp8_generic_kernel(SplitArgs a) {
  __shared__ float q[ROWE];
  __shared__ float pr[256];
  __shared__ float red[4];
  const int n = blockIdx.x, split = blockIdx.y, h = blockIdx.z;
  const int tid = threadIdx.x;
  int b;
  int64_t len;
  query_range(a, n, b, len);
  const int64_t lo = static_cast<int64_t>(split) * a.split_rows;
  const int64_t hi = min(lo + a.split_rows, len);
  float* zo = a.z_part + ((static_cast<int64_t>(n) * a.num_splits + split) * a.n_h + h) * D_C;
  float* lse_o = a.lse_part + (static_cast<int64_t>(n) * a.num_splits + split) * a.n_h + h;
  if (lo >= hi) {
    for (int c = tid; c < D_C; c += 256) zo[c] = 0.f;
    if (tid == 0) *lse_o = NEG_INF;
    return;
  }
  for (int e = tid; e < ROWE; e += 256) q[e] = load_q<uint16_t>(a.q_lat, a.q_lat_lo, static_cast<int64_t>(n) * a.n_h + h, ROWE, e);
  __syncthreads();
  const int64_t base_row = static_cast<int64_t>(b) * a.stride;
  const uint8_t* codes = static_cast<const uint8_t*>(a.cache);
  const uint16_t* rope = static_cast<const uint16_t*>(a.fp8_rope);
  float m = NEG_INF, lsum = 0.f, z0 = 0.f, z1 = 0.f;
  for (int64_t base = lo; base < hi; base += 256) {
    const int cnt = static_cast<int>(min(static_cast<int64_t>(256), hi - base));
    float s = NEG_INF;
    if (tid < cnt) {
      const int64_t r = base_row + base + tid;
      float acc = 0.f;
      for (int e = 0; e < D_C; ++e) acc = fmaf(q[e], fp8_value(codes[r * D_C + e]), acc);
      float accr = 0.f;
      for (int e = 0; e < D_R; ++e) accr = fmaf(q[D_C + e], bf16_to_f32(rope[r * D_R + e]), accr);
      s = fmaf(a.fp8_scale[r], acc, accr) * a.qscale;
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
      const int64_t rr = base_row + base + r;
      const float pv = pr[r] * a.fp8_scale[rr];
      z0 = fmaf(pv, fp8_value(codes[rr * D_C + tid]), z0);
      z1 = fmaf(pv, fp8_value(codes[rr * D_C + tid + 256]), z1);
    }
    __syncthreads();
  }
  const float inv = 1.f / lsum;
  zo[tid] = z0 * inv;
  zo[tid + 256] = z1 * inv;
  if (tid == 0) *lse_o = (m + log2f(lsum)) * LN2;
}

// ------------------------------------------------------------------------
// 16 heads over the FP8 cache, and the precise path of the 128-head kernel
// (queries that attend fewer than precise_below rows, one 16-head group at a
// time): the 16-head bf16 kernel's design (mla_splitkv.hip:
// each wave streams every fourth 16-row tile into LDS buffers of its own, with
// its own online softmax and Z, merged through LDS at the end) on the FP8
// tile, which per row is 644 bytes instead of 1,152: this shape is a stream of
// the cache, so the bytes are the time.  The smaller tiles leave room for
// three buffers per wave (two tiles in flight while one is computed).
//   * a tile buffer (11 KB) holds the 16 rows' codes (8 KB; row t at 512 t,
//     chunk k at k ^ t), RoPE keys (2 KB; row t at 128 t, chunk k of 8 at
//     k ^ ((t >> 1) & 7)) and scales (64 B; lanes 0-3 of the wave's DMA);
//   * score (v_mfma_f32_16x16x32_bf16, queries hi then lo): the latent
//     products accumulate apart from the RoPE ones, and a row's score is
//     s_t latent + rope;
//   * value: the K = 32 product pairs 4 rows with P hi and the same rows with
//     P lo (P = p s_t split as bf16 hi + lo), so its operand is 4 distinct
//     rows' codes of the lane's column, used twice.  One byte-transpose read
//     serves two column blocks: lane pairs 0-3 address the 4 rows in block c,
//     pairs 4-7 the same rows in block c + 1.
// ------------------------------------------------------------------------
constexpr int H8_TILE = 16;
constexpr int NQ16 = (D_C + D_R) / 32;   // 16-head score k-steps of 32 elements
constexpr int H8_CODES = 0, H8_ROPE = 8192, H8_SCALE = 10240, H8_BUF = 11264;
constexpr int H8_LOADS = 11;   // DMAs per lane per tile: 8 code, 2 RoPE, 1 scale
constexpr int H8_ZPAD = D_C * 4 + 16;   // merge: bytes per staged head row
constexpr int H8_NB = 3;      // LDS tile buffers per wave
constexpr int H8_SMEM = (4 * 16 * H8_ZPAD + 2 * 4 * 16 * 4 > 4 * H8_NB * H8_BUF) ? 4 * 16 * H8_ZPAD + 2 * 4 * 16 * 4
                                                                                 : 4 * H8_NB * H8_BUF;

// Heads h0..h0+15 of query n over split `split` (sequence b, attended length
// len): the 16-head kernel's body, also the precise path of the 128-head
// kernel.  smem: at least H8_SMEM bytes of LDS; the caller separates two
// calls with a barrier.
__device__ __forceinline__ void h8_group(const SplitArgs& a, uint8_t* smem, int n, int split, int h0, int b,
                                         int64_t len) {
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q4 = l >> 4, j16 = l & 15;
  const int64_t lo = static_cast<int64_t>(split) * a.split_rows;
  const int64_t hi = min(lo + a.split_rows, len);
  float* zo = a.z_part + ((static_cast<int64_t>(n) * a.num_splits + split) * a.n_h + h0) * D_C;
  float* lse_o = a.lse_part + (static_cast<int64_t>(n) * a.num_splits + split) * a.n_h + h0;
  if (lo >= hi) {
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    for (int idx = tid; idx < 16 * D_C / 4; idx += 256) reinterpret_cast<f32x4*>(zo)[idx] = zero;
    if (tid < 16) lse_o[tid] = NEG_INF;
    return;
  }
  const int64_t ntiles = (hi - lo + H8_TILE - 1) / H8_TILE;
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
  // buffer H8_NB w + k % H8_NB.  Code slot f = 64 i + l holds global chunk
  // (t, p ^ t) with (t, p) = (f / 32, f % 32); RoPE slot f = 64 i + l holds
  // (t, p ^ ((t >> 1) & 7)) with (t, p) = (f / 8, f % 8); scale lane l fetches
  // bytes 16 l .. (rows 4l..4l+3).  Each buffer resource spans the tile's rows
  // inside the split, so rows past its end arrive as zeros.
  const int64_t row0 = static_cast<int64_t>(b) * a.stride + lo;
  const uint64_t gc = reinterpret_cast<uint64_t>(a.cache) + static_cast<uint64_t>(row0) * D_C;
  const uint64_t gr = reinterpret_cast<uint64_t>(a.fp8_rope) + static_cast<uint64_t>(row0) * (2 * D_R);
  const uint64_t gs = reinterpret_cast<uint64_t>(a.fp8_scale) + static_cast<uint64_t>(row0) * 4;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) uint8_t*)smem));
  auto mk_rsrc = [&](uint64_t ga, int64_t bytes) {
    const i32x4 rs = {__builtin_amdgcn_readfirstlane(static_cast<int>(ga & 0xffffffffu)),
                      __builtin_amdgcn_readfirstlane(static_cast<int>((ga >> 32) & 0xffffu)),
                      __builtin_amdgcn_readfirstlane(static_cast<int>(bytes)), 0x00020000};
    return rs;
  };
  auto issue = [&](int k, int slot) {
    const int64_t it = w + 4 * static_cast<int64_t>(k);
    const int64_t rows = min(static_cast<int64_t>(H8_TILE), hi - lo - it * H8_TILE);
    const uint64_t off = static_cast<uint64_t>(it) * H8_TILE;
    const i32x4 rc = mk_rsrc(gc + off * D_C, rows * D_C);
    const i32x4 rr = mk_rsrc(gr + off * 2 * D_R, rows * 2 * D_R);
    const i32x4 rsc = mk_rsrc(gs + off * 4, rows * 4);
    const uint32_t dst = lds0 + static_cast<uint32_t>((H8_NB * w + slot) * H8_BUF);
    // the lane index passes through an empty asm so that the source offsets
    // are formed here, not hoisted out of the loop into live registers
    int lx = l;
    asm volatile("" : "+v"(lx));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int f = 64 * i + lx;
      const int t = f >> 5, p = f & 31;
      dma16(dst + H8_CODES + 1024u * i, 16 * (32 * t + (p ^ t)), rc, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int f = 64 * i + lx;
      const int t = f >> 3, p = f & 7;
      dma16(dst + H8_ROPE + 1024u * i, 16 * (8 * t + (p ^ ((t >> 1) & 7))), rr, 0);
    }
    dma16(dst + H8_SCALE, 16 * lx, rsc, 0);
  };
  if (my_tiles > 0) issue(0, 0);
  if (my_tiles > 1) issue(1, 1);
  if (my_tiles > 2) issue(2, 2);
  vm_wait<0>();

  // ---- per-lane LDS operand offsets
  // score A, latent step s: row j16, codes 32 s + 8 q4 .. +7 = half q4 & 1 of chunk 2 s + q4 / 2
  const int sc_row = H8_CODES + 512 * j16 + 8 * (q4 & 1);
  // score A, RoPE step r: row j16, elements 32 r + 8 q4 = chunk 4 r + q4 of the row's 8
  int sr_off[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) sr_off[r] = H8_ROPE + 128 * j16 + 16 * ((4 * r + q4) ^ ((j16 >> 1) & 7));
  // value A (byte transpose) of column blocks c, c + 1 (c even): lane pair
  // jp = (l & 15) / 2 of group q4 addresses row 4 q4 + jp % 4, half l & 1 of
  // block c + jp / 4's chunk; the lane receives bytes 0-3 = its column of
  // block c over the 4 rows, bytes 4-7 = block c + 1's
  const int tr_row = 4 * q4 + (((l & 15) >> 1) & 3);
  const int tr_blk = (l & 15) >> 3;
  const int tr_base = H8_CODES + 512 * tr_row + 8 * (l & 1);
  auto vread = [&](const uint8_t* buf, int c) {
    typedef int i32x2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (__attribute__((address_space(3))) i32x2*)(buf + tr_base + 16 * ((c + tr_blk) ^ tr_row)));
  };
  // 4 codes (one dword) -> the K = 32 operand: the 4 rows' bf16 values, twice
  auto dup4 = [](uint32_t x) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true);
    const uint32_t ua = __builtin_bit_cast(uint32_t, a), ub = __builtin_bit_cast(uint32_t, b);
    return __builtin_bit_cast(bf16x8, u32x4{ua, ub, ua, ub});
  };

  f32x4 zacc[32];  // Z^T of c-block c: columns 16 c + 4 q4 + i of head j16
#pragma unroll
  for (int c = 0; c < 32; ++c) zacc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = NEG_INF, l_run = 0.f;
  const float qscale = a.qscale;

  int slot = 0;   // k % H8_NB
  for (int k = 0; k < my_tiles; ++k) {
    // this tile has landed (the next two tiles' loads may stay in flight)
    if (k + 2 < my_tiles)
      vm_wait<2 * H8_LOADS>();
    else if (k + 1 < my_tiles)
      vm_wait<H8_LOADS>();
    else
      vm_wait<0>();
    const uint8_t* buf = smem + (H8_NB * w + slot) * H8_BUF;
    const int64_t it = w + 4 * static_cast<int64_t>(k);
    const int valid = static_cast<int>(min(hi - lo - it * H8_TILE, static_cast<int64_t>(H8_TILE)));

    // -------------------------------------------------- score
    constexpr int PF = 4;
    f32x4 slat = {0.f, 0.f, 0.f, 0.f}, srope = {0.f, 0.f, 0.f, 0.f};
    {
      uint2 kb[PF];
#pragma unroll
      for (int s = 0; s < PF; ++s) kb[s] = *reinterpret_cast<const uint2*>(buf + sc_row + 16 * ((2 * s + (q4 >> 1)) ^ j16));
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const uint2 raw = kb[s % PF];
        if (s + PF < 16)
          kb[s % PF] = *reinterpret_cast<const uint2*>(buf + sc_row + 16 * ((2 * (s + PF) + (q4 >> 1)) ^ j16));
        const bf16x8 kv = __builtin_bit_cast(bf16x8, fp8x8_to_bf16(raw.x, raw.y));
        slat = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, __builtin_bit_cast(bf16x8, qh[s]), slat, 0, 0, 0);
        slat = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, __builtin_bit_cast(bf16x8, ql[s]), slat, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const bf16x8 kv = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(buf + sr_off[r]));
        srope = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, __builtin_bit_cast(bf16x8, qh[16 + r]), srope, 0, 0, 0);
        srope = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, __builtin_bit_cast(bf16x8, ql[16 + r]), srope, 0, 0, 0);
      }
    }
    // first value operands: independent of P, so their latency overlaps the softmax
    constexpr int VPF = 4;   // reads (pairs of column blocks) in flight
    typedef int i32x2 __attribute__((ext_vector_type(2)));
    i32x2 vb[VPF];
#pragma unroll
    for (int c = 0; c < VPF; ++c) vb[c] = vread(buf, 2 * c);
    const f32x4 sv = *reinterpret_cast<const f32x4*>(buf + H8_SCALE + 16 * q4);   // rows 4 q4 .. +3

    // -------------------------------------------------- online softmax (log2)
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = (4 * q4 + i < valid) ? fmaf(sv[i], slat[i], srope[i]) : NEG_INF;
    float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mx = pair_max32(mx);
    mx = pair_max16(mx);
    const float mt = mx * qscale;
    const bool need = mt > m_run + RESCALE_TAU;
    if (__ballot(need)) {
      const float m_new = need ? mt : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
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
      const float ps = pv * sv[i];   // the row's scale folds into its weight
      const uint16_t h16 = f32_to_bf16(ps);
      ph[i] = static_cast<short>(h16);
      pl[i] = static_cast<short>(f32_to_bf16(ps - bf16_to_f32(h16)));
    }
    const bf16x8 pp = cat(ph, pl);

    // -------------------------------------------------- value Z^T += rows^T . P^T
#pragma unroll
    for (int cp = 0; cp < 16; ++cp) {
      const i32x2 raw = vb[cp % VPF];
      if (cp + VPF < 16) vb[cp % VPF] = vread(buf, 2 * (cp + VPF));
      zacc[2 * cp] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dup4(static_cast<uint32_t>(raw[0])), pp, zacc[2 * cp], 0,
                                                             0, 0);
      zacc[2 * cp + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dup4(static_cast<uint32_t>(raw[1])), pp,
                                                                 zacc[2 * cp + 1], 0, 0, 0);
    }

    // the buffer is free once this wave's reads of it returned: refill it
    if (k + H8_NB < my_tiles) {
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt at their maxima
      issue(k + H8_NB, slot);
    }
    slot = (slot + 1 == H8_NB) ? 0 : slot + 1;
  }

  // ---- merge the four waves (as the bf16 kernel)
  float lt = pair_sum32(l_run);
  lt = pair_sum16(lt);
  __syncthreads();
  float* mst = reinterpret_cast<float*>(smem + 4 * 16 * H8_ZPAD);
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
  const float f = (m_run != NEG_INF && L > 0.f) ? __builtin_amdgcn_exp2f(m_run - M) / L : 0.f;
  {
    uint8_t* row = smem + w * 16 * H8_ZPAD + j16 * H8_ZPAD + 16 * q4;
#pragma unroll
    for (int c = 0; c < 32; ++c) {
      const f32x4 v = {zacc[c][0] * f, zacc[c][1] * f, zacc[c][2] * f, zacc[c][3] * f};
      *reinterpret_cast<f32x4*>(row + 64 * c) = v;
    }
  }
  if (w == 0 && q4 == 0) lse_o[j16] = (L > 0.f) ? (M + log2f(L)) * LN2 : NEG_INF;
  __syncthreads();
  for (int idx = tid; idx < 16 * (D_C / 4); idx += 256) {
    const int h = idx >> 7, c4 = idx & 127;
    f32x4 acc = *reinterpret_cast<const f32x4*>(smem + h * H8_ZPAD + 16 * c4);
#pragma unroll
    for (int v = 1; v < 4; ++v) acc += *reinterpret_cast<const f32x4*>(smem + v * 16 * H8_ZPAD + h * H8_ZPAD + 16 * c4);
    *reinterpret_cast<f32x4*>(zo + h * D_C + 4 * c4) = acc;
  }
}

// n_h a multiple of 16: one workgroup per (query, split, group of 16 heads).
__global__ __launch_bounds__(256, 1) void splitkv_fp8_h16_kernel(SplitArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[H8_SMEM];
  int n = blockIdx.x, split = blockIdx.y, g = blockIdx.z;
  if (!a.prefill && gridDim.x * gridDim.y * gridDim.z > LPT_MIN_GRID)
    longest_first_unit(a, reinterpret_cast<int*>(smem), n, split, g);
  int b;
  int64_t len;
  query_range(a, n, b, len);
  h8_group(a, smem, n, split, 16 * g, b, len);
}

// ------------------------------------------------------------------------
// 128 heads over the FP8 cache.  The work split and the pipeline are those of
// the 128-head bf16 kernel (mla_splitkv.hip): wave w scores heads 32w..32w+31
// (absorbed queries in VGPRs, asm MFMAs into VGPR scores) and accumulates
// latent columns 128w..128w+127 of every head (Z in AGPRs); the softmax of
// tile t runs under the score MFMAs of tile t+1, P^T reaches every wave
// through LDS, then the value MFMAs of tile t.  What the FP8 tile changes:
//   * a tile buffer (24 KB) holds the 32 rows' codes (16 KB; row t at 512 t,
//     16-B chunk k at k ^ (t & 31)), their RoPE keys (4 KB; row t at 128 t,
//     chunk k of 8 at k ^ ((t >> 1) & 7)) and the 32 scales (one 128-B copy
//     per wave, at 1 KB apart: every wave issues the same DMAs);
//   * score: the 32 latent k-steps read 8 codes per lane (ds_read_b64) and
//     convert them to bf16 (exact) for the MFMA; after them the scores are
//     multiplied by their rows' scales, then the 4 RoPE k-steps add
//     q^R . k^R;
//   * value: one LDS byte-transpose read (ds_read_b64_tr_b8) gives a lane the
//     8 codes of its column over 8 rows; converted to bf16 they are the A
//     operand; the softmax weights go out as bf16(p s_j) while l sums p.
// ------------------------------------------------------------------------
// Score MFMAs from asm (VGPR accumulators).  Their A operands come from VALU
// conversions just before, and an MFMA reads a VALU-written source only after
// 2 wait states, which the compiler does not insert for asm: hence s_nop 1.
__device__ __forceinline__ void f8_mfma0(f32x16& acc, const u32x4& a, const u32x4& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void f8_mfma(f32x16& acc, const u32x4& a, const u32x4& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
// a VALU read of an asm MFMA's result waits for its write-back (24 wait states)
__device__ __forceinline__ void f8_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

constexpr int F8_TILE = 32;
constexpr int F8_CODES = 0;           // codes region of a tile buffer
constexpr int F8_ROPE = 16384;        // RoPE keys
constexpr int F8_SCALE = 20480;       // scales, one 1 KB slot per wave
constexpr int F8_BUF = 24576;         // bytes per tile buffer
constexpr int F8_LOADS = 6;           // DMAs per thread per tile: 4 code chunks, 1 RoPE chunk, 1 scale chunk

__global__ __launch_bounds__(256, 1) void splitkv_fp8_wide_kernel(SplitArgs a) {
  constexpr int NQ = 36;                           // score k-steps: 32 latent + 4 RoPE
  constexpr int NBUF = 4;                          // LDS tile ring
  constexpr int PF = 4;                            // score operand prefetch depth
  constexpr int P_OFF = NBUF * F8_BUF;             // P^T slots: [head group][row half][lane] x 16 B
  constexpr int A_OFF = P_OFF + 4 * 2 * 64 * 16;   // rescale factors: [head % 32][head group] floats
  constexpr int I_OFF = A_OFF + 128 * 4;           // 1 / l per head (128 floats)
  constexpr int T_OFF = I_OFF + 128 * 4;           // per-thread DMA source chunk indices, u16 [5][256]
  // (the precise path's 16-head groups need H8_SMEM bytes; one workgroup per CU either way)
  constexpr int SMEM = (T_OFF + 5 * 256 * 2 > H8_SMEM) ? T_OFF + 5 * 256 * 2 : H8_SMEM;
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int g32 = l >> 5, l32 = l & 31;
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
      h8_group(a, smem, n, split, 16 * g, b, len);
    }
    return;
  }

  // ---- tile DMA.  Code slot f = tid + 256 i (i < 4) of a tile holds global
  // chunk (t, p ^ (t & 31)) with (t, p) = (f / 32, f % 32); RoPE slot tid holds
  // chunk (t, p ^ ((t >> 1) & 7)) with (t, p) = (tid / 8, tid % 8); lane l of
  // each wave fetches scale chunk l (rows 4l..4l+3; lanes past the tile's rows
  // read zeros).  Source chunk indices live in a per-thread LDS table.
  const int64_t row0 = static_cast<int64_t>(b) * a.stride + lo;
  const uint64_t gc = reinterpret_cast<uint64_t>(a.cache) + static_cast<uint64_t>(row0) * D_C;
  const uint64_t gr = reinterpret_cast<uint64_t>(a.fp8_rope) + static_cast<uint64_t>(row0) * (2 * D_R);
  const uint64_t gs = reinterpret_cast<uint64_t>(a.fp8_scale) + static_cast<uint64_t>(row0) * 4;
  const int64_t ntiles = (hi - lo + F8_TILE - 1) / F8_TILE;
  const uint32_t lds_w = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
                             (__attribute__((address_space(3))) uint8_t*)smem)) +
                         1024u * static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(w));
  uint16_t* otab = reinterpret_cast<uint16_t*>(smem + T_OFF);
  auto mk_rsrc = [&](uint64_t ga, int64_t bytes) {
    const i32x4 rs = {__builtin_amdgcn_readfirstlane(static_cast<int>(ga & 0xffffffffu)),
                      __builtin_amdgcn_readfirstlane(static_cast<int>((ga >> 32) & 0xffffu)),
                      __builtin_amdgcn_readfirstlane(static_cast<int>(bytes)), 0x00020000};
    return rs;
  };
  // a tile's three buffer resources, sized to its rows inside the split (0 past
  // the last tile: such loads only zero-fill a free buffer)
  struct TileRs {
    i32x4 c, r, s;
  };
  auto tile_rsrc = [&](int64_t it) {
    const int64_t rows = max(min(static_cast<int64_t>(F8_TILE), hi - lo - it * F8_TILE), static_cast<int64_t>(0));
    const uint64_t off = static_cast<uint64_t>(it) * F8_TILE;
    return TileRs{mk_rsrc(gc + off * D_C, rows * D_C), mk_rsrc(gr + off * 2 * D_R, rows * 2 * D_R),
                  mk_rsrc(gs + off * 4, rows * 4)};
  };
  // DMA d (0..5) of tile it; chunk = source chunk index (16 B) inside the region
  auto dma = [&](int64_t it, const TileRs& rs, int d, uint32_t chunk) {
    const uint32_t base = lds_w + static_cast<uint32_t>((it & (NBUF - 1)) * F8_BUF);
    if (d < 4)
      dma16(base + F8_CODES + 4096u * d, static_cast<int>(chunk << 4), rs.c, 0);
    else if (d == 4)
      dma16(base + F8_ROPE, static_cast<int>(chunk << 4), rs.r, 0);
    else
      dma16(base + F8_SCALE, static_cast<int>(chunk << 4), rs.s, 0);
  };
  {
    uint32_t ch[F8_LOADS];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int f = tid + 256 * i;
      const int t = f >> 5, p = f & 31;
      ch[i] = static_cast<uint32_t>(32 * t + (p ^ (t & 31)));
      otab[i * 256 + tid] = static_cast<uint16_t>(ch[i]);
    }
    {
      const int t = tid >> 3, p = tid & 7;
      ch[4] = static_cast<uint32_t>(8 * t + (p ^ ((t >> 1) & 7)));
      otab[4 * 256 + tid] = static_cast<uint16_t>(ch[4]);
    }
    ch[5] = static_cast<uint32_t>(l);
#pragma unroll
    for (int it = 0; it < 3; ++it) {
      const TileRs rs = tile_rsrc(it);
#pragma unroll
      for (int d = 0; d < F8_LOADS; ++d) dma(it, rs, d, ch[d]);
    }
  }

  // ---- this wave's 32 absorbed queries: the hi parts are the B operands
  u32x4 qreg[NQ];
  {
    const uint16_t* qh = static_cast<const uint16_t*>(a.q_lat) +
                         (static_cast<int64_t>(n) * 128 + 32 * w + l32) * ROWE + 8 * g32;
#pragma unroll
    for (int s = 0; s < NQ; ++s) qreg[s] = *reinterpret_cast<const u32x4*>(qh + 16 * s);
  }

  // ---- per-lane LDS operand offsets
  // score A, latent step s: row l32, codes 16 s + 8 g .. +7 = half g of chunk s
  const int sc_row = F8_CODES + 512 * l32 + 8 * g32;
  // score A, RoPE step r: row l32, elements 16 r + 8 g = chunk 2 r + g of the row's 8
  int sr_off[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) sr_off[r] = F8_ROPE + 128 * l32 + 16 * ((2 * r + g32) ^ ((l32 >> 1) & 7));
  // value A (byte-transpose read): a 16-lane group's 8 lane pairs supply 8
  // rows (16 bytes each, the pair's two halves) and lane i of the group
  // receives byte i of each, in pair order.  K position k of the value product
  // must name the tile row that the softmax weights' B operand holds there:
  // row 16 u + 8 (k / 4) + 4 g + k % 4 for lanes of half g = l / 32 (the score
  // accumulator's layout).  So pair j of group G addresses that row for k = j,
  // bytes 8 (i % 2) .. +7 of chunk 2 cbg + G % 2, and lane i receives column
  // 16 (G % 2) + i of the 32-column block.
  const int tr_j = (l & 15) >> 1;
  const int tr_row = 8 * (tr_j >> 2) + 4 * (l >> 5) + (tr_j & 3);   // + 16 u
  const int tr_half = 8 * (l & 1);
  const int tr_g = (l >> 4) & 1;
  auto vread = [&](const uint8_t* buf, int cbg, int u) -> bf16x8 {
    const int row = tr_row + 16 * u;
    const int pos = (2 * cbg + tr_g) ^ (row & 31);
    typedef int i32x2 __attribute__((ext_vector_type(2)));
    const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (__attribute__((address_space(3))) i32x2*)(buf + F8_CODES + 512 * row + 16 * pos + tr_half));
    return __builtin_bit_cast(bf16x8, fp8x8_to_bf16(static_cast<uint32_t>(x[0]), static_cast<uint32_t>(x[1])));
  };
  // score operand of step s as raw bits (8 codes in .xy for a latent step,
  // 8 bf16 for a RoPE step)
  auto kread = [&](const uint8_t* buf, int s) -> u32x4 {
    if (s < 32) {
      const int pos = s ^ l32;
      const uint2 x = *reinterpret_cast<const uint2*>(buf + sc_row + 16 * pos);
      return u32x4{x.x, x.y, 0u, 0u};
    }
    return *reinterpret_cast<const u32x4*>(buf + sr_off[s - 32]);
  };
  auto kconv = [&](const u32x4& raw, int s) -> u32x4 { return (s < 32) ? fp8x8_to_bf16(raw[0], raw[1]) : raw; };
  // the lane's 16 rows' scales: rows 8 (j / 4) + 4 g + j % 4 -> four 16-B reads
  auto scales = [&](const uint8_t* buf, f32x4* sv) {
#pragma unroll
    for (int q = 0; q < 4; ++q) sv[q] = *reinterpret_cast<const f32x4*>(buf + F8_SCALE + 1024 * w + 4 * (8 * q + 4 * g32));
  };
  // latent scores of a tile -> times their rows' scales (after the drain)
  auto scale_scores = [&](f32x16& sc, const f32x4* sv) {
#pragma unroll
    for (int j = 0; j < 16; ++j) sc[j] *= sv[j >> 2][j & 3];
  };

  vm_wait<0>();  // queries and the first tiles resident
  __syncthreads();

  // sA: scores in softmax; sB: scores being accumulated by the asm MFMAs.
  f32x16 sA, sB;
  {
    u32x4 kb[PF];
    f32x4 sv[4];
#pragma unroll
    for (int s = 0; s < PF; ++s) kb[s] = kread(smem, s);
#pragma unroll
    for (int s = 0; s < NQ; ++s) {
      const u32x4 kv = kconv(kb[s % PF], s);
      if (s + PF < NQ) kb[s % PF] = kread(smem, s + PF);
      if (s == 28) scales(smem, sv);
      if (s == 32) {
        f8_drain();
        scale_scores(sA, sv);
      }
      if (s == 0)
        f8_mfma0(sA, kv, qreg[0]);
      else
        f8_mfma(sA, kv, qreg[s]);
      __builtin_amdgcn_sched_barrier(0);
    }
    f8_drain();
  }

  f32x16 zacc[16];  // [c-block cb][head group hb] at 4 cb + hb
#pragma unroll
  for (int c = 0; c < 16; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) zacc[c][r] = 0.f;
  float m_run = NEG_INF, l_run = 0.f;
  const float qscale = a.qscale;

  auto tile_valid = [&](int64_t t) {
    return static_cast<int>(max(min(hi - lo - t * F8_TILE, static_cast<int64_t>(F8_TILE)), static_cast<int64_t>(-1)));
  };
  // Reference update for a freshly scored tile, spread over `part` calls (as in
  // the bf16 kernel): mask, max over the head's 32 rows, lazy move by > tau,
  // factor 2^(m_old - m_new), l rescaled.
  float ma = 0.f, mb = 0.f, mc = 0.f, md = 0.f, me = 0.f, m_new = 0.f, alpha = 1.f;
  auto ref_update = [&](f32x16& sc, int part, int valid) {
    if (part == 0) {
      if (valid < F8_TILE) {
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
      ma = fmaxf(mb, mc) * qscale;
    } else if (part == 7) {
      m_new = (ma > m_run + RESCALE_TAU) ? ma : m_run;
    } else if (part == 8) {
      alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    } else if (part == 9) {
      l_run *= alpha;
      m_run = m_new;
    }
  };
#pragma unroll
  for (int part = 0; part < 10; ++part) ref_update(sA, part, tile_valid(0));

  // One tile step (as the bf16 kernel): phase 1 scores tile t+1 into sn with
  // tile t's exponentials and P^T export woven in; phase 2 runs tile t's value
  // MFMAs with tile t+1's reference update woven in.
  auto step = [&](int64_t t, f32x16& sx, f32x16& sn) {
    // tile t+1 landed (only tile t+2's loads may be in flight); tile t-1's
    // buffer is free for tile t+3
    vm_wait<F8_LOADS>();
    __syncthreads();
    const TileRs rs3 = tile_rsrc(t + 3);
    const uint8_t* nb = smem + ((t + 1) & (NBUF - 1)) * F8_BUF;
    const uint8_t* cbuf = smem + (t & (NBUF - 1)) * F8_BUF;
    uint32_t ch[F8_LOADS];

    // ---- phase 1
    bf16x8 va0, va1;
    f32x4 al4;
    {
      f32x4 pscale[4];   // tile t's scales of the lane's 16 rows (softmax weights)
      scales(cbuf, pscale);
      f32x4 sv[4];       // tile t+1's, for its scores
      u32x4 kb[PF];
#pragma unroll
      for (int s = 0; s < PF; ++s) kb[s] = kread(nb, s);
      const float neg_m = -m_run;
      float y[16], p[16], ls0 = 0.f, ls1 = 0.f;
      uint32_t pw[8];  // P^T of the lane's 16 rows (times the rows' scales) as bf16 pairs
#pragma unroll
      for (int s = 0; s < NQ; ++s) {
        const u32x4 kv = kconv(kb[s % PF], s);
        if (s + PF < NQ) kb[s % PF] = kread(nb, s + PF);
        if (s == 28) scales(nb, sv);
        if (s == 32) {
          f8_drain();
          scale_scores(sn, sv);
        }
        if (s == 0)
          f8_mfma0(sn, kv, qreg[0]);
        else
          f8_mfma(sn, kv, qreg[s]);
        if (s == 0) al4 = *reinterpret_cast<const f32x4*>(smem + A_OFF + 16 * l32);  // tile t's factors
        if (s < 16) y[s] = fmaf(sx[s], qscale, neg_m);
        if (s >= 1 && s <= 16) p[s - 1] = __builtin_amdgcn_exp2f(y[s - 1]);
        if (s >= 3 && s <= 17 && (s & 1) == 1) {
          const int k = s - 3;  // p[k], p[k+1] ready
          ls0 += p[k];
          ls1 += p[k + 1];
          pw[k >> 1] = pack_bf16x2(p[k] * pscale[k >> 2][k & 3], p[k + 1] * pscale[(k + 1) >> 2][(k + 1) & 3]);
        }
        if (s == 18 || s == 19) {
          const int o = 4 * (s - 18);
          const u32x4 pb = {pw[o], pw[o + 1], pw[o + 2], pw[o + 3]};
          *reinterpret_cast<u32x4*>(smem + P_OFF + 2048 * w + 1024 * (s - 18) + 16 * l) = pb;
        }
        if (s == 20) l_run += ls0 + ls1;
        if (s == 34) va0 = vread(cbuf, 4 * w, 0);
        if (s == 35) va1 = vread(cbuf, 4 * w, 1);
        if (s >= 10 && s <= 18 && (s & 1) == 0) {
          const int d = (s - 10) >> 1;  // 0..4 from the table, 5 = the lane's scale chunk
          ch[d] = (d < 5) ? otab[d * 256 + tid] : static_cast<uint32_t>(l);
        }
        if (s >= 12 && s <= 22 && (s & 1) == 0) {
          const int d = (s - 12) >> 1;
          if (d == 5) ch[5] = static_cast<uint32_t>(l);
          dma(t + 3, rs3, d, ch[d]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();  // P^T of every head group visible

    // ---- phase 2
    {
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
      for (int i = 0; i < 8; ++i) pv[i] = *reinterpret_cast<const u32x4*>(smem + P_OFF + 1024 * i + 16 * l);
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
        if (v >= 8 && v < 18) ref_update(sn, v - 8, valid1);
        if (v == 18) *reinterpret_cast<float*>(smem + A_OFF + 16 * l32 + 4 * w) = alpha;
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  for (int64_t t = 0; t < ntiles; ++t) {
    step(t, sA, sB);
#pragma unroll
    for (int j = 0; j < 16; ++j) asm volatile("v_mov_b32 %0, %1" : "=v"(sA[j]) : "v"(sB[j]));
  }

  // ---- finalize (as the bf16 kernel)
  vm_wait<0>();
  const float lt = pair_sum32(l_run);
  const float inv = (lt > 0.f) ? 1.f / lt : 0.f;
  if (l < 32) lse_o[32 * w + l] = (lt > 0.f) ? (m_run + log2f(lt)) * LN2 : NEG_INF;
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
}

hipError_t launch_splitkv_fp8(const SplitArgs& a, hipStream_t st) {
  if (a.n_q <= 0) return hipSuccess;
  if (a.n_h == 16 || (a.n_h == 128 && splitkv_all_precise(a.n_h, a.max_len, a.precise_below))) {
    splitkv_fp8_h16_kernel<<<dim3(a.n_q, a.num_splits, a.n_h / 16), 256, 0, st>>>(a);
  } else if (a.n_h == 128) {
    splitkv_fp8_wide_kernel<<<dim3(a.n_q, a.num_splits), 256, 0, st>>>(a);
  } else {
    splitkv_fp8_generic_kernel<<<dim3(a.n_q, a.num_splits, a.n_h), 256, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace mla
