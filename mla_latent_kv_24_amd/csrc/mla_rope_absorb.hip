// A1 (cache append with decoupled RoPE key) and A2 (absorbed query) for gfx950.
//
// A1 writes row = [c^KV ; RoPE(k_raw, pos)] (jiphyeonjeon.kr DeepSeek-V2 review,
// section 3: one 64-d RoPE key per token shared by all heads; DeepSeek-V3 report
// on xyznot.com, Metode 1: only c^KV and k^R are cached).
// A2 folds U^K_i into the query, q~_i = (U^K_i)^T q^C_i (review section 2), and
// rotates the per-head RoPE query by the token position (review section 3).
// Both are formed in fp32 and stored in the storage dtype: fp32, or bf16
// hi = bf16(v) (the matrix-core operand) with, when the caller provides the
// plane, lo = bf16(v - hi) beside it.
#include "mla_common.h"

namespace mla {

// ------------------------------------------------------------- A1: append
// One workgroup of 64 threads per token.  Threads copy the latent in 16-byte
// pieces; the first d_r/2 threads rotate one RoPE pair each.
template <typename T>
__global__ __launch_bounds__(64) void append_kernel(AppendArgs a) {
  const int t = blockIdx.x;
  const int64_t dst_row = a.row[t];
  const int32_t pos = a.pos[t];
  const T* src_c = static_cast<const T*>(a.c_kv) + static_cast<int64_t>(t) * a.d_c;
  const T* src_r = static_cast<const T*>(a.k_r) + static_cast<int64_t>(t) * a.d_r;
  T* dst = static_cast<T*>(a.cache) + dst_row * (a.d_c + a.d_r);
  for (int e = threadIdx.x; e < a.d_c; e += 64) dst[e] = src_c[e];
  for (int k = threadIdx.x; k < a.d_r / 2; k += 64) {
    float y0, y1;
    rope_pair(load_as_f32(src_r, 2 * k), load_as_f32(src_r, 2 * k + 1), pos, a.rope.theta[k], y0,
              y1);
    dst[a.d_c + 2 * k] = store_from_f32<T>(y0);
    dst[a.d_c + 2 * k + 1] = store_from_f32<T>(y1);
  }
}

// ------------------------------------------------------ A2, RoPE query part
// One workgroup per query: sine/cosine of the d_r/2 angles once, then every
// head's pair is rotated with them.
template <typename T>
__global__ __launch_bounds__(256) void rope_q_kernel(RopeQArgs a) {
  __shared__ float cs[MAX_PAIRS], sn[MAX_PAIRS];
  const int n = blockIdx.x;
  const int pairs = a.d_r / 2;
  const int32_t pos = a.q_pos[n];
  for (int k = threadIdx.x; k < pairs; k += blockDim.x) {
    double s, c;
    sincos(static_cast<double>(pos) * a.rope.theta[k], &s, &c);
    cs[k] = static_cast<float>(c);
    sn[k] = static_cast<float>(s);
  }
  __syncthreads();
  const T* src = static_cast<const T*>(a.q_r) + static_cast<int64_t>(n) * a.n_h * a.d_r;
  const int row_e = a.d_c + a.d_r;
  for (int idx = threadIdx.x; idx < a.n_h * pairs; idx += blockDim.x) {
    const int h = idx / pairs, k = idx % pairs;
    const float x0 = load_as_f32(src, h * a.d_r + 2 * k);
    const float x1 = load_as_f32(src, h * a.d_r + 2 * k + 1);
    const int64_t nh = static_cast<int64_t>(n) * a.n_h + h;
    store_q<T>(a.q_lat, a.q_lat_lo, nh, row_e, a.d_c + 2 * k, x0 * cs[k] - x1 * sn[k]);
    store_q<T>(a.q_lat, a.q_lat_lo, nh, row_e, a.d_c + 2 * k + 1, x0 * sn[k] + x1 * cs[k]);
  }
}

// --------------------------------------------- A2, latent part, generic fp32
// One workgroup per (query, head); thread c accumulates sum_d q_c[d] w_uk[d][c].
template <typename T>
__global__ __launch_bounds__(256) void absorb_generic_kernel(AbsorbArgs a) {
  __shared__ float q[1024];
  const int n = blockIdx.x, h = blockIdx.y;
  const T* qc = static_cast<const T*>(a.q_c) + (static_cast<int64_t>(n) * a.n_h + h) * a.d_h;
  for (int d = threadIdx.x; d < a.d_h; d += blockDim.x) q[d] = load_as_f32(qc, d);
  __syncthreads();
  const T* w = static_cast<const T*>(a.w_uk) + static_cast<int64_t>(h) * a.d_h * a.d_c;
  const int64_t nh = static_cast<int64_t>(n) * a.n_h + h;
  for (int c = threadIdx.x; c < a.d_c; c += blockDim.x) {
    float acc = 0.f;
    for (int d = 0; d < a.d_h; ++d) acc = fmaf(q[d], load_as_f32(w, static_cast<int64_t>(d) * a.d_c + c), acc);
    store_q<T>(a.q_lat, a.q_lat_lo, nh, a.d_c + a.d_r, c, acc);
  }
}

// ---------------------------------------------- A2, bf16 MFMA path (fused)
// Per head i: q_lat[n, i, 0:512] = q_c[n, i, :] @ w_uk[i]  ([n x 128] @ [128 x 512])
// and q_lat[n, i, 512:] = RoPE(q_r[n, i], q_pos[n]), in one launch.
// Grid (head, column quarter, query chunk of 256), two workgroups per CU so
// that one's loads overlap the other's products and stores.  The workgroup
// issues the loads of its [128 d][128 c] slab of W^UK, of its first query
// block and of its quarter of the head's RoPE pairs, stages the slab in LDS
// (a row stride of 64 B past a multiple of 128 B keeps the four rows of a
// transpose read in distinct banks), rotates its RoPE pairs,
// and runs 32-query blocks through v_mfma_f32_32x32x16_bf16: A = q_c rows from
// global memory (d contiguous), B = W^UK columns via ds_read_b64_tr_b16.
// Results are staged in LDS so that hi (and lo, when its plane is given)
// leave as 16-byte stores.
constexpr int ABS_QCHUNK = 256;
constexpr int ABS_COLS = 128;                      // latent columns per workgroup (a quarter of d_c)
constexpr int ABS_PARTS = D_C / ABS_COLS;          // workgroups per head
constexpr int ABS_WSTRIDE = ABS_COLS * 2 + 64;     // bytes per staged W row (bf16 + 64 B pad)
constexpr int ABS_SSTRIDE = ABS_COLS * 4 + 16;     // bytes per staged fp32 output row
constexpr int ABS_PAIRS = D_R / 2 / ABS_PARTS;     // RoPE pairs rotated per workgroup

// Fused A1 (mla_append_absorb): the workgroup with linear index k writes the
// appended rows t = k, k + (grid size), ...; per row, threads 0..63 copy the
// latent as 16-B pieces and threads 64..95 rotate one RoPE pair each (fp64
// angle, as append_kernel).  The first row's loads are issued before the A2
// loads, so that they land while the slab streams in.
struct AppendPiece {
  uint4 c;       // latent piece (threads 0..63)
  uint32_t k;    // pre-RoPE pair (threads 64..95)
  int32_t pos;
};
__device__ __forceinline__ AppendPiece append_load(const AbsorbArgs& a, int t, int tid) {
  AppendPiece p{make_uint4(0, 0, 0, 0), 0u, 0};
  if (tid < D_C / 8) {
    p.c = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.app_c) + static_cast<int64_t>(t) * D_C + 8 * tid);
  } else if (tid < D_C / 8 + D_R / 2) {
    const int k = tid - D_C / 8;
    p.k = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.app_k) + static_cast<int64_t>(t) * D_R + 2 * k);
    p.pos = a.app_pos[t];
  }
  return p;
}
__device__ __forceinline__ void append_store(const AbsorbArgs& a, int t, int tid, const AppendPiece& p) {
  uint16_t* dst = static_cast<uint16_t*>(a.app_cache) + a.app_row[t] * ROWE;
  if (tid < D_C / 8) {
    *reinterpret_cast<uint4*>(dst + 8 * tid) = p.c;
  } else if (tid < D_C / 8 + D_R / 2) {
    const int k = tid - D_C / 8;
    float y0, y1;
    rope_pair(bf16_to_f32(static_cast<uint16_t>(p.k & 0xffffu)), bf16_to_f32(static_cast<uint16_t>(p.k >> 16)),
              p.pos, a.rope.theta[k], y0, y1);
    *reinterpret_cast<uint32_t*>(dst + D_C + 2 * k) = pack_bf16x2(y0, y1);
  }
}

__global__ __launch_bounds__(256, 2) void absorb_mfma_kernel(AbsorbArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t wlds[D_H * ABS_WSTRIDE];
  __shared__ __attribute__((aligned(16))) uint8_t stage[32 * ABS_SSTRIDE];
  const int h = blockIdx.x, half_c = blockIdx.y;
  const int n_begin = blockIdx.z * ABS_QCHUNK;
  const int n_end = min(n_begin + ABS_QCHUNK, a.n_q);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int g = l >> 5;  // k-half of the 32x32x16 operand
  const uint16_t* qc = static_cast<const uint16_t*>(a.q_c);
  uint16_t* qout = static_cast<uint16_t*>(a.q_lat);
  uint16_t* qlo = static_cast<uint16_t*>(a.q_lat_lo);   // NULL: hi only

  // ---- fused A1: this workgroup's first appended row, loads in flight
  const int wg = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  const int nwg = gridDim.x * gridDim.y * gridDim.z;
  AppendPiece app{};
  if (wg < a.app_n) app = append_load(a, wg, tid);

  // ---- issue: W^UK slab (16 chunks of 16 B per thread) and the first query block
  constexpr int WCH = ABS_COLS / 8;             // 16-B chunks per W row of the slab
  constexpr int WLOADS = D_H * WCH / 256;         // chunks per thread
  const uint16_t* wsrc = static_cast<const uint16_t*>(a.w_uk) + static_cast<int64_t>(h) * D_H * D_C + half_c * ABS_COLS;
  uint4 wv[WLOADS];
#pragma unroll
  for (int i = 0; i < WLOADS; ++i) {
    const int f = tid + 256 * i, d = f / WCH, k = f % WCH;
    wv[i] = *reinterpret_cast<const uint4*>(wsrc + static_cast<int64_t>(d) * D_C + 8 * k);
  }
  auto load_q = [&](int n0, uint4 (&qa)[8]) {
    const int n = n0 + (l & 31);
#pragma unroll
    for (int s = 0; s < 8; ++s)
      qa[s] = (n < n_end) ? *reinterpret_cast<const uint4*>(qc + (static_cast<int64_t>(n) * a.n_h + h) * D_H + 16 * s + 8 * g)
                          : make_uint4(0, 0, 0, 0);
  };
  uint4 qa[8];
  load_q(n_begin, qa);

  // RoPE inputs of this workgroup's share of the pairs: column part pc rotates
  // pairs ABS_PAIRS pc .. +ABS_PAIRS-1 of its head for every query of the chunk
  constexpr int RITEMS = ABS_QCHUNK * ABS_PAIRS / 256;  // (query, pair) items per thread
  // (q_r holds bf16 pairs, or fp32 pairs when q_r_f32 is set)
  float2 xr[RITEMS];
  int32_t rpos[RITEMS];
#pragma unroll
  for (int it = 0; it < RITEMS; ++it) {
    const int idx = tid + 256 * it, n = n_begin + idx / ABS_PAIRS, k = ABS_PAIRS * half_c + idx % ABS_PAIRS;
    xr[it] = make_float2(0.f, 0.f);
    rpos[it] = 0;
    if (n < n_end) {
      const int64_t e = (static_cast<int64_t>(n) * a.n_h + h) * D_R + 2 * k;
      if (a.q_r_f32) {
        xr[it] = *reinterpret_cast<const float2*>(static_cast<const float*>(a.q_r) + e);
      } else {
        const uint32_t x = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.q_r) + e);
        xr[it] = make_float2(bf16_to_f32(static_cast<uint16_t>(x & 0xffffu)), bf16_to_f32(static_cast<uint16_t>(x >> 16)));
      }
      rpos[it] = a.q_pos[n];
    }
  }

  // the slab into LDS (its registers are free before the fp64 RoPE math)
#pragma unroll
  for (int i = 0; i < WLOADS; ++i) {
    const int f = tid + 256 * i, d = f / WCH, k = f % WCH;
    *reinterpret_cast<uint4*>(wlds + d * ABS_WSTRIDE + 16 * k) = wv[i];
  }

  // angle and sine/cosine in fp64, rotation in fp32
#pragma unroll
  for (int it = 0; it < RITEMS; ++it) {
    const int idx = tid + 256 * it, n = n_begin + idx / ABS_PAIRS, k = ABS_PAIRS * half_c + idx % ABS_PAIRS;
    if (n < n_end) {
      double sd, cd;
      sincos(static_cast<double>(rpos[it]) * a.rope.theta[k], &sd, &cd);
      const float cf = static_cast<float>(cd), sf = static_cast<float>(sd);
      const float x0 = xr[it].x, x1 = xr[it].y;
      const float y0 = x0 * cf - x1 * sf, y1 = x0 * sf + x1 * cf;
      const float h0 = bf16_to_f32(f32_to_bf16(y0)), h1 = bf16_to_f32(f32_to_bf16(y1));
      const int64_t e = (static_cast<int64_t>(n) * a.n_h + h) * ROWE + D_C + 2 * k;
      *reinterpret_cast<uint32_t*>(qout + e) = pack_bf16x2(y0, y1);
      if (qlo) *reinterpret_cast<uint32_t*>(qlo + e) = pack_bf16x2(y0 - h0, y1 - h1);
    }
  }
  // fused A1: the first row (its loads have landed with the slab's), then any
  // further rows of this workgroup (more rows than workgroups)
  if (wg < a.app_n) {
    append_store(a, wg, tid, app);
    for (int t = wg + nwg; t < a.app_n; t += nwg) append_store(a, t, tid, append_load(a, t, tid));
  }
  __syncthreads();

  const int j16 = l & 15, hf = (l >> 4) & 1;
  // transpose-read address pieces: row d = 16s + 8g + (j16>>2) [+4], column 32cb + 16hf + 4(j16&3)
  const int tr_row = 8 * g + (j16 >> 2);
  const int tr_col_b = 2 * (16 * hf + 4 * (j16 & 3));

  for (int n0 = n_begin; n0 < n_end; n0 += 32) {
    uint4 qn[8];
    if (n0 + 32 < n_end) load_q(n0 + 32, qn);  // next block in flight during this one
#pragma unroll
    for (int cbl = 0; cbl < ABS_COLS / 128; ++cbl) {
      const int cb = (ABS_COLS / 128) * w + cbl;  // 32-column block inside this part
      f32x16 acc = {0};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const uint8_t* p0 = wlds + (16 * s + tr_row) * ABS_WSTRIDE + 64 * cb + tr_col_b;
        i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p0));
        i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(p0 + 4 * ABS_WSTRIDE));
        struct { i16x4 lo, hi; } pr = {v0, v1};
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, qa[s]),
                                                      __builtin_bit_cast(bf16x8, pr), acc, 0, 0, 0);
      }
      // C layout: lane l holds column 32cb + l%32 of rows 8(j/4) + 4g + j%4
#pragma unroll
      for (int j = 0; j < 16; ++j)
        *reinterpret_cast<float*>(stage + (8 * (j >> 2) + 4 * g + (j & 3)) * ABS_SSTRIDE + 4 * (32 * cb + (l & 31))) = acc[j];
    }
    __syncthreads();
    // 32 rows x (ABS_COLS / 8) runs of 8 columns: hi and lo as 16-byte stores
#pragma unroll
    for (int it = 0; it < 32 * (ABS_COLS / 8) / 256; ++it) {
      const int idx = tid + 256 * it, r = idx / (ABS_COLS / 8), k = idx % (ABS_COLS / 8);
      const int n = n0 + r;
      if (n < n_end) {
        const f32x4 v0 = *reinterpret_cast<const f32x4*>(stage + r * ABS_SSTRIDE + 32 * k);
        const f32x4 v1 = *reinterpret_cast<const f32x4*>(stage + r * ABS_SSTRIDE + 32 * k + 16);
        const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          hw[e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
          const float h0 = bf16_to_f32(static_cast<uint16_t>(hw[e] & 0xffffu));
          const float h1 = bf16_to_f32(static_cast<uint16_t>(hw[e] >> 16));
          lw[e] = pack_bf16x2(v[2 * e] - h0, v[2 * e + 1] - h1);
        }
        const int64_t o = (static_cast<int64_t>(n) * a.n_h + h) * ROWE + half_c * ABS_COLS + 8 * k;
        *reinterpret_cast<uint4*>(qout + o) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        if (qlo) *reinterpret_cast<uint4*>(qlo + o) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
      }
    }
    __syncthreads();  // stage reused by the next block
    if (n0 + 32 < n_end) {
#pragma unroll
      for (int s = 0; s < 8; ++s) qa[s] = qn[s];
    }
  }
}

// ------------------------------------------------------------------ launchers
hipError_t launch_append(const AppendArgs& a, int bf16, hipStream_t st) {
  if (a.n_tok <= 0) return hipSuccess;
  if (bf16)
    append_kernel<uint16_t><<<a.n_tok, 64, 0, st>>>(a);
  else
    append_kernel<float><<<a.n_tok, 64, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_rope_q(const RopeQArgs& a, int bf16, hipStream_t st) {
  if (a.n_q <= 0) return hipSuccess;
  if (bf16)
    rope_q_kernel<uint16_t><<<a.n_q, 256, 0, st>>>(a);
  else
    rope_q_kernel<float><<<a.n_q, 256, 0, st>>>(a);
  return hipGetLastError();
}

bool absorb_fuses_rope(int bf16, int d_c, int d_h, int d_r) {
  return bf16 && d_c == D_C && d_h == D_H && d_r == D_R;
}

hipError_t launch_absorb(const AbsorbArgs& a, int bf16, hipStream_t st) {
  if (a.n_q <= 0) return hipSuccess;
  if (absorb_fuses_rope(bf16, a.d_c, a.d_h, a.d_r)) {
    dim3 grid(a.n_h, ABS_PARTS, (a.n_q + ABS_QCHUNK - 1) / ABS_QCHUNK);
    absorb_mfma_kernel<<<grid, 256, 0, st>>>(a);
  } else if (bf16) {
    absorb_generic_kernel<uint16_t><<<dim3(a.n_q, a.n_h), 256, 0, st>>>(a);
  } else {
    absorb_generic_kernel<float><<<dim3(a.n_q, a.n_h), 256, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace mla
