// A1 (cache append with decoupled RoPE key) and A2 (absorbed query) for gfx950.
//
// A1 writes row = [c^KV ; RoPE(k_raw, pos)] (jiphyeonjeon.kr DeepSeek-V2 review,
// section 3: one 64-d RoPE key per token shared by all heads; DeepSeek-V3 report
// on xyznot.com, Metode 1: only c^KV and k^R are cached).
// A2 folds U^K_i into the query, q~_i = (U^K_i)^T q^C_i (review section 2), and
// rotates the per-head RoPE query by the token position (review section 3).
// Both are formed in fp32 and written in the absorbed query layout: fp32 for
// fp32 storage, a bf16 hi/lo pair (the matrix-core operand format) for bf16.
#include "mla_common.h"

namespace mla {

// ----------------------------------------------------------------- RoPE pair
// Interleaved pair (x0, x1) rotated by angle pos * theta: the angle and its
// sine/cosine in fp64, the rotation itself in fp32.
__device__ __forceinline__ void rope_pair(float x0, float x1, int32_t pos, double theta,
                                          float& y0, float& y1) {
  double s, c;
  sincos(static_cast<double>(pos) * theta, &s, &c);
  const float cf = static_cast<float>(c), sf = static_cast<float>(s);
  y0 = x0 * cf - x1 * sf;
  y1 = x0 * sf + x1 * cf;
}

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
    store_q<T>(a.q_lat, nh, row_e, a.d_c + 2 * k, x0 * cs[k] - x1 * sn[k]);
    store_q<T>(a.q_lat, nh, row_e, a.d_c + 2 * k + 1, x0 * sn[k] + x1 * cs[k]);
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
    store_q<T>(a.q_lat, nh, a.d_c + a.d_r, c, acc);
  }
}

// ------------------------------------------- A2, latent part, bf16 MFMA path
// Per head i: q_lat[n, i, :] = q_c[n, i, :] @ w_uk[i]  ([n x 128] @ [128 x 512]).
// Grid (head, column half, query chunk of 256).  The workgroup stages its
// [128 d][256 c] slab of W^UK in LDS once (row stride 576 B keeps the four rows
// of a transpose read in distinct banks), then runs 32-query blocks through
// v_mfma_f32_32x32x16_bf16: A = q_c rows straight from global memory (d is
// contiguous), B = W^UK columns via ds_read_b64_tr_b16 (d is the LDS row index).
constexpr int ABS_QCHUNK = 256;
constexpr int ABS_WSTRIDE = 576;  // bytes per staged W row (256 bf16 + 64 B pad)

__global__ __launch_bounds__(256, 2) void absorb_mfma_kernel(AbsorbArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t wlds[D_H * ABS_WSTRIDE];
  const int h = blockIdx.x, half_c = blockIdx.y;
  const int n_begin = blockIdx.z * ABS_QCHUNK;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const uint16_t* wsrc = static_cast<const uint16_t*>(a.w_uk) +
                         static_cast<int64_t>(h) * D_H * D_C + half_c * 256;
  for (int f = tid; f < D_H * 32; f += 256) {  // 32 chunks of 16 B per row
    const int d = f >> 5, k = f & 31;
    *reinterpret_cast<uint4*>(wlds + d * ABS_WSTRIDE + 16 * k) =
        *reinterpret_cast<const uint4*>(wsrc + static_cast<int64_t>(d) * D_C + 8 * k);
  }
  __syncthreads();

  const int g = l >> 5;            // k-half of the 32x32x16 operand
  const int j16 = l & 15, hf = (l >> 4) & 1;
  // transpose-read address pieces: row d = 16s + 8g + (j16>>2) [+4], column 32cb + 16hf + 4(j16&3)
  const int tr_row = 8 * g + (j16 >> 2);
  const int tr_col_b = 2 * (16 * hf + 4 * (j16 & 3));
  const uint16_t* qc = static_cast<const uint16_t*>(a.q_c);
  const int row_e = a.d_c + a.d_r;

  for (int n0 = n_begin; n0 < min(n_begin + ABS_QCHUNK, a.n_q); n0 += 32) {
    const int n = n0 + (l & 31);
    uint4 qa[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      qa[s] = (n < a.n_q) ? *reinterpret_cast<const uint4*>(
                                qc + (static_cast<int64_t>(n) * a.n_h + h) * D_H + 16 * s + 8 * g)
                          : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int cbl = 0; cbl < 2; ++cbl) {
      const int cb = 2 * w + cbl;  // 32-column block inside this half
      f32x16 acc = {0};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const uint8_t* p0 = wlds + (16 * s + tr_row) * ABS_WSTRIDE + 64 * cb + tr_col_b;
        i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(p0));
        i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(p0 + 4 * ABS_WSTRIDE));
        struct { i16x4 lo, hi; } pr = {v0, v1};
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, qa[s]),
                                                      __builtin_bit_cast(bf16x8, pr), acc, 0, 0, 0);
      }
      const int c = half_c * 256 + 32 * cb + (l & 31);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int nn = n0 + 8 * (j >> 2) + 4 * g + (j & 3);
        if (nn < a.n_q) store_q<uint16_t>(a.q_lat, static_cast<int64_t>(nn) * a.n_h + h, row_e, c, acc[j]);
      }
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

hipError_t launch_absorb(const AbsorbArgs& a, int bf16, hipStream_t st) {
  if (a.n_q <= 0) return hipSuccess;
  if (bf16 && a.d_c == D_C && a.d_h == D_H) {
    dim3 grid(a.n_h, 2, (a.n_q + ABS_QCHUNK - 1) / ABS_QCHUNK);
    absorb_mfma_kernel<<<grid, 256, 0, st>>>(a);
  } else if (bf16) {
    absorb_generic_kernel<uint16_t><<<dim3(a.n_q, a.n_h), 256, 0, st>>>(a);
  } else {
    absorb_generic_kernel<float><<<dim3(a.n_q, a.n_h), 256, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace mla
