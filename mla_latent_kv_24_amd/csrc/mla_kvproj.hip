// A1 from hidden states -- the cache row of a token made from its hidden
// state h (irregular6612 notes, section 2.1.2 and DeepSeek-V3 report,
// Metode 1: c^KV = W^DKV h, k^R = RoPE(W^KR h); jiphyeonjeon.kr review,
// section 2: the model normalises the compressed latent with an RMSNorm):
//   x = [W^DKV ; W^KR] h                          (d_c + d_hR = 576 outputs)
//   row = [ RMSNorm(x[0:d_c]) * weight ; RoPE(x[d_c:], pos) ]
// Two launches:
//   kvproj_partial_*: split-K partial sums of x, fp32 [slice][token][576];
//     the MFMA version (bf16, d_model a multiple of 128) computes a 64-token x
//     64-output tile per workgroup from 16-byte row loads of both operands
//     (the weights' rows and the hidden states are both k-contiguous), eight
//     k-steps per batch with the next batch's loads in flight;
//   kvproj_finalize_kernel: per token, one thread per output sums the slices
//     in a fixed order, the latent's mean square is reduced over the
//     workgroup, and the row is stored in the cache's dtype (RoPE angle in
//     fp64, rotation in fp32, as A1).
// Every output is summed in a fixed order: the rows are bitwise reproducible.
#include <algorithm>

#include "mla_common.h"

namespace mla {

constexpr int KP_TOK = 64;   // tokens per partial workgroup (MFMA path)
constexpr int KP_OUT = 64;   // outputs per partial workgroup: ROWE = 9 blocks
constexpr int KP_CHUNK = 8;  // MFMA k-steps (16 each) per load batch
static_assert(ROWE % KP_OUT == 0 && D_C % KP_OUT == 0, "output blocks must not straddle W^DKV / W^KR");

// ------------------------------------------------------------------------
// bf16 MFMA partials.  Grid (9 output blocks, token blocks, k slices).  Wave
// w owns outputs 32 (w >> 1) .. +31 and tokens 32 (w & 1) .. +31 of the
// workgroup's tile: A = weight rows (the lane's output row, k contiguous),
// B = hidden-state rows (the lane's token), v_mfma_f32_32x32x16_bf16.
// Lane l holds in register j the sum for output 8 (j/4) + 4 (l/32) + j%4 and
// token l%32 of its wave's tile.
// ------------------------------------------------------------------------
__global__ __launch_bounds__(256) void kvproj_partial_mfma_kernel(KvProjArgs a) {
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 5, l32 = l & 31;
  const int ob = blockIdx.x, tb = blockIdx.y, s = blockIdx.z;
  const int o = KP_OUT * ob + 32 * (w >> 1) + l32;
  const int t = KP_TOK * tb + 32 * (w & 1) + l32;
  const bool tv = t < a.n_tok;
  const int64_t dm = a.d_model;
  const uint16_t* wrow = (o < D_C) ? static_cast<const uint16_t*>(a.w_dkv) + o * dm
                                   : static_cast<const uint16_t*>(a.w_kr) + (o - D_C) * dm;
  // a lane past the last token reads the last token's row (its sums are not stored)
  const uint16_t* hrow = static_cast<const uint16_t*>(a.h) + (tv ? t : a.n_tok - 1) * dm;
  const int k0 = s * a.k_per_slice;
  const int k1 = min(k0 + a.k_per_slice, a.d_model);
  const int nchunks = (k1 - k0) / (16 * KP_CHUNK);   // both multiples of 128 (host plan)

  f32x16 acc;
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = 0.f;
  auto load = [&](int c, u32x4* av, u32x4* bv) {
    const int kb = k0 + 16 * KP_CHUNK * c + 8 * g;
#pragma unroll
    for (int i = 0; i < KP_CHUNK; ++i) {
      av[i] = *reinterpret_cast<const u32x4*>(wrow + kb + 16 * i);
      bv[i] = *reinterpret_cast<const u32x4*>(hrow + kb + 16 * i);
    }
  };
  auto mfmas = [&](const u32x4* av, const u32x4* bv) {
#pragma unroll
    for (int i = 0; i < KP_CHUNK; ++i)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[i]),
                                                    __builtin_bit_cast(bf16x8, bv[i]), acc, 0, 0, 0);
  };
  // two register batches in ping-pong: batch c + 1 is in flight while batch c
  // feeds the matrix cores (no register copies, so no full wait per batch)
  u32x4 a0[KP_CHUNK], b0[KP_CHUNK], a1[KP_CHUNK], b1[KP_CHUNK];
  if (nchunks > 0) load(0, a0, b0);
  for (int c = 0; c < nchunks; c += 2) {
    if (c + 1 < nchunks) load(c + 1, a1, b1);
    mfmas(a0, b0);
    if (c + 2 < nchunks) load(c + 2, a0, b0);
    if (c + 1 < nchunks) mfmas(a1, b1);
  }
  if (!tv) return;
  float* dst = a.part + (static_cast<int64_t>(s) * a.n_tok + t) * ROWE + KP_OUT * ob + 32 * (w >> 1) + 4 * g;
#pragma unroll
  for (int jq = 0; jq < 4; ++jq) {
    const f32x4 v = {acc[4 * jq], acc[4 * jq + 1], acc[4 * jq + 2], acc[4 * jq + 3]};
    *reinterpret_cast<f32x4*>(dst + 8 * jq) = v;
  }
}

// ------------------------------------------------------------------------
// Generic partials (fp32 storage, or a d_model the MFMA tiling does not
// divide): grid (9 output blocks, tokens, k slices), one output per thread.
// ------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(64) void kvproj_partial_generic_kernel(KvProjArgs a) {
  const int o = KP_OUT * blockIdx.x + threadIdx.x;
  const int t = blockIdx.y, s = blockIdx.z;
  const int64_t dm = a.d_model;
  const T* wrow = (o < D_C) ? static_cast<const T*>(a.w_dkv) + o * dm : static_cast<const T*>(a.w_kr) + (o - D_C) * dm;
  const T* hrow = static_cast<const T*>(a.h) + t * dm;
  const int k0 = s * a.k_per_slice;
  const int k1 = min(k0 + a.k_per_slice, a.d_model);
  float acc = 0.f;
  for (int k = k0; k < k1; ++k) acc = fmaf(load_as_f32(wrow, k), load_as_f32(hrow, k), acc);
  a.part[(static_cast<int64_t>(s) * a.n_tok + t) * ROWE + o] = acc;
}

// ------------------------------------------------------------------------
// Finalize: one workgroup of 576 threads (9 waves) per token; thread o owns
// output o and has all its slice loads in flight together (batches of 16),
// summed in slice order.  Waves 0-7 hold the latent, wave 8 the RoPE key.
// ------------------------------------------------------------------------
constexpr int KF_BATCH = 16;
template <typename T>
__global__ __launch_bounds__(ROWE) void kvproj_finalize_kernel(KvProjArgs a) {
  __shared__ float kr[D_R];
  __shared__ float red[D_C / 64];
  const int t = blockIdx.x, o = threadIdx.x;
  const int S = a.k_slices;
  const int64_t ss = static_cast<int64_t>(a.n_tok) * ROWE;
  const float* p = a.part + static_cast<int64_t>(t) * ROWE + o;
  float v = 0.f;
  for (int s0 = 0; s0 < S; s0 += KF_BATCH) {
    float r[KF_BATCH];
#pragma unroll
    for (int i = 0; i < KF_BATCH; ++i) r[i] = (s0 + i < S) ? p[(s0 + i) * ss] : 0.f;
#pragma unroll
    for (int i = 0; i < KF_BATCH; ++i) v += r[i];
  }
  // mean square of the latent over waves 0-7
  float sq = (o < D_C) ? v * v : 0.f;
  for (int off = 32; off > 0; off >>= 1) sq += __shfl_xor(sq, off);
  if (o < D_C && (o & 63) == 0) red[o >> 6] = sq;
  if (o >= D_C) kr[o - D_C] = v;
  __syncthreads();
  T* dst = static_cast<T*>(a.cache) + a.row[t] * ROWE;
  if (o < D_C) {
    const float ms = (((red[0] + red[1]) + (red[2] + red[3])) + ((red[4] + red[5]) + (red[6] + red[7]))) /
                     static_cast<float>(D_C);
    const float inv = 1.0f / sqrtf(ms + a.eps);
    const T* nw = static_cast<const T*>(a.norm_w);
    const float wgt = nw ? load_as_f32(nw, o) : 1.f;
    dst[o] = store_from_f32<T>(v * inv * wgt);
  } else if (o < D_C + D_R / 2) {
    const int k = o - D_C;
    float y0, y1;
    rope_pair(kr[2 * k], kr[2 * k + 1], a.pos[t], a.rope.theta[k], y0, y1);
    dst[D_C + 2 * k] = store_from_f32<T>(y0);
    dst[D_C + 2 * k + 1] = store_from_f32<T>(y1);
  }
}

void kv_project_plan(int32_t n_tok, int32_t d_model, int32_t& k_slices, int32_t& k_per_slice) {
  // aim at ~256 partial workgroups, with slices of at least 128 k (one MFMA
  // load batch) and a multiple of 128
  const int64_t tiles = static_cast<int64_t>(ROWE / KP_OUT) * ((n_tok + KP_TOK - 1) / KP_TOK);
  int64_t s = (256 + tiles - 1) / tiles;
  s = std::max<int64_t>(1, std::min<int64_t>(s, std::max(1, d_model / 128)));
  int64_t kr = (d_model + s - 1) / s;
  kr = (kr + 127) / 128 * 128;
  k_per_slice = static_cast<int32_t>(kr);
  k_slices = static_cast<int32_t>((d_model + kr - 1) / kr);
}

hipError_t launch_kv_project_append(const KvProjArgs& a, int bf16, hipStream_t st) {
  if (a.n_tok <= 0) return hipSuccess;
  const bool mfma = bf16 && a.d_model % 128 == 0;
  if (mfma) {
    const dim3 grid(ROWE / KP_OUT, (a.n_tok + KP_TOK - 1) / KP_TOK, a.k_slices);
    kvproj_partial_mfma_kernel<<<grid, 256, 0, st>>>(a);
  } else {
    const dim3 grid(ROWE / KP_OUT, a.n_tok, a.k_slices);
    if (bf16)
      kvproj_partial_generic_kernel<uint16_t><<<grid, 64, 0, st>>>(a);
    else
      kvproj_partial_generic_kernel<float><<<grid, 64, 0, st>>>(a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (bf16)
    kvproj_finalize_kernel<uint16_t><<<a.n_tok, ROWE, 0, st>>>(a);
  else
    kvproj_finalize_kernel<float><<<a.n_tok, ROWE, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace mla
