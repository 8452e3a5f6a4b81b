// A1 from hidden states -- the cache row of a token made from its hidden
// state h (irregular6612 notes, section 2.1.2 and DeepSeek-V3 report,
// Metode 1: c^KV = W^DKV h, k^R = RoPE(W^KR h); jiphyeonjeon.kr review,
// section 2: the model normalises the compressed latent with an RMSNorm):
//   x = [W^DKV ; W^KR] h                          (d_c + d_hR = 576 outputs)
//   row = [ RMSNorm(x[0:d_c]) * weight ; RoPE(x[d_c:], pos) ]
// Two launches:
//   the split-K partial sums of x, fp32 [slice][token][576], by the shared
//     projection kernels (mla_gemm.hip; from 256 tokens on, the LDS-tiled
//     product of mla_gemm_lds.hip);
//   kvproj_finalize_kernel: per token, one thread per output sums the slices
//     in a fixed order, the latent's mean square is reduced over the
//     workgroup, and the row is stored in the cache's dtype (RoPE angle in
//     fp64, rotation in fp32, as A1).
// Every output is summed in a fixed order: the rows are bitwise reproducible.
#include "mla_common.h"

namespace mla {

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

// bf16 chunks of 256 tokens or more take the LDS-tiled product (three
// 192-output tiles per 256 tokens, split K for about one round of the CUs);
// fewer tokens, or fp32, the weight-streaming and generic kernels.
void kv_project_plan(int32_t n_tok, int32_t d_model, int bf16, int32_t& k_slices, int32_t& k_per_slice) {
  if (bf16 && gemm_lds_applies(n_tok, d_model, ROWE))
    gemm_lds_plan(n_tok, d_model, ROWE, k_slices, k_per_slice);
  else
    gemm_plan(n_tok, d_model, ROWE, D_C, k_slices, k_per_slice);
}

hipError_t launch_kv_project_append(const KvProjArgs& a, int bf16, hipStream_t st) {
  if (a.n_tok <= 0) return hipSuccess;
  GemmArgs g{};
  g.x = a.h;
  g.w0 = a.w_dkv;
  g.w1 = a.w_kr;
  g.part = a.part;
  g.n = a.n_tok;
  g.d_in = a.d_model;
  g.d_out = ROWE;
  g.split = D_C;
  g.k_slices = a.k_slices;
  g.k_per_slice = a.k_per_slice;
  hipError_t e = (bf16 && gemm_lds_applies(a.n_tok, a.d_model, ROWE)) ? launch_gemm_lds_partial(g, st)
                                                                        : launch_gemm_partial(g, bf16, st);
  if (e != hipSuccess) return e;
  if (bf16)
    kvproj_finalize_kernel<uint16_t><<<a.n_tok, ROWE, 0, st>>>(a);
  else
    kvproj_finalize_kernel<float><<<a.n_tok, ROWE, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace mla
