// The projections around the attention, as one split-K product
//   y[t][o] = sum_k x[t][k] W[o][k],   W = [w0 ; w1] (rows stacked),
// where x holds tokens' activations (hidden states, the query latent, the
// heads' outputs) and W a projection in nn-linear layout ([out][in]):
//   [W^DKV ; W^KR] h   (cache rows from hidden states; irregular6612 notes,
//                       section 2.1.2, DeepSeek-V3 report, Metode 1),
//   W^DQ h, [W^UQ ; W^QR] c^Q   (the query path; jiphyeonjeon.kr review,
//                       section 2: queries pass through a 1,536-wide latent),
//   W^O o              (the output projection; review section 2,
//                       u_t = sum_i O_i U^V_i sum_j a_ij c_j).
// gemm_partial_mfma_kernel (bf16, d_in a multiple of 128): a workgroup
// computes a 64-token x 64-output tile over one k slice from 16-byte row loads
// of both operands (both k-contiguous) with v_mfma_f32_32x32x16_bf16, eight
// k-steps per register batch and two batches in ping-pong (one loads while the
// other feeds the matrix cores).  Tiles never straddle w0 / w1 (split is a
// multiple of 64).  Sums leave as fp32 partials, or as bf16 when one slice
// covers k.  Generic VALU kernels cover fp32 storage and other shapes.
#include <algorithm>

#include "mla_common.h"

namespace mla {

constexpr int G_TOK = 64;   // tokens per workgroup
constexpr int G_OUT = 64;   // outputs per workgroup
constexpr int G_CHUNK = 8;  // MFMA k-steps (16 each) per load batch

// Wave w owns outputs 32 (w >> 1) .. +31 and tokens 32 (w & 1) .. +31 of the
// tile: A = weight rows (the lane's output row), B = activation rows (the
// lane's token).  Lane l holds in register j the sum for output
// 8 (j/4) + 4 (l/32) + j%4 and token l%32 of its wave's tile.
__global__ __launch_bounds__(256) void gemm_partial_mfma_kernel(GemmArgs a) {
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 5, l32 = l & 31;
  const int ob = blockIdx.x, tb = blockIdx.y, s = blockIdx.z;
  const int o = G_OUT * ob + 32 * (w >> 1) + l32;
  const int t = G_TOK * tb + 32 * (w & 1) + l32;
  const bool tv = t < a.n;
  const int64_t dk = a.d_in;
  const uint16_t* wrow = (o < a.split) ? static_cast<const uint16_t*>(a.w0) + o * dk
                                       : static_cast<const uint16_t*>(a.w1) + (o - a.split) * dk;
  // a lane past the last token reads the last token's row (its sums are not stored)
  const uint16_t* xrow = static_cast<const uint16_t*>(a.x) + static_cast<int64_t>(tv ? t : a.n - 1) * dk;
  const int k0 = s * a.k_per_slice;
  const int k1 = min(k0 + a.k_per_slice, a.d_in);
  const int nchunks = (k1 - k0) / (16 * G_CHUNK);   // both multiples of 128 (host plan)

  f32x16 acc;
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = 0.f;
  auto load = [&](int c, u32x4* av, u32x4* bv) {
    const int kb = k0 + 16 * G_CHUNK * c + 8 * g;
#pragma unroll
    for (int i = 0; i < G_CHUNK; ++i) {
      av[i] = *reinterpret_cast<const u32x4*>(wrow + kb + 16 * i);
      bv[i] = *reinterpret_cast<const u32x4*>(xrow + kb + 16 * i);
    }
  };
  auto mfmas = [&](const u32x4* av, const u32x4* bv) {
#pragma unroll
    for (int i = 0; i < G_CHUNK; ++i)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[i]),
                                                    __builtin_bit_cast(bf16x8, bv[i]), acc, 0, 0, 0);
  };
  u32x4 a0[G_CHUNK], b0[G_CHUNK], a1[G_CHUNK], b1[G_CHUNK];
  if (nchunks > 0) load(0, a0, b0);
  for (int c = 0; c < nchunks; c += 2) {
    if (c + 1 < nchunks) load(c + 1, a1, b1);
    mfmas(a0, b0);
    if (c + 2 < nchunks) load(c + 2, a0, b0);
    if (c + 1 < nchunks) mfmas(a1, b1);
  }
  if (!tv) return;
  const int obase = G_OUT * ob + 32 * (w >> 1) + 4 * g;   // + 8 jq: four consecutive outputs
  if (a.out0) {
    // one slice: straight to out0 / out1 (a tile lies on one side of split)
    if (obase >= a.split && a.out1_f32) {
      float* df = a.out1_f32 + static_cast<int64_t>(t) * (a.d_out - a.split) + (obase - a.split);
#pragma unroll
      for (int jq = 0; jq < 4; ++jq)
        *reinterpret_cast<f32x4*>(df + 8 * jq) = f32x4{acc[4 * jq], acc[4 * jq + 1], acc[4 * jq + 2], acc[4 * jq + 3]};
      return;
    }
    uint16_t* dst = (obase < a.split) ? a.out0 + static_cast<int64_t>(t) * a.split + obase
                                      : a.out1 + static_cast<int64_t>(t) * (a.d_out - a.split) + (obase - a.split);
#pragma unroll
    for (int jq = 0; jq < 4; ++jq)
      *reinterpret_cast<uint2*>(dst + 8 * jq) =
          make_uint2(pack_bf16x2(acc[4 * jq], acc[4 * jq + 1]), pack_bf16x2(acc[4 * jq + 2], acc[4 * jq + 3]));
    return;
  }
  float* dst = a.part + (static_cast<int64_t>(s) * a.n + t) * a.d_out + obase;
#pragma unroll
  for (int jq = 0; jq < 4; ++jq) {
    const f32x4 v = {acc[4 * jq], acc[4 * jq + 1], acc[4 * jq + 2], acc[4 * jq + 3]};
    *reinterpret_cast<f32x4*>(dst + 8 * jq) = v;
  }
}

// ------------------------------------------------------------------------
// Few tokens (n <= 64, the decode step): the product streams the weights, so
// a workgroup takes 256 outputs (wave w: 64 rows, as two 32-row MFMA tiles)
// against all tokens (two 32-token tiles): every weight row is loaded once,
// by its wave, into registers (two 128-deep batches in ping-pong), and the
// activation chunk [64 tokens][128 k] is loaded once per workgroup into a
// double-buffered LDS tile (16-B chunk kc of token row t at kc ^ (t & 15))
// that all four waves read as the B operand.
// ------------------------------------------------------------------------
constexpr int S_OUT = 256;
constexpr int S_XBYTES = 64 * 128 * 2;   // one activation chunk in LDS

__global__ __launch_bounds__(256, 2) void gemm_stream_mfma_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t xs[2 * S_XBYTES];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 5, l32 = l & 31;
  const int ob = blockIdx.x, s = blockIdx.z;
  const int o0 = S_OUT * ob + 64 * w;   // the wave's 64 rows (one side of split)
  const int64_t dk = a.d_in;
  const uint16_t* wbase = (o0 < a.split) ? static_cast<const uint16_t*>(a.w0) + static_cast<int64_t>(o0) * dk
                                         : static_cast<const uint16_t*>(a.w1) + static_cast<int64_t>(o0 - a.split) * dk;
  const uint16_t* wr0 = wbase + static_cast<int64_t>(l32) * dk + 8 * g;         // rows o0 + l32
  const uint16_t* wr1 = wbase + static_cast<int64_t>(32 + l32) * dk + 8 * g;    // rows o0 + 32 + l32
  const int k0 = s * a.k_per_slice;
  const int k1 = min(k0 + a.k_per_slice, a.d_in);
  const int nchunks = (k1 - k0) / 128;

  // activation chunk loads: thread tid moves 16-B chunks f = tid + 256 i: token
  // t = f / 16, k-chunk kc = f % 16 (tokens past n load zeros)
  const uint16_t* xg = static_cast<const uint16_t*>(a.x);
  auto xload = [&](int c, u32x4* xv) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int f = tid + 256 * i, t = f >> 4, kc = f & 15;
      xv[i] = (t < a.n) ? *reinterpret_cast<const u32x4*>(xg + static_cast<int64_t>(t) * dk + k0 + 128 * c + 8 * kc)
                        : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto xstore = [&](int buf, const u32x4* xv) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int f = tid + 256 * i, t = f >> 4, kc = f & 15;
      *reinterpret_cast<u32x4*>(xs + buf * S_XBYTES + 256 * t + 16 * (kc ^ (t & 15))) = xv[i];
    }
  };
  auto wload = [&](int c, u32x4* av) {
    const int kb = k0 + 128 * c;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      av[i] = *reinterpret_cast<const u32x4*>(wr0 + kb + 16 * i);
      av[8 + i] = *reinterpret_cast<const u32x4*>(wr1 + kb + 16 * i);
    }
  };
  f32x16 acc[2][2];   // [row tile u][token tile tt]
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[u][tt][j] = 0.f;
  auto mfmas = [&](int buf, const u32x4* av) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      u32x4 bv[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int t = 32 * tt + l32;
        bv[tt] = *reinterpret_cast<const u32x4*>(xs + buf * S_XBYTES + 256 * t + 16 * ((2 * i + g) ^ (t & 15)));
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
          acc[u][tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[8 * u + i]),
                                                               __builtin_bit_cast(bf16x8, bv[tt]), acc[u][tt], 0, 0, 0);
    }
  };

  u32x4 wa[16], wb[16], xv[4];
  if (nchunks > 0) {
    xload(0, xv);
    wload(0, wa);
    xstore(0, xv);
  }
  __syncthreads();
  for (int c = 0; c < nchunks; c += 2) {
    // chunk c from (wa, LDS buffer 0); chunk c + 1's loads in flight meanwhile
    if (c + 1 < nchunks) {
      xload(c + 1, xv);
      wload(c + 1, wb);
    }
    mfmas(0, wa);
    if (c + 1 < nchunks) xstore(1, xv);
    __syncthreads();   // buffer 1 written; every wave done with buffer 0
    if (c + 1 < nchunks) {
      if (c + 2 < nchunks) {
        xload(c + 2, xv);
        wload(c + 2, wa);
      }
      mfmas(1, wb);
      if (c + 2 < nchunks) xstore(0, xv);
      __syncthreads();
    }
  }

  // ---- results: lane holds output o0 + 32 u + 8 (j/4) + 4 g + j%4, token 32 tt + l32
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int t = 32 * tt + l32;
    if (t >= a.n) continue;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int obase = o0 + 32 * u + 4 * g;
      const f32x16& v = acc[u][tt];
      if (a.out0) {
        if (obase >= a.split && a.out1_f32) {
          float* df = a.out1_f32 + static_cast<int64_t>(t) * (a.d_out - a.split) + (obase - a.split);
#pragma unroll
          for (int jq = 0; jq < 4; ++jq)
            *reinterpret_cast<f32x4*>(df + 8 * jq) = f32x4{v[4 * jq], v[4 * jq + 1], v[4 * jq + 2], v[4 * jq + 3]};
        } else {
          uint16_t* dst = (obase < a.split) ? a.out0 + static_cast<int64_t>(t) * a.split + obase
                                            : a.out1 + static_cast<int64_t>(t) * (a.d_out - a.split) + (obase - a.split);
#pragma unroll
          for (int jq = 0; jq < 4; ++jq)
            *reinterpret_cast<uint2*>(dst + 8 * jq) =
                make_uint2(pack_bf16x2(v[4 * jq], v[4 * jq + 1]), pack_bf16x2(v[4 * jq + 2], v[4 * jq + 3]));
        }
      } else {
        float* dst = a.part + (static_cast<int64_t>(s) * a.n + t) * a.d_out + obase;
#pragma unroll
        for (int jq = 0; jq < 4; ++jq)
          *reinterpret_cast<f32x4*>(dst + 8 * jq) = f32x4{v[4 * jq], v[4 * jq + 1], v[4 * jq + 2], v[4 * jq + 3]};
      }
    }
  }
}

static bool use_stream(int32_t n, int32_t d_in, int32_t d_out, int32_t split) {
  return n <= 64 && d_in % 128 == 0 && d_out % S_OUT == 0 && split % S_OUT == 0;
}

// Generic partials: grid (ceil(d_out / 64), tokens, k slices), one output per thread.
template <typename T>
__global__ __launch_bounds__(64) void gemm_partial_generic_kernel(GemmArgs a) {
  const int o = G_OUT * blockIdx.x + threadIdx.x;
  const int t = blockIdx.y, s = blockIdx.z;
  if (o >= a.d_out) return;
  const int64_t dk = a.d_in;
  const T* wrow = (o < a.split) ? static_cast<const T*>(a.w0) + o * dk : static_cast<const T*>(a.w1) + (o - a.split) * dk;
  const T* xrow = static_cast<const T*>(a.x) + t * dk;
  const int k0 = s * a.k_per_slice;
  const int k1 = min(k0 + a.k_per_slice, a.d_in);
  float acc = 0.f;
  for (int k = k0; k < k1; ++k) acc = fmaf(load_as_f32(wrow, k), load_as_f32(xrow, k), acc);
  if (a.out0) {
    if (o < a.split)
      a.out0[static_cast<int64_t>(t) * a.split + o] = f32_to_bf16(acc);
    else if (a.out1_f32)
      a.out1_f32[static_cast<int64_t>(t) * (a.d_out - a.split) + (o - a.split)] = acc;
    else
      a.out1[static_cast<int64_t>(t) * (a.d_out - a.split) + (o - a.split)] = f32_to_bf16(acc);
    return;
  }
  a.part[(static_cast<int64_t>(s) * a.n + t) * a.d_out + o] = acc;
}

// Split-K plan (slices of at least one 128-deep batch): the streaming kernel
// aims at one round of 256 workgroups; the tile kernel at four workgroups per
// CU, since each of its waves has about one load batch in flight.
void gemm_plan(int32_t n, int32_t d_in, int32_t d_out, int32_t split, int32_t& k_slices, int32_t& k_per_slice) {
  const bool stream = use_stream(n, d_in, d_out, split);
  const int64_t tiles = stream ? d_out / S_OUT
                               : static_cast<int64_t>((d_out + G_OUT - 1) / G_OUT) * ((n + G_TOK - 1) / G_TOK);
  int64_t s = ((stream ? 256 : 1024) + tiles - 1) / tiles;
  // the fp32 partials (n d_out 4 B per slice) stay within half the bytes the
  // product moves anyway (weights and activations)
  const int64_t cap = static_cast<int64_t>(d_in) * (d_out + n) / (4 * static_cast<int64_t>(std::max(n, 1)) * d_out);
  s = std::min(s, std::max<int64_t>(1, cap));
  s = std::max<int64_t>(1, std::min<int64_t>(s, std::max(1, d_in / 128)));
  int64_t kr = (d_in + s - 1) / s;
  kr = (kr + 127) / 128 * 128;
  k_per_slice = static_cast<int32_t>(kr);
  k_slices = static_cast<int32_t>((d_in + kr - 1) / kr);
}

hipError_t launch_gemm_partial(const GemmArgs& a, int bf16, hipStream_t st) {
  if (a.n <= 0 || a.d_out <= 0) return hipSuccess;
  const bool mfma = bf16 && a.d_in % 128 == 0 && a.d_out % G_OUT == 0 && a.split % G_OUT == 0;
  if (bf16 && use_stream(a.n, a.d_in, a.d_out, a.split)) {
    gemm_stream_mfma_kernel<<<dim3(a.d_out / S_OUT, 1, a.k_slices), 256, 0, st>>>(a);
  } else if (mfma) {
    const dim3 grid(a.d_out / G_OUT, (a.n + G_TOK - 1) / G_TOK, a.k_slices);
    gemm_partial_mfma_kernel<<<grid, 256, 0, st>>>(a);
  } else {
    const dim3 grid((a.d_out + G_OUT - 1) / G_OUT, a.n, a.k_slices);
    if (bf16)
      gemm_partial_generic_kernel<uint16_t><<<grid, 64, 0, st>>>(a);
    else
      gemm_partial_generic_kernel<float><<<grid, 64, 0, st>>>(a);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------------
// Slice sums and the row epilogues
// ------------------------------------------------------------------------
__global__ __launch_bounds__(256) void sum_slices_kernel(const float* part, int32_t slices, int64_t n_elems, float* out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n_elems) return;
  float v = 0.f;
  for (int s = 0; s < slices; ++s) v += part[s * n_elems + i];
  out[i] = v;
}

// Slice sums of [n][d_out] partials to two outputs: columns < split as bf16
// rows of out0 [n][split], the rest as fp32 rows of out1 [n][d_out - split].
__global__ __launch_bounds__(256) void slices_to_outputs_kernel(const float* part, int32_t slices, int32_t n,
                                                                int32_t d_out, int32_t split, uint16_t* out0,
                                                                float* out1) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t n_elems = static_cast<int64_t>(n) * d_out;
  if (i >= n_elems) return;
  float v = 0.f;
  for (int s = 0; s < slices; ++s) v += part[s * n_elems + i];
  const int64_t t = i / d_out;
  const int o = static_cast<int>(i - t * d_out);
  if (o < split)
    out0[t * split + o] = f32_to_bf16(v);
  else
    out1[t * (d_out - split) + (o - split)] = v;
}

hipError_t launch_slices_to_outputs(const float* part, int32_t slices, int32_t n, int32_t d_out, int32_t split,
                                    uint16_t* out0, float* out1, hipStream_t st) {
  const int64_t n_elems = static_cast<int64_t>(n) * d_out;
  if (n_elems <= 0) return hipSuccess;
  slices_to_outputs_kernel<<<static_cast<unsigned>((n_elems + 255) / 256), 256, 0, st>>>(part, slices, n, d_out, split,
                                                                                        out0, out1);
  return hipGetLastError();
}

hipError_t launch_sum_slices(const float* part, int32_t slices, int64_t n_elems, float* out, hipStream_t st) {
  if (n_elems <= 0) return hipSuccess;
  sum_slices_kernel<<<static_cast<unsigned>((n_elems + 255) / 256), 256, 0, st>>>(part, slices, n_elems, out);
  return hipGetLastError();
}

// One workgroup per row: the slices summed in order, the mean square reduced
// over the workgroup, the row normalised, weighted (bf16 weight or none) and
// stored as bf16.  d <= 256 * RN_PER.
constexpr int RN_PER = 16;
__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(const float* part, int32_t slices, int32_t n, int32_t d,
                                                           const uint16_t* weight, float eps, uint16_t* out) {
  __shared__ float red[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  const int64_t ss = static_cast<int64_t>(n) * d;
  float v[RN_PER];
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < RN_PER; ++i) {
    const int o = tid + 256 * i;
    float x = 0.f;
    if (o < d) {
      const float* p = part + static_cast<int64_t>(t) * d + o;
      for (int s0 = 0; s0 < slices; s0 += 8) {   // eight slice loads in flight, summed in order
        float r[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) r[j] = (s0 + j < slices) ? p[(s0 + j) * ss] : 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) x += r[j];
      }
    }
    v[i] = x;
    sq = fmaf(x, x, sq);
  }
  for (int off = 32; off > 0; off >>= 1) sq += __shfl_xor(sq, off);
  if ((tid & 63) == 0) red[tid >> 6] = sq;
  __syncthreads();
  const float ms = ((red[0] + red[1]) + (red[2] + red[3])) / static_cast<float>(d);
  const float inv = 1.0f / sqrtf(ms + eps);
#pragma unroll
  for (int i = 0; i < RN_PER; ++i) {
    const int o = tid + 256 * i;
    if (o < d) out[static_cast<int64_t>(t) * d + o] = f32_to_bf16(v[i] * inv * (weight ? bf16_to_f32(weight[o]) : 1.f));
  }
}

hipError_t launch_rmsnorm_rows(const float* part, int32_t slices, int32_t n, int32_t d, const void* weight, float eps,
                               uint16_t* out, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (d > 256 * RN_PER) return hipErrorInvalidValue;
  rmsnorm_rows_kernel<<<n, 256, 0, st>>>(part, slices, n, d, static_cast<const uint16_t*>(weight), eps, out);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void to_bf16_kernel(const float* in, int64_t n_elems, uint16_t* out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n_elems) out[i] = f32_to_bf16(in[i]);
}

hipError_t launch_to_bf16(const float* in, int64_t n_elems, uint16_t* out, hipStream_t st) {
  if (n_elems <= 0) return hipSuccess;
  to_bf16_kernel<<<static_cast<unsigned>((n_elems + 255) / 256), 256, 0, st>>>(in, n_elems, out);
  return hipGetLastError();
}

}  // namespace mla
