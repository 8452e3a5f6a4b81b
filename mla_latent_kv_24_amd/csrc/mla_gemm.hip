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
// a workgroup takes 128 RT outputs (wave w: 32 RT rows, as RT 32-row MFMA
// tiles) against all tokens (two 32-token tiles): every weight row is loaded
// once, by its wave, into registers (two 128-deep batches in ping-pong), and
// the activation chunk [64 tokens][128 k] is loaded once per workgroup into a
// double-buffered LDS tile (16-B chunk kc of token row t at kc ^ (t & 15))
// that all four waves read as the B operand.  RT = 2 halves the activation
// traffic per weight byte; RT = 1 doubles the workgroups for narrow products.
// ------------------------------------------------------------------------
constexpr int S_XBYTES = 64 * 128 * 2;   // one activation chunk in LDS

template <int RT>
__global__ __launch_bounds__(256, 2) void gemm_stream_mfma_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t xs[2 * S_XBYTES];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 5, l32 = l & 31;
  const int ob = blockIdx.x, s = blockIdx.z;
  const int o0 = 128 * RT * ob + 32 * RT * w;   // the wave's 32 RT rows (one side of split)
  const int64_t dk = a.d_in;
  const uint16_t* wbase = (o0 < a.split) ? static_cast<const uint16_t*>(a.w0) + static_cast<int64_t>(o0) * dk
                                         : static_cast<const uint16_t*>(a.w1) + static_cast<int64_t>(o0 - a.split) * dk;
  const uint16_t* wr0 = wbase + static_cast<int64_t>(l32) * dk + 8 * g;         // rows o0 + l32
  const uint16_t* wr1 = wbase + static_cast<int64_t>(32 + l32) * dk + 8 * g;    // rows o0 + 32 + l32 (RT = 2)
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
      if (RT == 2) av[8 + i] = *reinterpret_cast<const u32x4*>(wr1 + kb + 16 * i);
    }
  };
  f32x16 acc[RT][2];   // [row tile u][token tile tt]
#pragma unroll
  for (int u = 0; u < RT; ++u)
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
      for (int u = 0; u < RT; ++u)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
          acc[u][tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[8 * u + i]),
                                                               __builtin_bit_cast(bf16x8, bv[tt]), acc[u][tt], 0, 0, 0);
    }
  };

  u32x4 wa[8 * RT], wb[8 * RT], xv[4];
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
    for (int u = 0; u < RT; ++u) {
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

constexpr int64_t kGemmCUs = 256;   // MI355X compute units (the plans are device independent)

// Split-K slices (each at least one 128-deep batch) for `tiles` output tiles:
// `want` slices, at most the cap that keeps the fp32 partials (n d_out 4 B per
// slice) within half the bytes the product moves anyway (weights and
// activations).
static void plan_slices(int32_t n, int32_t d_in, int32_t d_out, int64_t want, int32_t& k_slices,
                        int32_t& k_per_slice) {
  const int64_t cap = static_cast<int64_t>(d_in) * (d_out + n) / (4 * static_cast<int64_t>(std::max(n, 1)) * d_out);
  int64_t s = std::min(want, std::max<int64_t>(1, cap));
  s = std::max<int64_t>(1, std::min<int64_t>(s, std::max(1, d_in / 128)));
  int64_t kr = (d_in + s - 1) / s;
  kr = (kr + 127) / 128 * 128;
  k_per_slice = static_cast<int32_t>(kr);
  k_slices = static_cast<int32_t>((d_in + kr - 1) / kr);
}

// The streaming kernel's plan.  Its workgroups all move the same bytes, so the
// plan keeps them within one round of the 256 CUs (a few past 256 would double
// some CUs' share and set the time), and of the row-tile sizes takes the one
// with the most workgroups, then the fewer partial bytes (none for one
// slice), then RT = 2 (half the activation reads).  rt = 0: not applicable.
static void stream_plan(int32_t n, int32_t d_in, int32_t d_out, int32_t split, int& rt, int32_t& k_slices,
                        int32_t& k_per_slice) {
  rt = 0;
  int64_t best_wg = -1, best_part = 0;
  for (int r = 2; r >= 1; --r) {
    if (!(n <= 64 && d_in % 128 == 0 && d_out % (128 * r) == 0 && split % (128 * r) == 0)) continue;
    const int64_t tiles = d_out / (128 * r);
    int32_t S, kps;
    plan_slices(n, d_in, d_out, std::max<int64_t>(1, kGemmCUs / tiles), S, kps);
    const int64_t wg = std::min<int64_t>(tiles * S, kGemmCUs);
    const int64_t part = S > 1 ? static_cast<int64_t>(S) * n * d_out : 0;
    if (wg > best_wg || (wg == best_wg && part < best_part)) {
      best_wg = wg;
      best_part = part;
      rt = r;
      k_slices = S;
      k_per_slice = kps;
    }
  }
}

// Split-K plan: the streaming kernel as above; the tile kernel at four
// workgroups per CU, since each of its waves has about one load batch in flight.
void gemm_plan(int32_t n, int32_t d_in, int32_t d_out, int32_t split, int32_t& k_slices, int32_t& k_per_slice) {
  int rt;
  stream_plan(n, d_in, d_out, split, rt, k_slices, k_per_slice);
  if (rt > 0) return;
  const int64_t tiles = static_cast<int64_t>((d_out + G_OUT - 1) / G_OUT) * ((n + G_TOK - 1) / G_TOK);
  plan_slices(n, d_in, d_out, (4 * kGemmCUs + tiles - 1) / tiles, k_slices, k_per_slice);
}

hipError_t launch_gemm_partial(const GemmArgs& a, int bf16, hipStream_t st) {
  if (a.n <= 0 || a.d_out <= 0) return hipSuccess;
  const bool mfma = bf16 && a.d_in % 128 == 0 && a.d_out % G_OUT == 0 && a.split % G_OUT == 0;
  int rt = 0;
  if (bf16) {
    int32_t S, kps;
    stream_plan(a.n, a.d_in, a.d_out, a.split, rt, S, kps);
  }
  if (rt == 2) {
    gemm_stream_mfma_kernel<2><<<dim3(a.d_out / 256, 1, a.k_slices), 256, 0, st>>>(a);
  } else if (rt == 1) {
    gemm_stream_mfma_kernel<1><<<dim3(a.d_out / 128, 1, a.k_slices), 256, 0, st>>>(a);
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

// Four elements per thread (n_elems a multiple of 4, 16-B aligned arrays),
// the loads of SB slices in flight together; each element still sums its
// slices in order, so the result is the scalar kernel's bit for bit.
constexpr int SB = 4;
__device__ __forceinline__ f32x4 sum_slices4(const float* part, int32_t slices, int64_t n_elems, int64_t i) {
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < slices; s0 += SB) {
    f32x4 r[SB];
#pragma unroll
    for (int j = 0; j < SB; ++j)
      r[j] = (s0 + j < slices) ? *reinterpret_cast<const f32x4*>(part + (s0 + j) * n_elems + i)
                               : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < SB; ++j) v += r[j];
  }
  return v;
}

__global__ __launch_bounds__(256) void sum_slices4_kernel(const float* part, int32_t slices, int64_t n_elems,
                                                          float* out) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i >= n_elems) return;
  *reinterpret_cast<f32x4*>(out + i) = sum_slices4(part, slices, n_elems, i);
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

// Four elements per thread: d_out and split multiples of 4, 16-B aligned arrays.
__global__ __launch_bounds__(256) void slices_to_outputs4_kernel(const float* part, int32_t slices, int32_t n,
                                                                 int32_t d_out, int32_t split, uint16_t* out0,
                                                                 float* out1) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  const int64_t n_elems = static_cast<int64_t>(n) * d_out;
  if (i >= n_elems) return;
  const f32x4 v = sum_slices4(part, slices, n_elems, i);
  const int64_t t = i / d_out;
  const int o = static_cast<int>(i - t * d_out);
  if (o < split)
    *reinterpret_cast<uint2*>(out0 + t * split + o) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
  else
    *reinterpret_cast<f32x4*>(out1 + t * (d_out - split) + (o - split)) = v;
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

hipError_t launch_slices_to_outputs(const float* part, int32_t slices, int32_t n, int32_t d_out, int32_t split,
                                    uint16_t* out0, float* out1, hipStream_t st) {
  const int64_t n_elems = static_cast<int64_t>(n) * d_out;
  if (n_elems <= 0) return hipSuccess;
  if (d_out % 4 == 0 && split % 4 == 0 && aligned16(part) && (reinterpret_cast<uintptr_t>(out0) & 7) == 0 &&
      aligned16(out1))
    slices_to_outputs4_kernel<<<static_cast<unsigned>((n_elems / 4 + 255) / 256), 256, 0, st>>>(
        part, slices, n, d_out, split, out0, out1);
  else
    slices_to_outputs_kernel<<<static_cast<unsigned>((n_elems + 255) / 256), 256, 0, st>>>(part, slices, n, d_out,
                                                                                          split, out0, out1);
  return hipGetLastError();
}

hipError_t launch_sum_slices(const float* part, int32_t slices, int64_t n_elems, float* out, hipStream_t st) {
  if (n_elems <= 0) return hipSuccess;
  if (n_elems % 4 == 0 && aligned16(part) && aligned16(out))
    sum_slices4_kernel<<<static_cast<unsigned>((n_elems / 4 + 255) / 256), 256, 0, st>>>(part, slices, n_elems, out);
  else
    sum_slices_kernel<<<static_cast<unsigned>((n_elems + 255) / 256), 256, 0, st>>>(part, slices, n_elems, out);
  return hipGetLastError();
}

// One workgroup per row: the slices summed in order, the mean square reduced
// over the workgroup, the row normalised, weighted (bf16 weight or none) and
// stored as bf16.  d <= 256 * RN_PER.  A thread's loads of RN_SB slices of all
// its columns are in flight together.
constexpr int RN_PER = 16;
constexpr int RN_SB = 8;
__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(const float* part, int32_t slices, int32_t n, int32_t d,
                                                           const uint16_t* weight, float eps, uint16_t* out) {
  __shared__ float red[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  const int64_t ss = static_cast<int64_t>(n) * d;
  const float* p = part + static_cast<int64_t>(t) * d + tid;
  float v[RN_PER];
#pragma unroll
  for (int i = 0; i < RN_PER; ++i) v[i] = 0.f;
  for (int s0 = 0; s0 < slices; s0 += RN_SB) {
    float r[RN_SB][RN_PER];
#pragma unroll
    for (int j = 0; j < RN_SB; ++j)
#pragma unroll
      for (int i = 0; i < RN_PER; ++i)
        r[j][i] = (tid + 256 * i < d && s0 + j < slices) ? p[(s0 + j) * ss + 256 * i] : 0.f;
#pragma unroll
    for (int j = 0; j < RN_SB; ++j)
#pragma unroll
      for (int i = 0; i < RN_PER; ++i) v[i] += r[j][i];   // each column in slice order
  }
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < RN_PER; ++i) sq = fmaf(v[i], v[i], sq);
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

// Two passes for several slices and d a multiple of 256, so that the slice
// loads spread over n * d / 256 workgroups instead of n:
//   rowsum_kernel, per (row t, 256-column chunk c): one thread per column sums
//     the slices in order (all loads in flight) and writes the sum over slice
//     0's element, which only it reads; the chunk's sum of squares goes to
//     slice 1's element (t, 256 c), which only this workgroup reads, after
//     every thread of it has read its slices;
//   rownorm_kernel, per row: the chunks' sums of squares in chunk order, then
//     the row normalised, weighted and stored as bf16.
constexpr int RS_BATCH = 16;
__global__ __launch_bounds__(256) void rowsum_kernel(float* part, int32_t slices, int32_t n, int32_t d) {
  __shared__ float red[4];
  const int t = blockIdx.x, c = blockIdx.y, tid = threadIdx.x;
  const int64_t ss = static_cast<int64_t>(n) * d;
  float* p = part + static_cast<int64_t>(t) * d + 256 * c + tid;
  float v = 0.f;
  for (int s0 = 0; s0 < slices; s0 += RS_BATCH) {
    float r[RS_BATCH];
#pragma unroll
    for (int j = 0; j < RS_BATCH; ++j) r[j] = (s0 + j < slices) ? p[(s0 + j) * ss] : 0.f;
#pragma unroll
    for (int j = 0; j < RS_BATCH; ++j) v += r[j];
  }
  float sq = v * v;
  for (int off = 32; off > 0; off >>= 1) sq += __shfl_xor(sq, off);
  if ((tid & 63) == 0) red[tid >> 6] = sq;
  __syncthreads();   // every thread has read its slices
  p[0] = v;
  if (tid == 0) p[ss] = (red[0] + red[1]) + (red[2] + red[3]);
}

__global__ __launch_bounds__(256) void rownorm_kernel(const float* part, int32_t n, int32_t d, const uint16_t* weight,
                                                      float eps, uint16_t* out) {
  const int t = blockIdx.x, tid = threadIdx.x;
  const int64_t ss = static_cast<int64_t>(n) * d;
  const float* row = part + static_cast<int64_t>(t) * d;
  const int chunks = d / 256;   // <= RN_PER
  float cs[RN_PER], x[RN_PER], wv[RN_PER];  // every load in flight together
#pragma unroll
  for (int c = 0; c < RN_PER; ++c) cs[c] = (c < chunks) ? row[ss + 256 * c] : 0.f;
#pragma unroll
  for (int i = 0; i < RN_PER; ++i) {
    x[i] = (i < chunks) ? row[tid + 256 * i] : 0.f;
    wv[i] = (i < chunks && weight) ? bf16_to_f32(weight[tid + 256 * i]) : 1.f;
  }
  float sq = 0.f;
#pragma unroll
  for (int c = 0; c < RN_PER; ++c) sq += cs[c];   // chunk order
  const float inv = 1.0f / sqrtf(sq / static_cast<float>(d) + eps);
#pragma unroll
  for (int i = 0; i < RN_PER; ++i) {
    const int o = tid + 256 * i;
    if (i < chunks) out[static_cast<int64_t>(t) * d + o] = f32_to_bf16(x[i] * inv * wv[i]);
  }
}

hipError_t launch_rmsnorm_rows(float* part, int32_t slices, int32_t n, int32_t d, const void* weight, float eps,
                               uint16_t* out, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (d > 256 * RN_PER) return hipErrorInvalidValue;
  const uint16_t* wt = static_cast<const uint16_t*>(weight);
  if (slices >= 2 && d % 256 == 0) {
    rowsum_kernel<<<dim3(n, d / 256), 256, 0, st>>>(part, slices, n, d);
    rownorm_kernel<<<n, 256, 0, st>>>(part, n, d, wt, eps, out);
  } else {
    rmsnorm_rows_kernel<<<n, 256, 0, st>>>(part, slices, n, d, wt, eps, out);
  }
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void to_bf16_kernel(const float* in, int64_t n_elems, uint16_t* out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n_elems) out[i] = f32_to_bf16(in[i]);
}

// Eight elements per thread (n_elems a multiple of 8, 16-B aligned arrays).
__global__ __launch_bounds__(256) void to_bf16_x8_kernel(const float* in, int64_t n_elems, uint16_t* out) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 8;
  if (i >= n_elems) return;
  const f32x4 a = *reinterpret_cast<const f32x4*>(in + i);
  const f32x4 b = *reinterpret_cast<const f32x4*>(in + i + 4);
  *reinterpret_cast<u32x4*>(out + i) =
      u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])};
}

hipError_t launch_to_bf16(const float* in, int64_t n_elems, uint16_t* out, hipStream_t st) {
  if (n_elems <= 0) return hipSuccess;
  if (n_elems % 8 == 0 && aligned16(in) && aligned16(out))
    to_bf16_x8_kernel<<<static_cast<unsigned>((n_elems / 8 + 255) / 256), 256, 0, st>>>(in, n_elems, out);
  else
    to_bf16_kernel<<<static_cast<unsigned>((n_elems + 255) / 256), 256, 0, st>>>(in, n_elems, out);
  return hipGetLastError();
}

}  // namespace mla
