// A4 + A5 -- combine split-KV partials and lift the latent by W^UV, gfx950.
//
//   LSE = log sum_s exp(lse_s),   z = sum_s exp(lse_s - LSE) Z_s
// is softmax_j over all rows re-associated from per-split pieces, and
//   o_i = U^V_i z_i
// is the value up-projection moved outside the weighted sum
// (jiphyeonjeon.kr DeepSeek-V2 review, section 2: sum_j a_ij U^V_i c_j =
// U^V_i sum_j a_ij c_j).
#include <algorithm>

#include "mla_common.h"

namespace mla {

constexpr float CNEG_INF = -__builtin_huge_valf();
constexpr int CMB_MAX_SPLITS = 128;   // weights staged in LDS for the MFMA path
constexpr int ZSTRIDE = 1040;        // bytes per staged z row (512 bf16 + 16 B pad)

// ------------------------------------------------------------------------
// bf16 MFMA path.  Grid (head, nblk blocks of qb <= 32 queries, taken in turn
// with W^UV loaded once); 4 waves, wave w owns
// the 32 output dims d = 32w..32w+31.  z is combined in fp32, optionally
// written out, then split into bf16 hi + lo parts (z = hi + lo to ~2^-16
// relative) so the 32x32x16 MFMA lift keeps fp32-level accuracy:
//   out[n][d] = sum_c (hi[n][c] + lo[n][c]) * w_uv[h][d][c]
// A = z rows from LDS (c contiguous; rows past the block's queries are never
// stored), B = w_uv rows from global (c contiguous).
// The kernel is a stream of the partials and of W^UV.  The split weights are
// formed by all threads (8 per query row).  With at most G = 4 splits a
// thread's first two row chunks of partials are requested, then the wave's
// whole W^UV slice (32 rows x 512 columns, 128 VGPRs), which arrives while the
// partials are combined; two batches of two row chunks stay in flight (one
// combined while the next lands).  With more splits (G = 16), or one (G = 1:
// a prefill chunk, one split per query), W^UV comes first and the partial
// loads of G splits x 16 / G row chunks are in flight together.
// ------------------------------------------------------------------------
template <int G, bool MULTI>
__global__ __launch_bounds__(256, 1) void combine_mfma_kernel(CombineArgs a, int qb, int nblk) {
  __shared__ float wts[32][CMB_MAX_SPLITS];
  __shared__ __attribute__((aligned(16))) uint8_t zhi[32 * ZSTRIDE];
  __shared__ __attribute__((aligned(16))) uint8_t zlo[32 * ZSTRIDE];
  constexpr int KS = D_C / 16;  // MFMA k-steps of the lift
  constexpr int UB = 16 / G;    // row chunks per batch
  const int h = blockIdx.x;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int S = a.num_splits;

  // B operands of the lift: this lane's W^UV row d, 16 columns per k-step
  const int g = l >> 5;
  const int d = 32 * w + (l & 31);
  const uint16_t* wrow = static_cast<const uint16_t*>(a.w_uv) + (static_cast<int64_t>(h) * D_H + d) * D_C + 8 * g;
  u32x4 bw[KS];
  auto load_w = [&]() {
#pragma unroll
    for (int s = 0; s < KS; ++s) bw[s] = *reinterpret_cast<const u32x4*>(wrow + 16 * s);
  };

  // one split over several blocks: a block's 16 row chunks per thread are
  // requested while the previous block is lifted (z_part[n][0][h][:])
  f32x4 v1[16];
  auto load1 = [&](int nb, int rb, f32x4 (&v)[16]) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int u = tid + 256 * i;
      v[i] = (u < rb * (D_C / 4))
                 ? *reinterpret_cast<const f32x4*>(a.z_part + (static_cast<int64_t>(nb + (u >> 7)) * a.n_h + h) * D_C +
                                                   4 * (u & 127))
                 : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };

  // query blocks blockIdx.y * nblk .. +nblk-1 in turn; W^UV stays in registers
  // (MULTI = false: one block and no loop-end barrier, as the decode steps launch it)
  for (int blk = 0; blk < (MULTI ? nblk : 1); ++blk) {
  const int n0 = (blockIdx.y * nblk + blk) * qb;
  if (n0 >= a.n_q) break;  // uniform over the workgroup
  const int rows = min(qb, a.n_q - n0);
  const bool first = !MULTI || blk == 0;

  // ---- split weights exp(lse_s - LSE): thread (row r, phase p) covers splits
  // p, p+8, ...; max and sum are reduced over the row's 8 adjacent lanes
  {
    const int r = tid >> 3, p = tid & 7;
    const bool rv = r < rows;
    const float* ls = a.lse_part + static_cast<int64_t>(n0 + (rv ? r : 0)) * S * a.n_h + h;
    float m = CNEG_INF;
    if (rv)
      for (int s = p; s < S; s += 8) m = fmaxf(m, ls[static_cast<int64_t>(s) * a.n_h]);
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
    float tot = 0.f;
    if (rv)
      for (int s = p; s < S; s += 8) {
        const float e = (m == CNEG_INF) ? 0.f : expf(ls[static_cast<int64_t>(s) * a.n_h] - m);
        wts[r][s] = e;
        tot += e;
      }
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) tot += __shfl_xor(tot, o);
    const float inv = (tot > 0.f) ? 1.f / tot : 0.f;
    for (int s = p; s < S; s += 8) wts[r][s] = rv ? wts[r][s] * inv : 0.f;
  }
  __syncthreads();

  // ---- combined latent: unit u = (row u / 128, 4-column chunk u % 128), thread
  // tid takes units tid + 256 j; consecutive lanes read consecutive 16 B
  const int units = rows * (D_C / 4);
  const int64_t zs = static_cast<int64_t>(a.n_h) * D_C;  // split stride (floats)
  auto emit = [&](int u, const f32x4& acc) {
    if (u >= units) return;
    const int r = u >> 7, c4 = 4 * (u & 127);
    if (a.out_latent)
      *reinterpret_cast<f32x4*>(a.out_latent + (static_cast<int64_t>(n0 + r) * a.n_h + h) * D_C + c4) = acc;
    uint16_t hi4[4], lo4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      hi4[e] = f32_to_bf16(acc[e]);
      lo4[e] = f32_to_bf16(acc[e] - bf16_to_f32(hi4[e]));
    }
    *reinterpret_cast<uint2*>(zhi + r * ZSTRIDE + 2 * c4) =
        make_uint2(hi4[0] | (static_cast<uint32_t>(hi4[1]) << 16), hi4[2] | (static_cast<uint32_t>(hi4[3]) << 16));
    *reinterpret_cast<uint2*>(zlo + r * ZSTRIDE + 2 * c4) =
        make_uint2(lo4[0] | (static_cast<uint32_t>(lo4[1]) << 16), lo4[2] | (static_cast<uint32_t>(lo4[3]) << 16));
  };
  if constexpr (G == 1 && MULTI) {
    if (first) {
      load1(n0, rows, v1);
      load_w();
    }
    f32x4 cur[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) cur[i] = v1[i];
    const int n1 = n0 + qb;
    if (blk + 1 < nblk && n1 < a.n_q) load1(n1, min(qb, a.n_q - n1), v1);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int u = tid + 256 * i;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      acc += wts[(u >> 7) & 31][0] * cur[i];
      emit(u, acc);
    }
  } else if (G == 4 && S <= G) {
    // all splits of a unit in one batch of PB units; two batches in flight
    constexpr int PB = 2;
    f32x4 va[PB][G], vb[PB][G];
    auto load_b = [&](int j0, f32x4 (&v)[PB][G]) {
#pragma unroll
      for (int i = 0; i < PB; ++i) {
        const int u = tid + 256 * (j0 + i);
        const float* zp = a.z_part + ((static_cast<int64_t>(n0 + (u >> 7)) * S) * a.n_h + h) * D_C + 4 * (u & 127);
#pragma unroll
        for (int gg = 0; gg < G; ++gg)
          v[i][gg] = (u < units && gg < S) ? *reinterpret_cast<const f32x4*>(zp + gg * zs) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    };
    auto fold_b = [&](int j0, const f32x4 (&v)[PB][G]) {
#pragma unroll
      for (int i = 0; i < PB; ++i) {
        const int u = tid + 256 * (j0 + i);
        const int r = u >> 7;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int gg = 0; gg < G; ++gg)
          if (gg < S) acc += wts[r & 31][gg] * v[i][gg];
        emit(u, acc);
      }
    };
    load_b(0, va);
    if (first) load_w();
#pragma unroll
    for (int j0 = 0; j0 < 16; j0 += 2 * PB) {
      if (j0 + PB < 16) load_b(j0 + PB, vb);
      fold_b(j0, va);
      if (j0 + 2 * PB < 16) load_b(j0 + 2 * PB, va);
      fold_b(j0 + PB, vb);
    }
  } else {
    if (first) load_w();
    for (int j0 = 0; j0 < 16; j0 += UB) {
      if (tid + 256 * j0 >= units) break;
      f32x4 acc[UB];
#pragma unroll
      for (int i = 0; i < UB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int s0 = 0; s0 < S; s0 += G) {
        f32x4 v[UB][G];
#pragma unroll
        for (int i = 0; i < UB; ++i) {
          const int u = tid + 256 * (j0 + i);
          const float* zp = a.z_part + ((static_cast<int64_t>(n0 + (u >> 7)) * S + s0) * a.n_h + h) * D_C + 4 * (u & 127);
#pragma unroll
          for (int gg = 0; gg < G; ++gg)
            v[i][gg] = (u < units && s0 + gg < S) ? *reinterpret_cast<const f32x4*>(zp + gg * zs)
                                                  : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int i = 0; i < UB; ++i) {
          const int r = (tid + 256 * (j0 + i)) >> 7;
#pragma unroll
          for (int gg = 0; gg < G; ++gg)
            if (s0 + gg < S) acc[i] += wts[r & 31][s0 + gg] * v[i][gg];
        }
      }
#pragma unroll
      for (int i = 0; i < UB; ++i) emit(tid + 256 * (j0 + i), acc[i]);
    }
  }
  __syncthreads();

  const int arow = (l & 31) * ZSTRIDE + 16 * g;
  f32x16 acc = {0};
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const u32x4 b = bw[s];
    const u32x4 ah = *reinterpret_cast<const u32x4*>(zhi + arow + 32 * s);
    const u32x4 al = *reinterpret_cast<const u32x4*>(zlo + arow + 32 * s);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ah),
                                                  __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, al),
                                                  __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int r = 8 * (j >> 2) + 4 * g + (j & 3);
    if (r < rows) a.out[(static_cast<int64_t>(n0 + r) * a.n_h + h) * D_H + d] = acc[j];
  }
  if constexpr (MULTI) __syncthreads();  // the next block rewrites the weights and the staged z
  }
}

// ------------------------------------------------------------------------
// Generic fp32 path: one workgroup per (query, head).
// ------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void combine_generic_kernel(CombineArgs a) {
  __shared__ float z[1024];
  __shared__ float lsum[2];
  const int n = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int S = a.num_splits;
  const float* ls = a.lse_part + static_cast<int64_t>(n) * S * a.n_h + h;
  if (tid == 0) {
    float m = CNEG_INF;
    for (int s = 0; s < S; ++s) m = fmaxf(m, ls[static_cast<int64_t>(s) * a.n_h]);
    float tot = 0.f;
    for (int s = 0; s < S; ++s)
      tot += (m == CNEG_INF) ? 0.f : expf(ls[static_cast<int64_t>(s) * a.n_h] - m);
    lsum[0] = m;
    lsum[1] = tot;
  }
  __syncthreads();
  const float m = lsum[0], tot = lsum[1];
  for (int c = tid; c < a.d_c; c += 256) {
    float acc = 0.f;
    for (int s = 0; s < S; ++s) {
      const float e = (m == CNEG_INF) ? 0.f : expf(ls[static_cast<int64_t>(s) * a.n_h] - m) / tot;
      if (e != 0.f) acc = fmaf(e, a.z_part[((static_cast<int64_t>(n) * S + s) * a.n_h + h) * a.d_c + c], acc);
    }
    z[c] = acc;
    if (a.out_latent) a.out_latent[(static_cast<int64_t>(n) * a.n_h + h) * a.d_c + c] = acc;
  }
  __syncthreads();
  const T* wv = static_cast<const T*>(a.w_uv) + static_cast<int64_t>(h) * a.d_h * a.d_c;
  for (int d = tid; d < a.d_h; d += 256) {
    float acc = 0.f;
    for (int c = 0; c < a.d_c; ++c) acc = fmaf(load_as_f32(wv, static_cast<int64_t>(d) * a.d_c + c), z[c], acc);
    a.out[(static_cast<int64_t>(n) * a.n_h + h) * a.d_h + d] = acc;
  }
}

hipError_t launch_combine(const CombineArgs& a, int bf16, hipStream_t st) {
  if (a.n_q <= 0) return hipSuccess;
  if (bf16 && a.d_c == D_C && a.d_h == D_H && a.num_splits <= CMB_MAX_SPLITS) {
    // query block: the largest of 32, 16, ..., 1 that still gives >= 256
    // workgroups (W^UV is read once per block, mostly from the L2 of the XCD
    // that holds the head's blocks; the partials once in all)
    int qb = 32;
    while (qb > 1 && static_cast<int64_t>(a.n_h) * ((a.n_q + qb - 1) / qb) < 256) qb >>= 1;
    // many query blocks (a prefill chunk): a workgroup takes several in turn,
    // so that W^UV is read once per workgroup for all of them, keeping about
    // four rounds of the 256 CUs
    const int64_t blocks = (a.n_q + qb - 1) / qb;
    const int nblk = static_cast<int>(std::max<int64_t>(1, blocks * a.n_h / 1024));
    const dim3 grid(a.n_h, static_cast<unsigned>((blocks + nblk - 1) / nblk));
    if (nblk > 1) {
      if (a.num_splits == 1)
        combine_mfma_kernel<1, true><<<grid, 256, 0, st>>>(a, qb, nblk);
      else if (a.num_splits <= 4)
        combine_mfma_kernel<4, true><<<grid, 256, 0, st>>>(a, qb, nblk);
      else
        combine_mfma_kernel<16, true><<<grid, 256, 0, st>>>(a, qb, nblk);
    } else if (a.num_splits == 1) {
      combine_mfma_kernel<1, false><<<grid, 256, 0, st>>>(a, qb, nblk);
    } else if (a.num_splits <= 4) {
      combine_mfma_kernel<4, false><<<grid, 256, 0, st>>>(a, qb, nblk);
    } else {
      combine_mfma_kernel<16, false><<<grid, 256, 0, st>>>(a, qb, nblk);
    }
  } else if (bf16) {
    combine_generic_kernel<uint16_t><<<dim3(a.n_q, a.n_h), 256, 0, st>>>(a);
  } else {
    combine_generic_kernel<float><<<dim3(a.n_q, a.n_h), 256, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace mla
