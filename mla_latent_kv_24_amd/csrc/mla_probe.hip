// Measurement kernels of the probe build (build.py --probe defines
// MLA_PHASE_STAMPS); the product library compiles this file to nothing.
//   probe_read_kernel: a plain streaming read (16-B loads, 8 in flight per
//     lane), the board's read ceiling for a kernel that does nothing else;
//   probe_lds_kernel: conflict-free ds_read_b128 from a 64 KB LDS buffer,
//     bytes per shader cycle per CU;
//   probe_mfma_kernel: four independent chains of v_mfma_f32_32x32x16_bf16
//     per wave on random operands, the matrix cores' rate and the shader
//     clock under that load;
//   probe_overlap_kernel: MFMA and VALU work in the same or in different
//     waves of a SIMD;
//   probe_floor_kernel: the decode attention's bytes and products at the V2
//     decode step with nothing else, the floor of any design on this board.
#include "mla_common.h"

#ifdef MLA_PHASE_STAMPS

namespace mla {

__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4* p, int64_t n16, uint32_t* sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = p[i + k * stride];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc ^= v[k];
  }
  for (; i < n16; i += stride) acc ^= p[i];
  const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (x == 0x9e3779b9u) sink[blockIdx.x] = x;  // data-dependent: the loads stay
}

__global__ __launch_bounds__(256) void probe_lds_kernel(int iters, uint64_t* out) {
  __shared__ u32x4 buf[4096];  // 64 KB
  const int t = threadIdx.x;
  for (int i = t; i < 4096; i += 256) buf[i] = u32x4{static_cast<uint32_t>(i), 1u, 2u, 3u};
  __syncthreads();
  u32x4 acc = {0u, 0u, 0u, 0u};
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 16; ++k) acc ^= buf[(t + 256 * k + 64 * it) & 4095];  // consecutive 16 B per lane
  }
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  if (t == 0) {
    out[2 * blockIdx.x] = c1 - c0;
    out[2 * blockIdx.x + 1] = static_cast<uint64_t>(iters) * 16 * 256 * 16;  // bytes read by the workgroup
  }
  if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x9e3779b9u) out[2 * blockIdx.x] = 0;
}

__global__ __launch_bounds__(256) void probe_mfma_kernel(int iters, uint64_t* out, float* sink) {
  // random operand bits per lane (a hash of the lane and block)
  uint32_t h = (blockIdx.x * 256u + threadIdx.x) * 2654435761u + 0x7f4a7c15u;
  u32x4 ra, rb;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    h ^= h << 13;
    h ^= h >> 17;
    h ^= h << 5;
    ra[k] = h & 0xbfffbfffu;  // finite bf16 pairs
    h ^= h << 13;
    h ^= h >> 17;
    h ^= h << 5;
    rb[k] = h & 0xbfffbfffu;
  }
  const bf16x8 a = __builtin_bit_cast(bf16x8, ra), b = __builtin_bit_cast(bf16x8, rb);
  f32x16 c[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) c[k][r] = 0.f;
  const uint64_t c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 4; ++k) c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[k], 0, 0, 0);
  }
  const uint64_t c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    out[2 * blockIdx.x] = c1 - c0;
    out[2 * blockIdx.x + 1] = r1 - r0;
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) s += c[k][0];
  if (s != s) sink[blockIdx.x] = s;  // the products stay
}

// Does VALU work overlap matrix-core work on a SIMD?  Per iteration a wave
// issues NM v_mfma_f32_32x32x16_bf16 (four independent chains) and/or NV
// v_fma_f32 (16 independent chains), all unrolled so that every operand stays
// in registers; mode 0: every wave does both, one MFMA then NV/NM FMAs; mode 1:
// waves 0-3 only the MFMAs, waves 4-7 only the FMAs (one of each per SIMD);
// mode 2: every wave only the MFMAs; mode 3: every wave only the FMAs.  Each
// wave's cycles over the loop go to out.
template <int NM, int NV>
__global__ __launch_bounds__(512) void probe_overlap_kernel(int iters, int mode, uint64_t* out, float* sink) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint32_t h = (blockIdx.x * 512u + threadIdx.x) * 2654435761u + 0x7f4a7c15u;
  u32x4 ra, rb;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    h ^= h << 13;
    h ^= h >> 17;
    h ^= h << 5;
    ra[k] = h & 0xbfffbfffu;
    h ^= h << 13;
    h ^= h >> 17;
    h ^= h << 5;
    rb[k] = h & 0xbfffbfffu;
  }
  const bf16x8 a = __builtin_bit_cast(bf16x8, ra), b = __builtin_bit_cast(bf16x8, rb);
  f32x16 c[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) c[k][r] = 0.f;
  float x[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) x[k] = static_cast<float>(threadIdx.x + k) * 1e-3f;
  const float fa = 0.999f, fb = 1e-4f;
  const bool do_m = mode == 0 || mode == 2 || (mode == 1 && w < 4);
  const bool do_v = mode == 0 || mode == 3 || (mode == 1 && w >= 4);
  constexpr int PER = NV / NM;
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  if (do_m && do_v) {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        c[m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[m & 3], 0, 0, 0);
#pragma unroll
        for (int v = 0; v < PER; ++v) x[(m * PER + v) & 15] = fmaf(x[(m * PER + v) & 15], fa, fb);
      }
    }
  } else if (do_m) {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int m = 0; m < NM; ++m) c[m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[m & 3], 0, 0, 0);
    }
  } else {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int v = 0; v < NV; ++v) x[v & 15] = fmaf(x[v & 15], fa, fb);
    }
  }
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  if ((threadIdx.x & 63) == 0) out[blockIdx.x * 8 + w] = c1 - c0;
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) s += c[k][0];
#pragma unroll
  for (int k = 0; k < 16; ++k) s += x[k];
  if (s != s) sink[blockIdx.x] = s;
}

// The decode attention's work at the V2 decode step and nothing else: each
// workgroup (4 waves, one per SIMD, one workgroup per CU as in the attention
// kernel) streams `tiles` tiles of 36,864 B (the attention kernel's 32-row
// tile) from its own contiguous share of p, three tiles in flight in
// registers, and per tile each wave issues 68 v_mfma_f32_32x32x16_bf16 (the
// attention kernel's 36 score and 32 value products of a tile) with the
// streamed data as the A operand.  No LDS, no softmax, no barrier: a floor
// for any kernel that must both stream those bytes and issue those products
// on this board.  MODE 0: both; 1: the products alone (operands from
// registers, no loads); 2: the loads alone (one product per tile on the
// tile's xor keeps them).
template <int MODE>
__global__ __launch_bounds__(256, 1) void probe_floor_kernel(const u32x4* p, int64_t tiles, uint64_t* out,
                                                             float* sink) {
  constexpr int PER = 36864 / 16 / 256;  // 16-B loads per thread per tile (9)
  constexpr int NM = 68;
  const int tid = threadIdx.x;
  const u32x4* base = p + static_cast<int64_t>(blockIdx.x) * tiles * (PER * 256) + tid;
  uint32_t h = (blockIdx.x * 256u + tid) * 2654435761u + 0x7f4a7c15u;
  u32x4 rb;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    h ^= h << 13;
    h ^= h >> 17;
    h ^= h << 5;
    rb[k] = h & 0xbfffbfffu;  // finite bf16 pairs
  }
  const bf16x8 b = __builtin_bit_cast(bf16x8, rb);
  f32x16 c[8];
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) c[k][r] = 0.f;
  u32x4 buf[4][PER];
  // Tiles t, t+1, t+2 are in flight while tile t-1 is worked on; the
  // scheduling barriers keep each tile's loads ahead of the earlier tile's
  // work (the compiler would otherwise sink them to their first use).
  auto load = [&](int slot, int64_t t) {
    const u32x4* q = base + min(t, tiles - 1) * (PER * 256);  // past the end: the last tile again
#pragma unroll
    for (int i = 0; i < PER; ++i) buf[slot][i] = q[256 * i];
    __builtin_amdgcn_sched_barrier(0);
  };
  auto work = [&](int slot) {
    if constexpr (MODE == 2) {  // one product on the tile's xor: the loads stay, almost no matrix work
      u32x4 x = buf[slot][0];
#pragma unroll
      for (int i = 1; i < PER; ++i) x ^= buf[slot][i];
      c[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, x & 0xbfffbfffu), b, c[0], 0, 0, 0);
    } else {
#pragma unroll
      for (int m = 0; m < NM; ++m)
        c[m & 7] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, buf[slot][m % PER]), b,
                                                           c[m & 7], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  if constexpr (MODE == 1) {
#pragma unroll
    for (int k = 0; k < 4; ++k) load(k, k);
  }
  const uint64_t c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  if constexpr (MODE != 1) {
    load(0, 0);
    load(1, 1);
    load(2, 2);
  }
  // tiles is a multiple of 4 (checked by the host)
  for (int64_t t = 0; t < tiles; t += 4) {
    if constexpr (MODE != 1) load(3, t + 3);
    work(0);
    if constexpr (MODE != 1) load(0, t + 4);
    work(1);
    if constexpr (MODE != 1) load(1, t + 5);
    work(2);
    if constexpr (MODE != 1) load(2, t + 6);
    work(3);
  }
  const uint64_t c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  if (tid == 0) {
    out[2 * blockIdx.x] = c1 - c0;
    out[2 * blockIdx.x + 1] = r1 - r0;
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += c[k][0];
  if (s != s) sink[blockIdx.x] = s;  // the products and the loads stay
}

}  // namespace mla

// Host entry points of the probe build.  Each launches on `stream` and returns
// the launch status; the caller times the launch with events.
extern "C" int mla_probe_read(const void* p, int64_t bytes, void* sink, int32_t workgroups, void* stream) {
  mla::probe_read_kernel<<<workgroups, 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const mla::u32x4*>(p), bytes / 16, static_cast<uint32_t*>(sink));
  return static_cast<int>(hipGetLastError());
}
extern "C" int mla_probe_lds(int32_t iters, void* out, int32_t workgroups, void* stream) {
  mla::probe_lds_kernel<<<workgroups, 256, 0, static_cast<hipStream_t>(stream)>>>(iters, static_cast<uint64_t*>(out));
  return static_cast<int>(hipGetLastError());
}
extern "C" int mla_probe_mfma(int32_t iters, void* out, void* sink, int32_t workgroups, void* stream) {
  mla::probe_mfma_kernel<<<workgroups, 256, 0, static_cast<hipStream_t>(stream)>>>(iters, static_cast<uint64_t*>(out),
                                                                                    static_cast<float*>(sink));
  return static_cast<int>(hipGetLastError());
}

// nv is 64 or 128 FMAs per 8 MFMAs per iteration
extern "C" int mla_probe_overlap(int32_t iters, int32_t mode, int32_t nv, void* out, void* sink, int32_t workgroups,
                                 void* stream) {
  auto* o = static_cast<uint64_t*>(out);
  auto* k = static_cast<float*>(sink);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (nv == 64)
    mla::probe_overlap_kernel<8, 64><<<workgroups, 512, 0, st>>>(iters, mode, o, k);
  else if (nv == 128)
    mla::probe_overlap_kernel<8, 128><<<workgroups, 512, 0, st>>>(iters, mode, o, k);
  else
    return static_cast<int>(hipErrorInvalidValue);
  return static_cast<int>(hipGetLastError());
}

extern "C" int mla_probe_floor(const void* p, int64_t tiles, int32_t mode, void* out, void* sink, int32_t workgroups,
                               void* stream) {
  const auto* q = static_cast<const mla::u32x4*>(p);
  auto* o = static_cast<uint64_t*>(out);
  auto* k = static_cast<float*>(sink);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (tiles < 4 || tiles % 4) return static_cast<int>(hipErrorInvalidValue);
  switch (mode) {
    case 0: mla::probe_floor_kernel<0><<<workgroups, 256, 0, st>>>(q, tiles, o, k); break;
    case 1: mla::probe_floor_kernel<1><<<workgroups, 256, 0, st>>>(q, tiles, o, k); break;
    case 2: mla::probe_floor_kernel<2><<<workgroups, 256, 0, st>>>(q, tiles, o, k); break;
    default: return static_cast<int>(hipErrorInvalidValue);
  }
  return static_cast<int>(hipGetLastError());
}

#endif  // MLA_PHASE_STAMPS
