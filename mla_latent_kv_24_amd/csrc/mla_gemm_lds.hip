// LDS-tiled bf16 product for the projections of many tokens, gfx950:
//   part[s][n][m] = sum_{k in slice s} A[m][k] B[n][k]
// with both operands K-contiguous: A = weight rows (two blocks stacked at
// `split`, nn-linear layout), B = activation rows, fp32 accumulation, one k
// slice per workgroup (the KV down-projection of a chunk of hidden states:
// irregular6612 notes, section 2.1.2, and the DeepSeek-V3 report, Metode 1).
// Workgroup tile 192 x 256 over 64-deep k stages: each stage of A (192 rows)
// and B (256 rows), 128 B per row, reaches LDS by DMA (buffer_load ... lds,
// 8 rows per instruction), double-buffered, one barrier per stage.  Four
// waves in a 2 x 2 grid each own 96 x 128 of the tile as 3 x 4 blocks of
// v_mfma_f32_32x32x16_bf16, A and B fragments read from LDS one k-step ahead.
// A staged row's 16-byte slot s holds chunk s ^ ((row >> 1) & 7): the 16 rows
// that one pass of a fragment read touches then hit distinct banks.
#include <algorithm>

#include "mla_common.h"
#include "mla_tile.h"

namespace mla {

constexpr int LG_BM = 192;                  // A rows (outputs) per tile
constexpr int LG_BN = 256;                  // B rows (tokens) per tile
constexpr int LG_BK = 64;                   // k per stage
constexpr int LG_ROW = LG_BK * 2;           // bytes per staged row
constexpr int LG_A_BYTES = LG_BM * LG_ROW;
constexpr int LG_STAGE = (LG_BM + LG_BN) * LG_ROW;
constexpr int LG_MB = LG_BM / 64;           // 32-row A blocks per wave
constexpr int LG_A_DMA = LG_BM / 32;        // 8-row DMA groups per wave per stage (A)
constexpr int LG_B_DMA = LG_BN / 32;        // (B)

// A raw buffer resource over `bytes` bytes at address ga (reads past them return zeros).
__device__ __forceinline__ i32x4 lg_rsrc(uint64_t ga, int64_t bytes) {
  const i32x4 rs = {__builtin_amdgcn_readfirstlane(static_cast<int>(ga & 0xffffffffu)),
                    __builtin_amdgcn_readfirstlane(static_cast<int>((ga >> 32) & 0xffffu)),
                    __builtin_amdgcn_readfirstlane(static_cast<int>(bytes)), 0x00020000};
  return rs;
}

// Grid (d_out / 192, token tiles, k slices).
__global__ __launch_bounds__(256, 1) void gemm_lds_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * LG_STAGE];
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = l >> 5, l32 = l & 31;
  const int wm = w >> 1, wn = w & 1;
  const int m0 = blockIdx.x * LG_BM;
  const int64_t n0 = static_cast<int64_t>(blockIdx.y) * LG_BN;
  const int slice = blockIdx.z;
  const int kb = slice * a.k_per_slice;
  const int ke = min(kb + a.k_per_slice, a.d_in);
  const int64_t stride = static_cast<int64_t>(a.d_in) * 2;  // bytes per operand row

  // ---- operand row groups, 8 rows per DMA instruction: group q of A is rows
  // m0 + 8q .., of B rows n0 + 8q ..; the group's first row at k = 0 and the
  // bytes of its valid rows (a split and d_out multiple of 8 keep a group on
  // one side of split)
  auto a_group = [&](int q, uint64_t& ga, int64_t& bytes) {
    const int r = m0 + 8 * q;
    const int rows = max(min(8, a.d_out - r), 0);
    const uint16_t* base = (r < a.split) ? static_cast<const uint16_t*>(a.w0) + static_cast<int64_t>(r) * a.d_in
                                         : static_cast<const uint16_t*>(a.w1) + static_cast<int64_t>(r - a.split) * a.d_in;
    ga = reinterpret_cast<uint64_t>(rows > 0 ? base : static_cast<const uint16_t*>(a.w0));
    bytes = rows * stride;
  };
  auto b_group = [&](int q, uint64_t& ga, int64_t& bytes) {
    const int64_t t = n0 + 8 * q;
    const int64_t rows = max(min(static_cast<int64_t>(8), static_cast<int64_t>(a.n) - t), static_cast<int64_t>(0));
    ga = reinterpret_cast<uint64_t>(static_cast<const uint16_t*>(a.x) + (rows > 0 ? t : 0) * a.d_in);
    bytes = rows * stride;
  };
  // lane L of a DMA instruction: row L / 8 of the group, slot L % 8 holding
  // chunk (L % 8) ^ ((row >> 1) & 7); a group's first row is a multiple of 8
  const int drow = l >> 3;
  auto lane_off = [&](int q) { return static_cast<int>(drow * stride) + 16 * ((l & 7) ^ (((8 * q + drow) >> 1) & 7)); };
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) uint8_t*)smem));
  // stage st (k0 = kb + 64 st) into buffer buf; every row's range starts at
  // k0 and runs to the end of its valid rows, so k0 + 64 <= d_in keeps each
  // valid chunk inside it
  auto issue = [&](int st, int buf) {
    const int k0 = kb + st * LG_BK;
    const uint32_t sbase = lds0 + static_cast<uint32_t>(buf * LG_STAGE);
#pragma unroll
    for (int i = 0; i < LG_A_DMA; ++i) {
      const int q = 4 * i + w;
      uint64_t ga;
      int64_t bytes;
      a_group(q, ga, bytes);
      dma16(sbase + 1024u * q, lane_off(q), lg_rsrc(ga + 2 * static_cast<uint64_t>(k0), bytes > 0 ? bytes - 2 * k0 : 0), 0);
    }
#pragma unroll
    for (int i = 0; i < LG_B_DMA; ++i) {
      const int q = 4 * i + w;
      uint64_t ga;
      int64_t bytes;
      b_group(q, ga, bytes);
      dma16(sbase + LG_A_BYTES + 1024u * q, lane_off(q),
            lg_rsrc(ga + 2 * static_cast<uint64_t>(k0), bytes > 0 ? bytes - 2 * k0 : 0), 0);
    }
  };

  // ---- fragments: row 32 blk + l32 of the wave's part, chunk 2 ks + g
  const int sw = (l32 >> 1) & 7;
  auto afrag = [&](int buf, int i, int ks) -> bf16x8 {
    const int row = (LG_BM / 2) * wm + 32 * i + l32;
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(smem + buf * LG_STAGE + row * LG_ROW +
                                                                       16 * ((2 * ks + g) ^ sw)));
  };
  auto bfrag = [&](int buf, int j, int ks) -> bf16x8 {
    const int row = 128 * wn + 32 * j + l32;
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(smem + buf * LG_STAGE + LG_A_BYTES +
                                                                       row * LG_ROW + 16 * ((2 * ks + g) ^ sw)));
  };

  f32x16 acc[LG_MB][4];
#pragma unroll
  for (int i = 0; i < LG_MB; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nst = (ke - kb) / LG_BK;  // the plan makes k ranges multiples of 64
  if (nst > 0) issue(0, 0);
  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    // stage st landed; every wave is done with stage st-1, whose buffer takes st+1
    vm_wait<0>();
    __syncthreads();
    if (st + 1 < nst) issue(st + 1, buf ^ 1);
    bf16x8 af[2][LG_MB], bf[2][4];
#pragma unroll
    for (int i = 0; i < LG_MB; ++i) af[0][i] = afrag(buf, i, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[0][j] = bfrag(buf, j, 0);
#pragma unroll
    for (int ks = 0; ks < LG_BK / 16; ++ks) {
      const int c = ks & 1;
      if (ks + 1 < LG_BK / 16) {
#pragma unroll
        for (int i = 0; i < LG_MB; ++i) af[c ^ 1][i] = afrag(buf, i, ks + 1);
#pragma unroll
        for (int j = 0; j < 4; ++j) bf[c ^ 1][j] = bfrag(buf, j, ks + 1);
      }
#pragma unroll
      for (int i = 0; i < LG_MB; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[c][i], bf[c][j], acc[i][j], 0, 0, 0);
    }
  }

  // ---- partial sums: lane l holds output m0 + 96 wm + 32 i + 8 jq + 4 g + e,
  // token n0 + 128 wn + 32 j + l32, in acc[i][j][4 jq + e]
  float* dst = a.part + static_cast<int64_t>(slice) * a.n * a.d_out;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t t = n0 + 128 * wn + 32 * j + l32;
    if (t >= a.n) continue;
#pragma unroll
    for (int i = 0; i < LG_MB; ++i)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        const int o = m0 + (LG_BM / 2) * wm + 32 * i + 8 * jq + 4 * g;
        if (o < a.d_out)
          *reinterpret_cast<f32x4*>(dst + t * a.d_out + o) =
              f32x4{acc[i][j][4 * jq], acc[i][j][4 * jq + 1], acc[i][j][4 * jq + 2], acc[i][j][4 * jq + 3]};
      }
  }
}

bool gemm_lds_applies(int32_t n, int32_t d_in, int32_t d_out) {
  return n >= LG_BN && d_in % LG_BK == 0 && d_out % LG_BM == 0;
}

// k slices for about one round of 256 workgroups, each at least 4 stages deep
void gemm_lds_plan(int32_t n, int32_t d_in, int32_t d_out, int32_t& k_slices, int32_t& k_per_slice) {
  const int64_t tiles = static_cast<int64_t>(d_out / LG_BM) * ((n + LG_BN - 1) / LG_BN);
  int64_t s = std::max<int64_t>(1, (256 + tiles / 2) / tiles);
  s = std::min<int64_t>(s, std::max(1, d_in / (4 * LG_BK)));
  int64_t kr = (d_in + s - 1) / s;
  kr = (kr + LG_BK - 1) / LG_BK * LG_BK;
  k_per_slice = static_cast<int32_t>(kr);
  k_slices = static_cast<int32_t>((d_in + kr - 1) / kr);
}

// rows [w0 ; w1] (split at `split`, a multiple of 8) against n activation
// rows, into part[k_slices][n][d_out]; with gemm_lds_applies and gemm_lds_plan
hipError_t launch_gemm_lds_partial(const GemmArgs& g, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(g.d_out / LG_BM), static_cast<unsigned>((g.n + LG_BN - 1) / LG_BN),
                  static_cast<unsigned>(g.k_slices));
  gemm_lds_kernel<<<grid, 256, 0, st>>>(g);
  return hipGetLastError();
}

}  // namespace mla
