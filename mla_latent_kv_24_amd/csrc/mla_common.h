// Shared device/host definitions of the gfx950 MLA kernels (internal).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

constexpr int D_C = 512;           // latent width d_c (fast path)
constexpr int D_H = 128;           // per-head content dim d_h
constexpr int D_R = 64;            // decoupled RoPE dim d_hR
constexpr int ROWE = D_C + D_R;    // elements per cache row
constexpr int ROWB = ROWE * 2;     // bytes per bf16 cache row (1152)
constexpr int TILE = 32;           // cache rows per LDS tile
constexpr int TILE_BYTES = TILE * ROWB;
constexpr int MAX_PAIRS = 64;      // RoPE pairs supported by the generic kernels (d_hR <= 128)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// RoPE frequencies theta_k = base^(-2k/d_hR), formed on the host in fp64.
struct RopeTable {
  double theta[MAX_PAIRS];
};

struct AppendArgs {
  const void* c_kv;
  const void* k_r;
  const int32_t* pos;
  const int64_t* row;
  void* cache;
  int32_t n_tok, d_c, d_r;
  RopeTable rope;
  // FP8 latent cache: `cache` receives the E4M3 codes, these the RoPE keys and scales
  void* fp8_rope;
  float* fp8_scale;
};

// Absorbed queries: q_lat [n_q][n_h][d_c + d_r] in the storage dtype (fp32, or
// bf16 = RNE of the fp32 value v), and for bf16 an optional second plane
// q_lat_lo of the same shape holding bf16(v - bf16(v)), so that hi + lo
// carries v to ~2^-17.  Kernels that refine their score with lo take it as 0
// when the plane is absent.
struct RopeQArgs {
  const void* q_r;       // [n_q][n_h][d_r] (storage dtype)
  const int32_t* q_pos;  // [n_q]
  void* q_lat;           // absorbed queries (hi plane for bf16)
  void* q_lat_lo;        // bf16 lo plane or NULL
  int32_t n_q, n_h, d_c, d_r;
  RopeTable rope;
};

struct AbsorbArgs {
  const void* q_c;   // [n_q][n_h][d_h] (storage dtype)
  const void* w_uk;  // [n_h][d_h][d_c] (storage dtype)
  void* q_lat;       // absorbed queries (hi plane for bf16)
  void* q_lat_lo;    // bf16 lo plane or NULL (not written)
  int32_t n_q, n_h, d_c, d_h, d_r;
  const void* q_r;       // [n_q][n_h][d_r] (storage dtype); used by the fused bf16 kernel
  const int32_t* q_pos;  // [n_q]
  RopeTable rope;
  int32_t q_r_f32;       // fused bf16 kernel: q_r holds fp32 values instead
  // A1 in the same launch (fused bf16 kernel only; app_n = 0: none): the bf16
  // cache rows cache[app_row[t]] = [app_c[t] ; RoPE(app_k[t], app_pos[t])],
  // t < app_n, written by the launch's workgroups besides their A2 work
  const void* app_c;        // [app_n][d_c]
  const void* app_k;        // [app_n][d_r] (pre-RoPE)
  const int32_t* app_pos;   // [app_n]
  const int64_t* app_row;   // [app_n]
  void* app_cache;          // [*][d_c + d_r]
  int32_t app_n;
};
// true when launch_absorb also writes the RoPE part (no launch_rope_q needed)
bool absorb_fuses_rope(int bf16, int d_c, int d_h, int d_r);

struct SplitArgs {
  const void* q_lat;      // absorbed queries (hi plane for bf16)
  const void* q_lat_lo;   // bf16 lo plane or NULL (read as zeros)
  const void* cache;      // rows of d_c + d_r
  const int32_t* lens;    // decode: seq_lens[batch]; prefill: prefix_lens[batch]
  float* z_part;          // [n_q][num_splits][n_h][d_c]
  float* lse_part;        // [n_q][num_splits][n_h]
  int64_t stride;         // rows per sequence slot
  int64_t split_rows;     // rows per split
  int32_t n_q, n_h, d_c, d_r;
  int32_t num_splits;
  int32_t max_len;        // host bound on the attended length
  int32_t q_per_seq;      // 1 for decode, chunk for prefill
  int32_t prefill;        // 0 decode, 1 causal prefill
  float qscale;           // softmax_scale * log2(e)
  // queries that attend fewer rows than this take the 16-head-group body,
  // which scores with hi + lo and carries the softmax weights as hi + lo
  int32_t precise_below;
  // paged cache (block_table != NULL): `cache` is the page pool, row r of
  // sequence b is row r & (2^page_shift - 1) of page block_table[b][r >> page_shift],
  // and stride = bt_stride << page_shift bounds the attended length
  const int32_t* block_table;  // [batch][bt_stride]
  int64_t num_pages;
  int32_t bt_stride;
  int32_t page_shift;          // >= 5: a page holds whole 32-row tiles
  // FP8 latent cache: `cache` holds the E4M3 codes [rows][d_c], these the bf16
  // RoPE keys [rows][d_r] and the per-row scales [rows]
  const void* fp8_rope;
  const float* fp8_scale;
};

struct CombineArgs {
  const float* z_part;
  const float* lse_part;
  const void* w_uv;       // [n_h][d_h][d_c]
  float* out;             // [n_q][n_h][d_h]
  float* out_latent;      // optional [n_q][n_h][d_c]
  int32_t n_q, n_h, d_c, d_h, num_splits;
};

// Unabsorbed prefill.  Expanded rows x[b][h][row][576] (bf16) keep the cache
// row geometry: [k^C hi | v^C hi | k^C lo | v^C lo] (4 x 128) then k^R (64),
// with k^C = U^K_h c_row, v^C = U^V_h c_row formed in fp32 and split as
// hi = bf16(v), lo = bf16(v - hi).
constexpr int XROWS_ALIGN = 128;   // rows_cap is a multiple of this
struct ExpandArgs {
  const void* cache;            // bf16 rows of d_c + d_r
  const int32_t* prefix_lens;   // [batch]
  const void* w_uk;             // [n_h][d_h][d_c] bf16
  const void* w_uv;             // [n_h][d_h][d_c] bf16
  void* x;                      // [batch][n_h][rows_cap][576] bf16
  int64_t stride;               // cache rows per sequence slot
  int64_t rows_cap;             // expanded rows per (sequence, head)
  int32_t batch, n_h, chunk, max_len;  // max_len: host bound on prefix + chunk
  int32_t lo_rows;              // lo parts are written for rows below this only
  // paged cache, as SplitArgs (block_table != NULL)
  const int32_t* block_table;
  int64_t num_pages;
  int32_t bt_stride;
  int32_t page_shift;
};
struct PrefillArgs {
  const void* q_c;              // [batch][chunk][n_h][d_h] bf16
  const void* q_r;              // [batch][chunk][n_h][d_r] bf16, before RoPE
  const void* x;                // expanded rows (ExpandArgs::x)
  const int32_t* prefix_lens;   // [batch]
  float* out;                   // [batch][chunk][n_h][d_h] fp32
  int64_t rows_cap;
  int32_t batch, n_h, chunk, max_len;
  int32_t precise_below;        // workgroups whose first query sees fewer keys take hi + lo products
  float qscale;                 // softmax_scale * log2(e)
  RopeTable rope;
};

// y[t][o] = sum_k x[t][k] W[o][k] for W = [w0 (rows 0..split-1); w1 (rows
// split..d_out-1)], split-K over k.  part [k_slices][n][d_out] fp32; with one
// slice and out0 set, the sums go straight out as bf16: rows of out0 [n][split]
// and out1 [n][d_out - split] (or fp32 rows of out1_f32).
struct GemmArgs {
  const void* x;
  const void* w0;
  const void* w1;
  float* part;
  uint16_t* out0;
  uint16_t* out1;
  float* out1_f32;      // with out0: rows of the w1 part as fp32 here instead of out1
  int32_t n, d_in, d_out, split, k_slices, k_per_slice;
};
// split-K plan: slices (k per slice a multiple of 128) for ~256 workgroups
void gemm_plan(int32_t n, int32_t d_in, int32_t d_out, int32_t split, int32_t& k_slices, int32_t& k_per_slice);
// bf16 storage with d_in % 128 == 0 and split, d_out multiples of 64 take the
// matrix-core kernel; otherwise T = `bf16 ? uint16_t : float` generic kernels
hipError_t launch_gemm_partial(const GemmArgs& a, int bf16, hipStream_t st);
// slice sums to two outputs: columns < split as bf16 rows of out0, the rest fp32 rows of out1
hipError_t launch_slices_to_outputs(const float* part, int32_t slices, int32_t n, int32_t d_out, int32_t split,
                                    uint16_t* out0, float* out1, hipStream_t st);
// out[t][o] = sum_s part[s][t][o] (fp32)
hipError_t launch_sum_slices(const float* part, int32_t slices, int64_t n_elems, float* out, hipStream_t st);
// per row t: v = sum_s part[s][t][:d]; out[t][:] = bf16(v / sqrt(mean(v^2) + eps) * weight);
// the partials are scratch (slices 0 and 1 may be overwritten)
hipError_t launch_rmsnorm_rows(float* part, int32_t slices, int32_t n, int32_t d, const void* weight, float eps,
                               uint16_t* out, hipStream_t st);
// out[i] = bf16(in[i])
hipError_t launch_to_bf16(const float* in, int64_t n_elems, uint16_t* out, hipStream_t st);

// Cache rows from hidden states: split-K partial sums of [W^DKV; W^KR] h, then
// per token the sum over slices, the latent RMSNorm, RoPE and the row store.
struct KvProjArgs {
  const void* h;                // [n_tok][d_model]
  const void* w_dkv;            // [d_c][d_model]
  const void* w_kr;             // [d_r][d_model]
  const void* norm_w;           // [d_c] or NULL (weight 1)
  const int32_t* pos;           // [n_tok]
  const int64_t* row;           // [n_tok] destination cache rows
  void* cache;
  float* part;                  // [k_slices][n_tok][d_c + d_r] fp32
  int32_t n_tok, d_model, k_slices, k_per_slice;
  float eps;
  RopeTable rope;
};

// host launchers (defined in the .hip files); return hipGetLastError() after launch
hipError_t launch_append(const AppendArgs& a, int bf16, hipStream_t st);
hipError_t launch_rope_q(const RopeQArgs& a, int bf16, hipStream_t st);
hipError_t launch_absorb(const AbsorbArgs& a, int bf16, hipStream_t st);
hipError_t launch_splitkv(const SplitArgs& a, int bf16, hipStream_t st);
hipError_t launch_combine(const CombineArgs& a, int bf16, hipStream_t st);
hipError_t launch_prefill_unabsorbed(const ExpandArgs& e, const PrefillArgs& p, hipStream_t st);
hipError_t launch_kv_project_append(const KvProjArgs& a, int bf16, hipStream_t st);
hipError_t launch_append_fp8(const AppendArgs& a, hipStream_t st);
hipError_t launch_splitkv_fp8(const SplitArgs& a, hipStream_t st);
// split-K plan of launch_kv_project_append for the storage dtype: slices and k per slice
void kv_project_plan(int32_t n_tok, int32_t d_model, int bf16, int32_t& k_slices, int32_t& k_per_slice);
// LDS-tiled product (mla_gemm_lds.hip): split-K partials of [w0 ; w1] x^T
// for n >= 256 activation rows, d_in % 64 == 0, d_out % 192 == 0
bool gemm_lds_applies(int32_t n, int32_t d_in, int32_t d_out);
void gemm_lds_plan(int32_t n, int32_t d_in, int32_t d_out, int32_t& k_slices, int32_t& k_per_slice);
hipError_t launch_gemm_lds_partial(const GemmArgs& g, hipStream_t st);
bool splitkv_has_fast_path(int n_h, int bf16, int d_c, int d_r);
// every query of a launch takes the 16-head-group (hi + lo) path: the grouped
// kernel runs it over (query, split, head group)
bool splitkv_all_precise(int n_h, int32_t max_len, int32_t precise_below);

// ---------------------------------------------------------------- device helpers
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {  // round to nearest even
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}
// bf16 pair (round to nearest even), lo in the low half: one v_cvt_pk_bf16_f32
// (the conversion of each half alone is the same instruction, so the bits are
// those of f32_to_bf16 on each value)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
template <typename T>
__device__ __forceinline__ float load_as_f32(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load_as_f32<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_as_f32<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_to_f32(p[i]);
}
// element e of (query n, head h) of the absorbed queries: the storage value,
// plus for bf16 the lo plane's refinement when that plane is present
template <typename T>
__device__ __forceinline__ void store_q(void* q_lat, void* q_lo, int64_t nh, int row_e, int e, float v);
template <>
__device__ __forceinline__ void store_q<float>(void* q_lat, void*, int64_t nh, int row_e, int e, float v) {
  static_cast<float*>(q_lat)[nh * row_e + e] = v;
}
template <>
__device__ __forceinline__ void store_q<uint16_t>(void* q_lat, void* q_lo, int64_t nh, int row_e, int e, float v) {
  const uint16_t hi = f32_to_bf16(v);
  static_cast<uint16_t*>(q_lat)[nh * row_e + e] = hi;
  if (q_lo) static_cast<uint16_t*>(q_lo)[nh * row_e + e] = f32_to_bf16(v - bf16_to_f32(hi));
}
template <typename T>
__device__ __forceinline__ float load_q(const void* q_lat, const void* q_lo, int64_t nh, int row_e, int e);
template <>
__device__ __forceinline__ float load_q<float>(const void* q_lat, const void*, int64_t nh, int row_e, int e) {
  return static_cast<const float*>(q_lat)[nh * row_e + e];
}
template <>
__device__ __forceinline__ float load_q<uint16_t>(const void* q_lat, const void* q_lo, int64_t nh, int row_e, int e) {
  const float h = bf16_to_f32(static_cast<const uint16_t*>(q_lat)[nh * row_e + e]);
  return q_lo ? h + bf16_to_f32(static_cast<const uint16_t*>(q_lo)[nh * row_e + e]) : h;
}

// RoPE of the interleaved pair (x0, x1) by angle pos * theta: the angle and
// its sine/cosine in fp64, the rotation itself in fp32.
__device__ __forceinline__ void rope_pair(float x0, float x1, int64_t pos, double theta,
                                          float& y0, float& y1) {
  double s, c;
  sincos(static_cast<double>(pos) * theta, &s, &c);
  const float cf = static_cast<float>(c), sf = static_cast<float>(s);
  y0 = x0 * cf - x1 * sf;
  y1 = x0 * sf + x1 * cf;
}

template <typename T>
__device__ __forceinline__ T store_from_f32(float v);
template <>
__device__ __forceinline__ float store_from_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ uint16_t store_from_f32<uint16_t>(float v) { return f32_to_bf16(v); }

}  // namespace mla
